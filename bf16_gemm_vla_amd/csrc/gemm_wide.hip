// Wide GEMM (M > 64) for gfx950.
//
// Output tile 192 (rows of A) x BN (weight rows, 128 or 256) per workgroup
// of 8 waves arranged 2 x 4; each wave owns 96 x BN/4.  MFMA shapes with the
// full gfx950 rate: v_mfma_f32_32x32x16_bf16 for bf16 activations (FP8
// weights are converted to bf16 exactly in registers) and
// v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3 x E4M3, unit E8M0 scales) for
// FP8 x FP8.  The packed weight tile is the MFMA "A" operand (32 output
// channels), the activation tile the "B" operand (32 rows), so a lane's
// accumulator holds runs of 4 consecutive output channels of one row.
//
// Both operands enter LDS through direct global->LDS loads, 1 KiB per wave
// instruction, STAGES deep:
//  * activations, row-major, 128 bytes of K per row per stage, with the
//    16-byte chunk c of row r stored at position c ^ ((r >> 1) & 7) so the
//    32-row fragment reads hit distinct banks;
//  * weights, already in MFMA fragment order, copied as-is per 16-row tile
//    with 128 bytes of padding between tiles.
// Lanes whose source lies outside A or W load from an always-zero page at
// the end of the workspace's counter region instead, so ragged M, N and K
// tails contribute nothing and every wave issues the same number of loads
// per stage (which lets a partial vmcnt wait keep later stages in flight).
#include "gemm_common.h"

#include <type_traits>

namespace vla {
namespace {

using namespace gemm_detail;

constexpr int kWideBM = 192;
constexpr int kArowBytes = 128;   // K bytes of one activation row per stage

template <AType AT, WType WT, int BN, int WMW, int WNW>
struct WideCfg {
    static constexpr int WAVES = WMW * WNW;                           // WMW along M x WNW along N
    static constexpr int THREADS = WAVES * 64;
    static constexpr int AB = (AT == AType::FP8) ? 1 : 2;            // activation bytes / element
    static constexpr int WLB = (WT == WType::FP8) ? 8 : 16;          // weight bytes per lane slot
    static constexpr int BK = kArowBytes / AB;                       // K elements per stage
    static constexpr int FRAGS = BK / 32;                            // 16x32 fragments per tile row
    static constexpr int WT_BYTES = FRAGS * 64 * WLB;                // one 16-row tile per stage
    static constexpr int WT_STRIDE = WT_BYTES + 128;                 // + bank padding
    static constexpr int A_BYTES = kWideBM * kArowBytes;             // 24 KiB
    static constexpr int W_BYTES = (BN / 16) * WT_STRIDE;
    static constexpr int DUMMY = A_BYTES + W_BYTES;                  // 1 KiB sink for padding loads
    static constexpr int STAGE = DUMMY + 1024;
    static constexpr int STAGES = (3 * STAGE <= 160 * 1024) ? 3 : 2;
    static constexpr int WN = BN / WNW;                               // wave tile width
    static constexpr int NSUB = WN / 32;
    static constexpr int WMR = kWideBM / WMW;                         // wave tile height
    static constexpr int MSUB = WMR / 32;
    // loads per wave per stage; instructions beyond the real count load the
    // zero page into the sink, so every wave issues the same number
    static constexpr int A_INSTR = kWideBM / 8;
    static constexpr int W_INSTR = (BN / 16) * (WT_BYTES / 1024);
    static constexpr int TA = (A_INSTR + WAVES - 1) / WAVES;
    static constexpr int TW = (W_INSTR + WAVES - 1) / WAVES;
    static constexpr int VM_PER_STAGE = TA + TW;
};

// Global weight tile (16 rows) of local tile tt in group g.
template <Epi EPI, int BN>
__device__ __forceinline__ int wide_wtile(int g, int tt, int N) {
    if constexpr (EPI == Epi::PLAIN) {
        return g * (BN / 16) + tt;
    } else {
        // wave wn holds gate columns g*128 + wn*32 .. +31 (sub-tile 0) and
        // the matching up columns (sub-tile 1): local rows wn*64 + nsub*32 + r
        const int wn = tt >> 2, nsub = (tt >> 1) & 1, h = tt & 1;
        return (nsub ? (N >> 5) : 0) + g * 8 + wn * 2 + h;
    }
}

template <AType AT, WType WT, Epi EPI, int BN, int WMW, int WNW>
__global__ __launch_bounds__(WMW * WNW * 64) void wide_gemm_kernel(KArgs a) {
    using C = WideCfg<AT, WT, BN, WMW, WNW>;
    static_assert(EPI == Epi::PLAIN || (BN == 256 && WNW == 4), "the fused gate/up epilogue pairs two 32-column sub-tiles");
    // one LDS object per pipeline stage, so the compiler's wait insertion can
    // tell the buffer being read from the ones being filled
    __shared__ __attribute__((aligned(16))) uint8_t lds0[C::STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t lds1[C::STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t lds2[C::STAGES == 3 ? C::STAGE : 16];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WNW, wn = wave % WNW;  // wave grid WMW x WNW
    const int g = blockIdx.x, mb = blockIdx.y, split = blockIdx.z;
    const int m0 = mb * kWideBM;
    const int ksteps = a.K >> 5;
    const int ntiles16 = a.N >> 4;
    const int kt_total = (a.K + C::BK - 1) / C::BK;
    const int kt_per = (kt_total + a.ksplit - 1) / a.ksplit;
    const int kt_begin = split * kt_per;
    const int kt_end = min(kt_total, kt_begin + kt_per);
    const int nkt = max(0, kt_end - kt_begin);
    // out-of-range lanes load from an always-zero page of the workspace, so
    // every wave issues the same number of loads per stage
    const uint8_t* zero_page = reinterpret_cast<const uint8_t*>(a.tickets) + kZeroPageOffset;

    // ---- global -> LDS: load number t (0 <= t < VM_PER_STAGE) of this wave
    //      for K tile kt into stage buffer sa.  Loads t < TA carry activation
    //      rows, the rest weight tiles.
    auto load = [&](int kt, uint8_t* sa, int t) __attribute__((always_inline)) {
        if (t < C::TA) {
            // activations: A_INSTR instructions of 8 rows x 128 B
            const int i = wave + t * C::WAVES;
            const int row = i * 8 + (lane >> 3), pos = lane & 7;
            const int c = pos ^ ((row >> 1) & 7);
            const int gm = m0 + row;
            const int64_t kel = static_cast<int64_t>(kt) * C::BK + c * (16 / C::AB);
            const bool real = i < C::A_INSTR;
            const uint8_t* src = (real && gm < a.M && kel < a.K)
                ? static_cast<const uint8_t*>(a.A) + (static_cast<int64_t>(gm) * a.K + kel) * C::AB
                : zero_page + lane * 16;
            __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(sa + (real ? i * 1024 : C::DUMMY)), 16, 0, 0);
        } else {
            // weights: per 16-row tile WT_BYTES contiguous bytes, 1 KiB per instruction
            constexpr int PER_TILE = C::WT_BYTES / 1024;
            uint8_t* sw = sa + C::A_BYTES;
            const int j = wave + (t - C::TA) * C::WAVES;
            const bool real = j < C::W_INSTR;
            const int tt = real ? j / PER_TILE : 0, p = real ? j % PER_TILE : 0;
            const int gt = wide_wtile<EPI, BN>(g, tt, a.N);
            const int sb = p * 1024 + lane * 16;
            const int f = sb / (64 * C::WLB);
            const int k0 = kt * C::FRAGS + f;
            const uint8_t* src = (real && gt < ntiles16 && k0 < ksteps)
                ? static_cast<const uint8_t*>(a.W) + (static_cast<int64_t>(gt) * ksteps + kt * C::FRAGS) * 64 * C::WLB + sb
                : zero_page + lane * 16;
            __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(sw + (real ? tt * C::WT_STRIDE + p * 1024 : C::DUMMY - C::A_BYTES)), 16, 0, 0);
        }
    };
    auto issue = [&](int kt, uint8_t* sa) __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < C::VM_PER_STAGE; ++t) load(kt, sa, t);
    };

    using Acc = __attribute__((ext_vector_type(16))) float;
    Acc acc[C::NSUB][C::MSUB];
#pragma unroll
    for (int i = 0; i < C::NSUB; ++i)
#pragma unroll
        for (int j = 0; j < C::MSUB; ++j) acc[i][j] = Acc{};

    const int l32 = lane & 31, g2 = lane >> 5;
    // ---- one stage of MFMAs from stage buffer sa
    // While computing, the wave spreads the loads of the K tile kt_next into
    // nxt over the K sub-steps (LOADS false: no loads), so a wave stalled on
    // a full memory queue still has MFMAs issued around its loads.
    auto compute = [&](const uint8_t* sa, int kt_next, uint8_t* nxt, auto LOADS) __attribute__((always_inline)) {
        const uint8_t* sw = sa + C::A_BYTES;
        constexpr int NKS = (AT == AType::FP8) ? 2 : 4;
        auto loads_of = [&](int ks) __attribute__((always_inline)) {
            if constexpr (decltype(LOADS)::value) {
#pragma unroll
                for (int t = ks * C::VM_PER_STAGE / NKS; t < (ks + 1) * C::VM_PER_STAGE / NKS; ++t) load(kt_next, nxt, t);
            }
        };
        if constexpr (AT == AType::FP8) {
            // two 32x32x64 steps per stage
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                loads_of(ks);
                typedef __attribute__((ext_vector_type(8))) int i32x8_t;
                i32x8_t wop[C::NSUB], aop[C::MSUB];
#pragma unroll
                for (int ns = 0; ns < C::NSUB; ++ns) {
                    const int nl = wn * C::WN + ns * 32 + l32;
                    const uint8_t* base = sw + (nl >> 4) * C::WT_STRIDE + ((2 * ks + g2) * 64 + (nl & 15)) * 8;
                    u32x2_t q0 = *reinterpret_cast<const u32x2_t*>(base);
                    u32x2_t q1 = *reinterpret_cast<const u32x2_t*>(base + 16 * 8);
                    u32x2_t q2 = *reinterpret_cast<const u32x2_t*>(base + 32 * 8);
                    u32x2_t q3 = *reinterpret_cast<const u32x2_t*>(base + 48 * 8);
                    wop[ns] = i32x8_t{(int)q0.x, (int)q0.y, (int)q1.x, (int)q1.y, (int)q2.x, (int)q2.y, (int)q3.x, (int)q3.y};
                }
#pragma unroll
                for (int ms = 0; ms < C::MSUB; ++ms) {
                    const int r = wm * C::WMR + ms * 32 + l32;
                    const int c0 = 4 * ks + 2 * g2;
                    const int sw_ = (r >> 1) & 7;
                    u32x4_t v0 = *reinterpret_cast<const u32x4_t*>(sa + r * kArowBytes + ((c0 ^ sw_) * 16));
                    u32x4_t v1 = *reinterpret_cast<const u32x4_t*>(sa + r * kArowBytes + (((c0 + 1) ^ sw_) * 16));
                    aop[ms] = i32x8_t{(int)v0.x, (int)v0.y, (int)v0.z, (int)v0.w, (int)v1.x, (int)v1.y, (int)v1.z, (int)v1.w};
                }
#pragma unroll
                for (int ns = 0; ns < C::NSUB; ++ns)
#pragma unroll
                    for (int ms = 0; ms < C::MSUB; ++ms)
                        acc[ns][ms] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wop[ns], aop[ms], acc[ns][ms], 0, 0, 0, 127, 0, 127);
            }
        } else {
            // four 32x32x16 bf16 steps per stage
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                loads_of(ks);
                bf16x8_t wop[C::NSUB], aop[C::MSUB];
#pragma unroll
                for (int ns = 0; ns < C::NSUB; ++ns) {
                    const int nl = wn * C::WN + ns * 32 + l32;
                    const int k1 = 2 * (ks & 1) + g2;
                    const uint8_t* p = sw + (nl >> 4) * C::WT_STRIDE + (((ks >> 1) * 64 + 16 * k1 + (nl & 15)) * C::WLB);
                    if constexpr (WT == WType::FP8) wop[ns] = ocp8_to_bf16x8(*reinterpret_cast<const u32x2_t*>(p));
                    else wop[ns] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(p));
                }
#pragma unroll
                for (int ms = 0; ms < C::MSUB; ++ms) {
                    const int r = wm * C::WMR + ms * 32 + l32;
                    const int c = 2 * ks + g2;
                    aop[ms] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(sa + r * kArowBytes + ((c ^ ((r >> 1) & 7)) * 16)));
                }
#pragma unroll
                for (int ns = 0; ns < C::NSUB; ++ns)
#pragma unroll
                    for (int ms = 0; ms < C::MSUB; ++ms)
                        acc[ns][ms] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wop[ns], aop[ms], acc[ns][ms], 0, 0, 0);
            }
        }
    };

    // ---- pipeline: STAGES-1 K tiles in flight ahead of the one being computed.
    // Tile i lives in buffer i % STAGES.  Every step issues one tile (tiles
    // past the split's range load zeros or unused data, never computed), so
    // each wave has exactly VM_PER_STAGE loads per tile outstanding and a
    // partial vmcnt wait keeps the next tile in flight.  The barrier after
    // the wait makes every wave's loads of tile i visible and guarantees no
    // wave still reads the buffer the step's issue overwrites.
    constexpr int VM_KEEP1 = (C::VM_PER_STAGE & 15) | ((C::VM_PER_STAGE >> 4) << 14) | 0x0F70;  // vmcnt(VM)
    constexpr int VM_ZERO = 0x0F70;                                                              // vmcnt(0)
    auto step = [&](int i, const uint8_t* cur, uint8_t* nxt) __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt(C::STAGES == 3 ? VM_KEEP1 : VM_ZERO);
        __builtin_amdgcn_s_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        compute(cur, kt_begin + i + C::STAGES - 1, nxt, std::true_type{});
    };
    auto tail = [&](const uint8_t* cur) __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt(VM_ZERO);
        __builtin_amdgcn_s_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        compute(cur, 0, nullptr, std::false_type{});
    };
    if (nkt > 0) {
        issue(kt_begin, lds0);
        if constexpr (C::STAGES == 3) issue(kt_begin + 1, lds1);
        const int full = nkt / C::STAGES;
        for (int it = 0; it < full; ++it) {
            const int i = it * C::STAGES;
            if constexpr (C::STAGES == 3) {
                step(i, lds0, lds2);
                step(i + 1, lds1, lds0);
                step(i + 2, lds2, lds1);
            } else {
                step(i, lds0, lds1);
                step(i + 1, lds1, lds0);
            }
        }
        const int rem = nkt - full * C::STAGES;   // tiles left, already issued
        if (rem > 0) tail(lds0);
        if (rem > 1) tail(lds1);
    }
    __builtin_amdgcn_s_waitcnt(VM_ZERO);

    // ---- epilogue.  acc[ns][ms] register r: row (output channel) 8*(r/4) + 4*(lane/32) + r%4
    //      of the 32-column sub-tile, activation row lane%32 of the 32-row sub-tile.
    constexpr int NACC = C::NSUB * C::MSUB * 4;
    if (a.ksplit > 1) {
        // partial layout: [split][mblock][group][NACC][512 threads] of f32x4
        const int64_t slot = static_cast<int64_t>(mb) * a.groups + g;
        const int64_t per = static_cast<int64_t>(C::THREADS) * NACC;
        const int64_t sstride = static_cast<int64_t>(gridDim.y) * a.groups * per;
        const Coherent part(a.part, a.part_bytes);
        auto off = [&](int sp, int f) { return static_cast<uint32_t>((sp * sstride + slot * per + f * C::THREADS + tid) * 16); };
#pragma unroll
        for (int ns = 0; ns < C::NSUB; ++ns)
#pragma unroll
            for (int ms = 0; ms < C::MSUB; ++ms)
#pragma unroll
                for (int rq = 0; rq < 4; ++rq) {
                    const Acc& v = acc[ns][ms];
                    part.store(off(split, (ns * C::MSUB + ms) * 4 + rq), f32x4_t{v[4 * rq], v[4 * rq + 1], v[4 * rq + 2], v[4 * rq + 3]});
                }
        if (!splitk_arrive_last(a.tickets, static_cast<int>(slot), a.ksplit)) return;
#pragma unroll
        for (int ns = 0; ns < C::NSUB; ++ns)
#pragma unroll
            for (int ms = 0; ms < C::MSUB; ++ms)
#pragma unroll
                for (int rq = 0; rq < 4; ++rq) {
                    const int f = (ns * C::MSUB + ms) * 4 + rq;
                    f32x4_t v = part.load(off(0, f));
                    for (int sp = 1; sp < a.ksplit; ++sp) v += part.load(off(sp, f));
                    acc[ns][ms][4 * rq] = v[0];
                    acc[ns][ms][4 * rq + 1] = v[1];
                    acc[ns][ms][4 * rq + 2] = v[2];
                    acc[ns][ms][4 * rq + 3] = v[3];
                }
        splitk_reset(a.tickets, static_cast<int>(slot));
    }
    // ---- output: one pass per 32-row sub-tile ms.  Each wave scales (and
    //      biases, or applies GELU * up to) its accumulators in registers and
    //      writes the bf16 results into a [WMW*32][OUT_W] LDS tile; then the
    //      whole workgroup stores those rows as 16-byte column chunks, adding
    //      the residual on the way, so every wave writes full row segments.
    //      The passes alternate between two stage buffers: a wave writing
    //      pass ms+2 has passed the barrier every wave reaches only after
    //      storing pass ms.
    constexpr int OUT_W = (EPI == Epi::PLAIN) ? BN : 128;   // output columns of the tile
    constexpr int PR = WMW * 32;                             // rows per pass
    constexpr int OSTRIDE = OUT_W * 2 + 16;                  // bytes per LDS row (+ bank padding)
    constexpr int CPR = OUT_W / 8;                           // 16-byte chunks per row
    static_assert(PR * OSTRIDE <= C::STAGE, "an output pass fits one stage buffer");
    const float sa = (AT == AType::FP8) ? *a.s_a : 1.0f;
    const int outN = (EPI == Epi::PLAIN) ? a.N : (a.N >> 1);
    __syncthreads();   // every wave has finished reading the stage buffers
#pragma unroll
    for (int ms = 0; ms < C::MSUB; ++ms) {
        uint8_t* ot = (ms & 1) ? lds1 : lds0;
        const int m = m0 + wm * C::WMR + ms * 32 + l32;
        uint8_t* orow = ot + (wm * 32 + l32) * OSTRIDE;
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
            const int nrow = 8 * rq + 4 * g2;    // first of 4 consecutive channels in the sub-tile
            if constexpr (EPI == Epi::PLAIN) {
#pragma unroll
                for (int ns = 0; ns < C::NSUB; ++ns) {
                    const int nl = wn * C::WN + ns * 32 + nrow;
                    const int n = g * BN + nl;
                    if (n >= a.N) continue;
                    const Acc& v = acc[ns][ms];
                    *reinterpret_cast<uint2*>(orow + nl * 2) =
                        epi_plain4<AT, WT>(a, f32x4_t{v[4 * rq], v[4 * rq + 1], v[4 * rq + 2], v[4 * rq + 3]},
                                           load_epi<WT, EPI>(a, m, n, false), sa);
                }
            } else {
                const int nl = wn * 32 + nrow;
                const int n = g * 128 + nl;        // gate column
                if (n >= outN) continue;
                const Acc& vg = acc[0][ms];
                const Acc& vu = acc[1][ms];
                uint2 gq, uq;
                *reinterpret_cast<uint2*>(orow + nl * 2) =
                    epi_gelu4(f32x4_t{vg[4 * rq], vg[4 * rq + 1], vg[4 * rq + 2], vg[4 * rq + 3]},
                              f32x4_t{vu[4 * rq], vu[4 * rq + 1], vu[4 * rq + 2], vu[4 * rq + 3]},
                              load_epi<WT, EPI>(a, m, n, false), gq, uq);
                if (a.gu && m < a.M) {
                    *reinterpret_cast<uint2*>(a.gu + static_cast<int64_t>(m) * a.N + n) = gq;
                    *reinterpret_cast<uint2*>(a.gu + static_cast<int64_t>(m) * a.N + outN + n) = uq;
                }
            }
        }
        __syncthreads();
#pragma unroll
        for (int c = tid; c < PR * CPR; c += C::THREADS) {
            const int row = c / CPR, ch = c % CPR;
            const int gm = m0 + (row >> 5) * C::WMR + ms * 32 + (row & 31);
            const int n = g * OUT_W + ch * 8;
            if (gm >= a.M || n >= outN) continue;
            uint4 v = *reinterpret_cast<const uint4*>(ot + row * OSTRIDE + ch * 16);
            if constexpr (EPI == Epi::PLAIN) {
                if (a.resid) {
                    const uint4 r = *reinterpret_cast<const uint4*>(a.resid + static_cast<int64_t>(gm) * a.N + n);
                    v.x = add_resid2(v.x, r.x);
                    v.y = add_resid2(v.y, r.y);
                    v.z = add_resid2(v.z, r.z);
                    v.w = add_resid2(v.w, r.w);
                }
            }
            *reinterpret_cast<uint4*>(a.Y + static_cast<int64_t>(gm) * outN + n) = v;
        }
    }
}

}  // namespace

size_t wide_part_bytes(const GemmPlan& p) {
    // p.nt = BN; per thread NSUB x MSUB x 4 f32x4
    const int wmw = p.waves / p.wnw;
    const int nsub = p.nt / p.wnw / 32, msub = kWideBM / wmw / 32;
    return static_cast<size_t>(p.ksplit) * p.mblocks * p.groups * (p.waves * 64) * (nsub * msub * 4) * 16;
}

template <AType AT, WType WT, Epi EPI>
hipError_t launch_wide(const gemm_detail::KArgs& ka, const GemmPlan& p, hipStream_t s) {
    const dim3 grid(p.groups, p.mblocks, p.ksplit);
#define VLA_WIDE(BN_, WMW_, WNW_)                                                             \
    if (p.nt == BN_ && p.waves == WMW_ * WNW_ && p.wnw == WNW_) {                              \
        wide_gemm_kernel<AT, WT, EPI, BN_, WMW_, WNW_><<<grid, WMW_ * WNW_ * 64, 0, s>>>(ka);  \
        return hipGetLastError();                                                              \
    }
    if constexpr (EPI == Epi::GELU_MUL) {
        VLA_WIDE(256, 2, 4)
    } else if constexpr (AT == AType::FP8) {
        VLA_WIDE(256, 3, 4)
        VLA_WIDE(128, 3, 4)
        VLA_WIDE(256, 2, 4)
        VLA_WIDE(128, 2, 4)
    } else {
        VLA_WIDE(256, 2, 4)
        VLA_WIDE(128, 2, 4)
    }
#undef VLA_WIDE
    return hipErrorInvalidValue;
}

template hipError_t launch_wide<AType::BF16, WType::FP8, Epi::PLAIN>(const gemm_detail::KArgs&, const GemmPlan&, hipStream_t);
template hipError_t launch_wide<AType::BF16, WType::FP8, Epi::GELU_MUL>(const gemm_detail::KArgs&, const GemmPlan&, hipStream_t);
template hipError_t launch_wide<AType::BF16, WType::BF16, Epi::PLAIN>(const gemm_detail::KArgs&, const GemmPlan&, hipStream_t);
template hipError_t launch_wide<AType::FP8, WType::FP8, Epi::PLAIN>(const gemm_detail::KArgs&, const GemmPlan&, hipStream_t);

}  // namespace vla
