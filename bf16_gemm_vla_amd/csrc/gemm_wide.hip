// Wide GEMM (M > 64) for gfx950.
//
// Output tile 192 (rows of A) x BN (weight rows, 256 or 128) per workgroup
// of 8 waves, two per SIMD, arranged 2 (rows) x 4 (columns); each wave
// owns a 96 x BN/4 tile (3 x BN/128 accumulators of 32 x 32).  MFMA shapes
// with the full gfx950 rate: v_mfma_f32_32x32x16_bf16 for bf16 activations (FP8
// weights, and MXFP4 weights with their E8M0 block scales, are converted to
// bf16 exactly in registers) and the scaled
// v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3 x E4M3, unit E8M0 scales) for
// FP8 x FP8.  The packed weight tile is the MFMA "A" operand (32 output
// channels), the activation tile the "B" operand (32 rows), so a lane's
// accumulator holds runs of 4 consecutive output channels of one row.
//
// Operands move global -> LDS with buffer loads that write LDS directly
// (16 bytes per lane, 1 KiB per wave instruction), 64 K values per stage
// (128 for FP8 x FP8 on 128-column tiles), in a ring of four stage buffers:
//  * activations row-major, 128 bytes of K per row (64 for FP8 on
//    256-column tiles), the 16-byte chunks of each row XOR-swizzled so the
//    32-row operand reads hit distinct banks;
//  * weights in their packed fragment order, one 1 KiB (FP8), 512-byte
//    (MXFP4) or 2 KiB (bf16) block per 16-row tile; FP8 blocks of odd tiles
//    have their 128-byte halves swapped (MXFP4: 64-byte halves), so the two
//    16-row halves of a 32-row operand read fall in different banks;
//  * MXFP4 block scales: per stage and weight sub-tile, each lane's 4-byte
//    word of E8M0 bytes holding the stage's two blocks of its weight row,
//    loaded into LDS with the stage's other operands (256 bytes per wave
//    and sub-tile).
// Out-of-range rows, tiles and the ragged K tail fall outside the buffer
// resource and load zeros, so every wave issues the same number of loads
// per stage.  Each stage has one barrier, placed before the stage's last
// MFMA step: it publishes the next stage (its loads were waited for with a
// partial vmcnt that keeps the following stage in flight) and frees the
// buffer read two stages ago, which the loads of stage i+3 then refill.
// Operand fragments are double-buffered in registers, so the LDS reads of
// step s+1 (and of the next stage's first step, right after the barrier)
// overlap the MFMAs of step s.
#include "gemm_common.h"

#include <type_traits>

namespace vla {
namespace {

using namespace gemm_detail;

constexpr int kWideBM = 192;
constexpr int kWideStages = 4;
constexpr uint32_t kOOB = 0x80000000u;   // voffset beyond every resource's range

template <AType AT, WType WT, int BN, int WNW, int BK_>
struct WideCfg {
    static constexpr int BK = BK_;                              // K elements per pipeline stage
    static constexpr int WAVES = 2 * WNW;                       // 2 along M x WNW along N
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int AB = (AT == AType::FP8) ? 1 : 2;       // activation bytes / element
    static constexpr int WLB = (WT == WType::FP8) ? 8 : (WT == WType::FP4 ? 4 : 16);   // weight bytes per lane slot
    static constexpr int KMF = (AT == AType::FP8) ? 64 : 16;    // K of one MFMA
    static constexpr int NKS = BK / KMF;                        // MFMA steps per stage
    static constexpr int ARB = BK * AB;                         // A bytes per row per stage
    static constexpr int CPR = ARB / 16;                        // 16-byte chunks per A row
    static constexpr int RPI = 1024 / ARB;                      // A rows per load instruction
    static constexpr int WTB = (BK / 32) * 64 * WLB;            // W bytes per 16-row tile per stage
    static constexpr int A_BYTES = kWideBM * ARB;
    static constexpr int W_BYTES = (BN / 16) * WTB;
    static constexpr int A_LOADS = A_BYTES / 1024;
    // activation load slots per stage, rounded up to a multiple of the wave
    // count: the extra slots load nothing (offsets outside the resource) into
    // a pad of the stage buffer, so every wave still issues the same loads
    static constexpr int A_SLOTS = (A_LOADS + WAVES - 1) / WAVES * WAVES;
    static constexpr int A_REGION = A_SLOTS * 1024;
    static constexpr int W_LOADS = W_BYTES / 1024;
    // weight load slots, rounded up to a multiple of the wave count the same
    // way (MXFP4 on 128-column tiles: 4 KiB of codes, half a load per wave)
    static constexpr int W_SLOTS = (W_LOADS + WAVES - 1) / WAVES * WAVES;
    static constexpr int W_REGION = W_SLOTS * 1024;
    static constexpr int S_REGION = (WT == WType::FP4) ? WAVES * (BN / WNW / 32) * 256 : 0;   // MXFP4 scales
    static constexpr int STAGE = A_REGION + W_REGION + S_REGION;
    static constexpr int LA = A_SLOTS / WAVES;                  // activation slots per wave per stage
    static constexpr int L = LA + W_SLOTS / WAVES;              // loads per wave per stage
    static constexpr int MSUB = 3;                              // 96-row wave tile
    static constexpr int WN = BN / WNW;                         // wave tile width
    static constexpr int NSUB = WN / 32;
    static constexpr int LV = L + (WT == WType::FP4 ? NSUB : 0);  // vector-memory ops per wave per stage
    static_assert(A_BYTES % 1024 == 0 && W_BYTES % 1024 == 0, "whole 1 KiB loads");
    static_assert(kWideStages * STAGE <= 160 * 1024, "the stage ring fits the LDS");
    static_assert(L <= 15 && 2 * LV <= 63, "the partial vmcnt waits fit their field");
    static_assert(WT != WType::FP4 || (AT == AType::BF16 && BK == 64), "MXFP4 weights: bf16 activations, 64 K per stage");
};


// Global 16-row weight tile held in LDS tile slot tt of group g, or -1 when
// the slot lies past the weight matrix.  For the fused gate/up epilogue
// wave wn owns slots wn*WN/16 .. +WN/16-1 holding WN/32 sub-tiles of 32
// rows: the first half are gate columns g*BN/2 + wn*WN/2 + ns*32 .. +31,
// the second half the matching up columns.
template <Epi EPI, int BN, int WN>
__device__ __forceinline__ int wide_wtile(int g, int tt, int N) {
    const int ntiles = N >> 4;
    if constexpr (EPI == Epi::PLAIN) {
        const int t = g * (BN / 16) + tt;
        return t < ntiles ? t : -1;
    } else {
        constexpr int HALF = WN / 64;   // gate sub-tiles per wave
        const int gates = N >> 5;       // gate tiles
        const int wn = tt / (WN / 16), q = tt % (WN / 16), ns = q >> 1, h = q & 1;
        const int gt = g * (BN / 32) + wn * (WN / 32) + (ns % HALF) * 2 + h;
        if (gt >= gates) return -1;
        return ns < HALF ? gt : gates + gt;
    }
}

typedef __attribute__((ext_vector_type(8))) int i32x8_t;

// 16 bytes per lane from a buffer resource straight into LDS at
// lds + 16 * lane (lds is wave-uniform); offsets past the resource read 0.
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t r, uint8_t* lds, uint32_t voff, int soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
}

// Operand fragments of one MFMA step for one wave.
template <AType AT, WType WT, int MSUB, int NSUB>
struct Frags;
template <WType WT, int MSUB, int NSUB>
struct Frags<AType::BF16, WT, MSUB, NSUB> {
    u32x4_t a[MSUB];
    typename std::conditional<WT == WType::FP8, u32x2_t,
                              typename std::conditional<WT == WType::FP4, uint32_t, u32x4_t>::type>::type
        w[NSUB];                                                                   // as read from LDS
    bf16x8_t wb[NSUB];                                                             // MFMA operands
};
template <WType WT, int MSUB, int NSUB>
struct Frags<AType::FP8, WT, MSUB, NSUB> {
    u32x4_t a[MSUB][2];
    u32x2_t w[NSUB][4];
};

template <AType AT, WType WT, Epi EPI, int BN, int WNW, int BK>
__global__ __launch_bounds__(128 * WNW) __attribute__((amdgpu_waves_per_eu(WNW / 2, WNW / 2)))
void wide_gemm_kernel(KArgs a) {
    using C = WideCfg<AT, WT, BN, WNW, BK>;
    static_assert(AT == AType::FP8 || BK == 64, "bf16 activations stage 64 K values (128 bytes per row)");
    using F = Frags<AT, WT, C::MSUB, C::NSUB>;
    static_assert(EPI == Epi::PLAIN || (C::NSUB % 2 == 0 && AT == AType::BF16 && WT == WType::FP8),
                  "the fused gate/up epilogue pairs gate and up sub-tiles within a wave");
    // one LDS object per stage buffer, so the compiler's wait insertion can
    // tell the buffer being read from the ones being filled
    __shared__ __attribute__((aligned(16))) uint8_t lds0[C::STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t lds1[C::STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t lds2[C::STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t lds3[C::STAGE];
    uint8_t* const bufs[4] = {lds0, lds1, lds2, lds3};

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: LDS destinations in SGPRs
    const int wm = wave / WNW, wn = wave % WNW;
    const int l32 = lane & 31, g2 = lane >> 5;
    // Tile order.  The dispatcher deals workgroups to the 8 XCDs
    // round-robin by linear id, so with the grid's own order (column group
    // fastest, a multiple of 8 column groups) XCD j holds column groups
    // j, j+8, ... with all their row blocks: each weight slice streams into
    // one L2.  With K split that order makes every XCD read all of A (each
    // holds every row block of every split); there the workgroups are
    // renumbered so XCD j runs one contiguous run of the order (split
    // slowest, then column group, row block fastest) and reads the rows of
    // one split only (M = 768 down-projection: 210 -> 97 MB fetched beyond
    // L2 per launch).  Without a split the grid's order measured faster.
    int g = blockIdx.x, mb = blockIdx.y, split = blockIdx.z;
    if (a.ksplit > 1) {
        const int gx = gridDim.x, gy = gridDim.y;
        const int tiles = gx * gy * gridDim.z;
        const int lin = blockIdx.x + gx * (blockIdx.y + gy * blockIdx.z);
        const int xq = tiles >> 3, xr = tiles & 7, xj = lin & 7, xi = lin >> 3;
        const int order = (xj < xr) ? xj * (xq + 1) + xi : xr * (xq + 1) + (xj - xr) * xq + xi;
        mb = order % gy;
        g = (order / gy) % gx;
        split = order / (gy * gx);
    }
    const int m0 = mb * kWideBM;
    const int ksteps = a.K >> 5;
    const int kt_total = (a.K + BK - 1) / BK;
    const int kt_per = (kt_total + a.ksplit - 1) / a.ksplit;
    const int kt_begin = split * kt_per;
    const int kt_end = min(kt_total, kt_begin + kt_per);
    const int nkt = max(0, kt_end - kt_begin);
    // split-K counters of this output tile: [0] workgroups started,
    // [1] arrivals (+ slices handed to the last arrival), [2] workgroups done
    uint32_t* const ctr = a.tickets + (static_cast<int64_t>(mb) * a.groups + g) * kWideCounters;
    if (a.ksplit > 1 && tid == 0) __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

    // buffer resources bounded to A and W: loads past the end read zero
    const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(a.A), 0, a.M * a.K * C::AB, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rW = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(a.W), 0, ksteps * (a.N >> 4) * 64 * C::WLB, kRsrcWord3);

    // ---- per-lane source offsets of this wave's L loads per stage (without
    //      the stage term) and the K position each covers (ragged-K mask).
    //      Load t of wave w is instruction q = w + WAVES*t of the stage; it
    //      fills LDS bytes q*1024 .. +1023 of the stage buffer (A slots
    //      first, then W).
    uint32_t voff[C::L], voffT[C::L];   // voffT: the same for the ragged last K tile
    const int krem = a.K - (kt_total - 1) * BK;         // K values in the last K tile
#pragma unroll
    for (int t = 0; t < C::L; ++t) {
        const int q = wave + C::WAVES * t;
        bool in_tail;   // does this lane's chunk lie within the last K tile's krem values?
        if (t < C::LA) {
            const int row = q * C::RPI + lane / C::CPR, pos = lane % C::CPR;
            const int c = (C::CPR == 8) ? (pos ^ ((row >> 1) & 7)) : (pos ^ ((row >> 2) & 3));
            const int gm = m0 + row;
            voff[t] = (q < C::A_LOADS && gm < a.M) ? static_cast<uint32_t>((gm * a.K) * C::AB + c * 16) : kOOB;
            in_tail = c * (16 / C::AB) < krem;
        } else {
            const int j = q - C::A_SLOTS;
            int tt, sb;                                         // tile slot, byte within its stage block
            if constexpr (WT == WType::FP4) {
                // two 512-byte tile blocks per load, odd tiles' 64-byte halves swapped
                tt = 2 * j + (lane >> 5);
                sb = ((lane & 31) ^ (4 * (tt & 1))) * 16;
            } else {
                constexpr int PER_TILE = C::WTB / 1024;
                tt = j / PER_TILE;
                const int chunk = (WT == WType::FP8) ? (lane ^ (8 * (tt & 1))) : lane;
                sb = (j % PER_TILE) * 1024 + chunk * 16;
            }
            const int gt = (j < C::W_LOADS) ? wide_wtile<EPI, BN, C::WN>(g, tt, a.N) : -1;   // pad slots: none
            voff[t] = gt >= 0 ? static_cast<uint32_t>(gt * ksteps * 64 * C::WLB + sb) : kOOB;
            in_tail = (sb / (64 * C::WLB)) * 32 < krem;         // packed fragment within the tile
        }
        voffT[t] = in_tail ? voff[t] : kOOB;
    }
    // MXFP4 block scales: E8M0 bytes after the codes, one row of P = K/32
    // (rounded up to 8) bytes per weight row.  The lane's weight row of
    // sub-tile ns is (tile slot of its 32-row operand half) * 16 + l32 % 16;
    // stage kt's blocks 2kt, 2kt + 1 lie in the aligned word at byte
    // 2kt & ~3 of the row, at byte 2 (kt & 1) of it.
    const int sP = ((a.K >> 5) + 7) & ~7;
    const __amdgpu_buffer_rsrc_t rS = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(static_cast<const uint8_t*>(a.W)) + static_cast<int64_t>(a.N >> 4) * ksteps * 64 * C::WLB,
        0, a.N * sP, kRsrcWord3);
    uint32_t svoff[C::NSUB];
    if constexpr (WT == WType::FP4) {
#pragma unroll
        for (int ns = 0; ns < C::NSUB; ++ns) {
            const int gt = wide_wtile<EPI, BN, C::WN>(g, ((wn * C::WN + ns * 32) >> 4) + ((l32 >> 4) & 1), a.N);
            svoff[ns] = gt >= 0 ? static_cast<uint32_t>((gt * 16 + (l32 & 15)) * sP) : kOOB;
        }
    }
    // Loads of a stage past the range (real == false) are pushed outside the
    // resources through the scalar offset: they only write zeros into a free
    // buffer, which keeps every stage's load count and wait identical.
    // Stage buffer (and scale ring slot) RC.
    auto issue = [&](auto RC, int kt, bool real) __attribute__((always_inline)) {
        constexpr int r = decltype(RC)::value;
        uint8_t* const buf = bufs[r];
        const bool ktail = kt == kt_total - 1;                  // uniform
        const int sA = real ? kt * C::ARB : static_cast<int>(kOOB);
        const int sW = real ? kt * C::WTB : static_cast<int>(kOOB);
#pragma unroll
        for (int t = 0; t < C::L; ++t) {
            buffer_load_lds16(t < C::LA ? rA : rW, buf + (wave + C::WAVES * t) * 1024, ktail ? voffT[t] : voff[t],
                              t < C::LA ? sA : sW);
        }
        if constexpr (WT == WType::FP4) {
            const int sS = real ? ((2 * kt) & ~3) : static_cast<int>(kOOB);
#pragma unroll
            for (int ns = 0; ns < C::NSUB; ++ns)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rS, (__attribute__((address_space(3))) void*)(buf + C::A_REGION + C::W_REGION + (wave * C::NSUB + ns) * 256),
                    4, svoff[ns], sS, 0, 0);
        }
    };

    // ---- LDS operand addresses (byte offsets within a stage buffer).
    //      Activation row r = wm*96 + ms*32 + l32; its 16-byte chunk c sits
    //      at position c ^ swz with swz taken from bits of l32 only (the
    //      wm/ms terms are multiples of 32 rows).  Weight tile slot of the
    //      lane's row: (wn*WN + ns*32)/16 + (l32 >> 4).
    const int swzA = (C::CPR == 8) ? ((l32 >> 1) & 7) : ((l32 >> 2) & 3);
    const int oddW = (l32 >> 4) & 1;
    const int aoff = (wm * 96 + l32) * C::ARB;
    int woff;
    if constexpr (WT == WType::BF16)
        woff = C::A_REGION + ((wn * C::WN) >> 4) * C::WTB + oddW * C::WTB + (l32 & 15) * 16 + g2 * 256;
    else if constexpr (WT == WType::FP4)
        woff = C::A_REGION + ((wn * C::WN) >> 4) * C::WTB + oddW * C::WTB + (l32 & 15) * 4 + (g2 ^ oddW) * 64;
    else if constexpr (AT == AType::BF16)
        woff = C::A_REGION + ((wn * C::WN) >> 4) * C::WTB + oddW * C::WTB + (l32 & 15) * 8 + (g2 ^ oddW) * 128;
    else
        woff = C::A_REGION + ((wn * C::WN) >> 4) * C::WTB + oddW * C::WTB + (l32 & 15) * 8 + g2 * 512;

    auto read_step = [&](const uint8_t* buf, int ks, F& f) __attribute__((always_inline)) {
        if constexpr (AT == AType::BF16) {
            // 32x32x16: chunk (2ks + g2) ^ swz = ((ks ^ (swz >> 1)) << 1) | (g2 ^ (swz & 1))
            const int cpos = ((((ks ^ (swzA >> 1)) << 1)) | (g2 ^ (swzA & 1))) * 16;
#pragma unroll
            for (int ms = 0; ms < C::MSUB; ++ms)
                f.a[ms] = *reinterpret_cast<const u32x4_t*>(buf + aoff + ms * 32 * C::ARB + cpos);
#pragma unroll
            for (int ns = 0; ns < C::NSUB; ++ns) {
                // packed fragment ks/2, K group 2(ks&1) + g2 (FP8 tiles of odd slots: 128-byte halves swapped)
                if constexpr (WT == WType::FP8)
                    f.w[ns] = *reinterpret_cast<const u32x2_t*>(buf + woff + ns * 2 * C::WTB + ks * 256);
                else if constexpr (WT == WType::FP4)
                    f.w[ns] = *reinterpret_cast<const uint32_t*>(buf + woff + ns * 2 * C::WTB + ks * 128);
                else
                    f.w[ns] = *reinterpret_cast<const u32x4_t*>(buf + woff + ns * 2 * C::WTB + ks * 512);
            }
        } else {
            // 32x32x64: the lane's row holds K 64ks + 32g2 .. +31 = chunks c0, c0+1
            const int c0 = 4 * ks + 2 * g2;
            const int p0 = (c0 ^ swzA) * 16, p1 = ((c0 + 1) ^ swzA) * 16;
#pragma unroll
            for (int ms = 0; ms < C::MSUB; ++ms) {
                f.a[ms][0] = *reinterpret_cast<const u32x4_t*>(buf + aoff + ms * 32 * C::ARB + p0);
                f.a[ms][1] = *reinterpret_cast<const u32x4_t*>(buf + aoff + ms * 32 * C::ARB + p1);
            }
            // packed fragment 2ks + g2, K groups k1 = 0..3
#pragma unroll
            for (int ns = 0; ns < C::NSUB; ++ns)
#pragma unroll
                for (int k1 = 0; k1 < 4; ++k1)
                    f.w[ns][k1] = *reinterpret_cast<const u32x2_t*>(buf + woff + ns * 2 * C::WTB + ks * 1024 + ((k1 ^ oddW) * 128));
        }
    };

    using Acc = __attribute__((ext_vector_type(16))) float;
    Acc acc[C::NSUB][C::MSUB];
#pragma unroll
    for (int i = 0; i < C::NSUB; ++i)
#pragma unroll
        for (int j = 0; j < C::MSUB; ++j) acc[i][j] = Acc{};

    // weight operands as bf16 (an exact conversion for FP8 and MXFP4
    // weights); f holds step ks of K tile kt, staged in buffer RC.  MXFP4:
    // step ks uses block ks / 2 of the tile's two; their scales are read
    // from the buffer's scale area with step 0 (every step of a tile is
    // converted after its step 0 and before the next tile's)
    float sf[C::NSUB][2];
    auto convert = [&](F& f, auto RC, int kt, int ks) __attribute__((always_inline)) {
        if constexpr (AT == AType::BF16) {
#pragma unroll
            for (int ns = 0; ns < C::NSUB; ++ns) {
                if constexpr (WT == WType::FP8) {
                    f.wb[ns] = ocp8_to_bf16x8(f.w[ns]);
                } else if constexpr (WT == WType::FP4) {
                    if (ks == 0) {
                        const uint32_t sw = *reinterpret_cast<const uint32_t*>(
                            bufs[decltype(RC)::value] + C::A_REGION + C::W_REGION + (wave * C::NSUB + ns) * 256 + lane * 4);
                        const uint32_t pair = sw >> (16 * (kt & 1));
                        sf[ns][0] = e8m0_to_f32(pair & 0xFFu);
                        sf[ns][1] = e8m0_to_f32((pair >> 8) & 0xFFu);
                    }
                    f.wb[ns] = fp4_to_bf16x8(f.w[ns], sf[ns][ks >> 1]);
                } else {
                    f.wb[ns] = as_bf16x8(f.w[ns]);
                }
            }
        }
    };
    // MFMAs number lo .. hi-1 of a step, in the order (ns, ms)
    auto mfmas = [&](const F& f, int lo, int hi) __attribute__((always_inline)) {
#pragma unroll
        for (int ns = 0; ns < C::NSUB; ++ns) {
#pragma unroll
            for (int ms = 0; ms < C::MSUB; ++ms) {
                const int idx = ns * C::MSUB + ms;
                if (idx < lo || idx >= hi) continue;
                if constexpr (AT == AType::BF16) {
                    acc[ns][ms] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.wb[ns], as_bf16x8(f.a[ms]), acc[ns][ms], 0, 0, 0);
                } else {
                    const i32x8_t wop = {(int)f.w[ns][0].x, (int)f.w[ns][0].y, (int)f.w[ns][1].x, (int)f.w[ns][1].y,
                                         (int)f.w[ns][2].x, (int)f.w[ns][2].y, (int)f.w[ns][3].x, (int)f.w[ns][3].y};
                    const i32x8_t aop = {(int)f.a[ms][0].x, (int)f.a[ms][0].y, (int)f.a[ms][0].z, (int)f.a[ms][0].w,
                                         (int)f.a[ms][1].x, (int)f.a[ms][1].y, (int)f.a[ms][1].z, (int)f.a[ms][1].w};
                    acc[ns][ms] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wop, aop, acc[ns][ms], 0, 0, 0, 127, 0, 127);
                }
            }
        }
    };

    // ---- pipeline.  Stage i (K tile kt_begin + i) lives in buffer i % 4.
    //      Before stage 0: stages 0..2 issued.  In stage i, before its last
    //      MFMA step: wait until stage i+1 has landed (stage i+2 stays in
    //      flight: at most L loads outstanding), barrier, read the first
    //      fragments of stage i+1, issue stage i+3 into the buffer of stage
    //      i-1.  Stages past the range are issued and read like the others
    //      (zeros, never multiplied), so every stage runs the same code and
    //      the waits are compile-time constants.
    constexpr int S = kWideStages;
    static_assert(S == 4, "the stage body is unrolled over a ring of four buffers");
    //      Within a step the order is pinned: the next step's LDS reads go
    //      out first, interleaved with the first half of the MFMAs, and the
    //      next step's weight conversions fill the gaps of the second half.
    //      The stage's last step issues half of its MFMAs before the barrier,
    //      so the matrix pipe is busy while the waves meet.  With bf16
    //      activations on 128-column tiles the MFMA blocks run at raised
    //      wave priority, so a wave with MFMAs ready issues ahead of its SIMD
    //      partner's memory work; the other tilings measured faster without
    //      (M = 768 and 571, alternating runs: FP8 x FP8 1-4%, W8A16 on
    //      256-column tiles 2%, while W8A16 on 128-column tiles lost 2%).
    constexpr bool PRIO = AT == AType::BF16 && BN == 128;
    auto prio_on = [&]() __attribute__((always_inline)) {
        if constexpr (PRIO) __builtin_amdgcn_s_setprio(1);
    };
    auto prio_off = [&]() __attribute__((always_inline)) {
        if constexpr (PRIO) __builtin_amdgcn_s_setprio(0);
    };
    constexpr int NM = C::NSUB * C::MSUB;        // MFMAs per step
    constexpr int HALF = NM / 2;
    F f0, f1;
    auto stage = [&](auto UC, int i) __attribute__((always_inline)) {
        constexpr int u = decltype(UC)::value;
        const uint8_t* cur = bufs[u];
#pragma unroll
        for (int ks = 0; ks < C::NKS; ++ks) {
            const bool odd = ((u * C::NKS + ks) & 1) != 0;
            F& cf = odd ? f1 : f0;
            F& of = odd ? f0 : f1;
            if (ks + 1 < C::NKS) {
                __builtin_amdgcn_sched_barrier(0);
                read_step(cur, ks + 1, of);
                prio_on();
                mfmas(cf, 0, NM);
                prio_off();
                convert(of, UC, kt_begin + i, ks + 1);
#pragma unroll
                for (int j = 0; j < HALF; ++j) {
                    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // DS reads
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
                }
#pragma unroll
                for (int j = HALF; j < NM; ++j) {
                    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);   // VALU
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
            } else {
                __builtin_amdgcn_sched_barrier(0);
                prio_on();
                mfmas(cf, 0, HALF);
                prio_off();
                __builtin_amdgcn_sched_barrier(0);
                __builtin_amdgcn_s_waitcnt(vmcnt_imm((S - 3) * C::LV));
                __builtin_amdgcn_s_barrier();
                __atomic_signal_fence(__ATOMIC_SEQ_CST);
                __builtin_amdgcn_sched_barrier(0);
                read_step(bufs[(u + 1) % S], 0, of);
                issue(std::integral_constant<int, (u + S - 1) % S>{}, kt_begin + i + S - 1, i + S - 1 < nkt);
                prio_on();
                mfmas(cf, HALF, NM);
                prio_off();
                convert(of, std::integral_constant<int, (u + 1) % S>{}, kt_begin + i + 1, 0);
#pragma unroll
                for (int j = HALF; j < NM; ++j) {
                    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);   // DS reads
                    __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);   // VMEM loads
                    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);   // VALU
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };
    if (nkt > 0) {
        issue(std::integral_constant<int, 0>{}, kt_begin, 0 < nkt);
        issue(std::integral_constant<int, 1>{}, kt_begin + 1, 1 < nkt);
        issue(std::integral_constant<int, 2>{}, kt_begin + 2, 2 < nkt);
        __builtin_amdgcn_s_waitcnt(vmcnt_imm((S - 2) * C::LV));
        __builtin_amdgcn_s_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        read_step(lds0, 0, f0);
        convert(f0, std::integral_constant<int, 0>{}, kt_begin, 0);
        const int full = nkt & ~(S - 1);
        for (int i0 = 0; i0 < full; i0 += S) {
            stage(std::integral_constant<int, 0>{}, i0);
            stage(std::integral_constant<int, 1>{}, i0 + 1);
            stage(std::integral_constant<int, 2>{}, i0 + 2);
            stage(std::integral_constant<int, 3>{}, i0 + 3);
        }
        const int rem = nkt - full;
        if (rem > 0) stage(std::integral_constant<int, 0>{}, full);
        if (rem > 1) stage(std::integral_constant<int, 1>{}, full + 1);
        if (rem > 2) stage(std::integral_constant<int, 2>{}, full + 2);
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));

    // ---- epilogue inputs (scales, bias; gate and up scales for the fused
    //      epilogue) of this lane's output columns, all requested at once so
    //      their latency is paid once, overlapping the split-K exchange.
    constexpr int NE = (EPI == Epi::PLAIN) ? C::NSUB : C::NSUB / 2;
    EpiIn ein[NE][4];
#pragma unroll
    for (int ns = 0; ns < NE; ++ns)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
            const int nrow = 8 * rq + 4 * g2;
            const int n = (EPI == Epi::PLAIN) ? g * BN + wn * C::WN + ns * 32 + nrow
                                              : g * (BN / 2) + wn * (C::WN / 2) + ns * 32 + nrow;
            if (n < ((EPI == Epi::PLAIN) ? a.N : (a.N >> 1))) ein[ns][rq] = load_epi<WT, EPI>(a, 0, n, false);
            else ein[ns][rq] = EpiIn{};
        }
    const float sa = (AT == AType::FP8) ? *a.s_a : 1.0f;
    // Wait for these loads here, once: gfx9 counts stores in vmcnt too, so a
    // wait for them placed after the first output stores would also wait for
    // every store issued so far.
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));

    // ---- epilogue.  acc[ns][ms] register r: row (output channel) 8*(r/4) + 4*(lane/32) + r%4
    //      of the 32-column sub-tile, activation row lane%32 of the 32-row sub-tile.
    //      The tile is finished in MSUB slices (slice ms = accumulators acc[*][ms]).
    //      With K split over workgroups, the workgroup of split s < MSUB owns
    //      slice s and finishes it itself, waiting for the other splits'
    //      partials, but only if every split of the tile had started when it
    //      decided (then all of them are running and arrive without waiting
    //      on anything, so the wait ends); otherwise it hands the slice to
    //      whichever workgroup arrives last, which also takes slices without
    //      an owner.  Every workgroup stores its partials of the slices it
    //      does not own, and an owner that hands its slice over stores that
    //      one too; a keeping owner adds its own partials from registers.  The
    //      hand-over travels in the same atomic as the arrival, so no fence is
    //      needed.  Partials are summed in split order, whoever finishes
    //      (bitwise repeatable).
    constexpr int NACC = C::NSUB * C::MSUB * 4;
    uint32_t todo = (1u << C::MSUB) - 1;     // slices this workgroup outputs
    if (a.ksplit > 1) {
        // partial layout: [split][mblock][group][NACC][threads] of f32x4
        const int64_t slot = static_cast<int64_t>(mb) * a.groups + g;
        const int64_t per = static_cast<int64_t>(C::THREADS) * NACC;
        const int64_t sstride = static_cast<int64_t>(gridDim.y) * a.groups * per;
        const Coherent part(a.part, a.part_bytes);
        auto off = [&](int sp, int f) { return static_cast<uint32_t>((sp * sstride + slot * per + f * C::THREADS + tid) * 16); };
        // have all splits of the tile started?  (read while the stores drain)
        const uint32_t ks = static_cast<uint32_t>(a.ksplit);
        const int own = split < C::MSUB ? split : -1;
        uint32_t started = 0;
        if (tid == 0) started = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        auto store_slice = [&](int ms) __attribute__((always_inline)) {
#pragma unroll
            for (int ns = 0; ns < C::NSUB; ++ns)
#pragma unroll
                for (int rq = 0; rq < 4; ++rq) {
                    const Acc& v = acc[ns][ms];
                    part.store(off(split, (ns * C::MSUB + ms) * 4 + rq), f32x4_t{v[4 * rq], v[4 * rq + 1], v[4 * rq + 2], v[4 * rq + 3]});
                }
        };
        // the slices other workgroups may finish; an owner keeps its own
        // slice's partials in registers unless it hands the slice over
#pragma unroll
        for (int ms = 0; ms < C::MSUB; ++ms)
            if (ms != own) store_slice(ms);
        // every wave's partial stores have completed (stores count in vmcnt),
        // then the barrier orders them before the arrival; the flag lives in
        // stage buffer 0, which every wave has finished reading
        int* const flags = reinterpret_cast<int*>(lds0);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        // an owner that finds a split not yet started hands its slice over:
        // then its partials of that slice are stored too, before the arrival
        bool keep = false;
        if (own >= 0) {
            if (tid == 0) flags[0] = started == ks ? 1 : 0;
            __syncthreads();
            keep = flags[0] != 0;
            if (!keep) {
#pragma unroll
                for (int ms = 0; ms < C::MSUB; ++ms)
                    if (ms == own) store_slice(ms);
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            }
            __syncthreads();
        }
        if (tid == 0) {
            const bool wait_own = keep;
            const uint32_t add = 1u + ((own >= 0 && !wait_own) ? (1u << (16 + own)) : 0u);
            const uint32_t prev = __hip_atomic_fetch_add(ctr + 1, add, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            uint32_t mine = 0;
            if ((prev & 0xFFFFu) == ks - 1) {
                const uint32_t handed = (prev + add) >> 16;
#pragma unroll
                for (int ms = 0; ms < C::MSUB; ++ms)
                    if (((handed >> ms) & 1u) || ms >= a.ksplit) mine |= 1u << ms;
            }
            uint32_t poison = 0;
            if (wait_own) {
                // bounded: an owner that gives up writes NaN over its slice
                // (the incomplete output shows in the data) and records the
                // cause in the workspace's status word
                bool arrived = false;
                for (uint32_t it = 0; it < a.wait_polls; ++it) {
                    if ((__hip_atomic_load(ctr + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & 0xFFFFu) == ks) {
                        arrived = true;
                        break;
                    }
                    __builtin_amdgcn_s_sleep(2);
                }
                mine |= 1u << own;
                if (!arrived) {
                    poison = 1u << own;
                    report_wait_timeout(a.err, kStatusWideSplitK);
                }
            }
            // no counter of the tile is read after this point; the last
            // workgroup past it clears them for the next call
            if (__hip_atomic_fetch_add(ctr + 2, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == ks - 1) {
                __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(ctr + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(ctr + 2, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            flags[0] = static_cast<int>(mine);
            flags[1] = static_cast<int>(poison);
        }
        __syncthreads();
        todo = static_cast<uint32_t>(flags[0]);
        const uint32_t poisoned = static_cast<uint32_t>(flags[1]);
        if (todo == 0) return;
#pragma unroll
        for (int ms = 0; ms < C::MSUB; ++ms) {
            if (!(todo & (1u << ms))) continue;
            if (poisoned & (1u << ms)) {
#pragma unroll
                for (int ns = 0; ns < C::NSUB; ++ns) acc[ns][ms] = Acc{} + __builtin_nanf("");
                continue;
            }
            // two splits' loads in flight at a time, summed in split order;
            // this workgroup's own split of a slice it kept comes from its
            // registers (the values it would have stored)
            const int reg_sp = (keep && ms == own) ? split : -1;
            auto part_or_reg = [&](int sp, int ns, int rq) __attribute__((always_inline)) {
                const Acc& v = acc[ns][ms];
                return sp == reg_sp ? f32x4_t{v[4 * rq], v[4 * rq + 1], v[4 * rq + 2], v[4 * rq + 3]}
                                    : part.load(off(sp, (ns * C::MSUB + ms) * 4 + rq));
            };
            f32x4_t sum[C::NSUB][4];
            for (int sp = 0; sp < a.ksplit; sp += 2) {
                f32x4_t p0[C::NSUB][4], p1[C::NSUB][4];
                const bool two = sp + 1 < a.ksplit;
#pragma unroll
                for (int ns = 0; ns < C::NSUB; ++ns)
#pragma unroll
                    for (int rq = 0; rq < 4; ++rq) {
                        p0[ns][rq] = part_or_reg(sp, ns, rq);
                        p1[ns][rq] = two ? part_or_reg(sp + 1, ns, rq) : f32x4_t{};
                    }
#pragma unroll
                for (int ns = 0; ns < C::NSUB; ++ns)
#pragma unroll
                    for (int rq = 0; rq < 4; ++rq) {
                        sum[ns][rq] = sp == 0 ? p0[ns][rq] : sum[ns][rq] + p0[ns][rq];
                        if (two) sum[ns][rq] += p1[ns][rq];
                    }
            }
#pragma unroll
            for (int ns = 0; ns < C::NSUB; ++ns)
#pragma unroll
                for (int rq = 0; rq < 4; ++rq)
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[ns][ms][4 * rq + e] = sum[ns][rq][e];
        }
    }
    // ---- output: one pass per 32-row sub-tile ms (64 rows: both wm halves).
    //      Each wave scales (and biases, or applies GELU * up to) its
    //      accumulators in registers and writes the bf16 results into LDS
    //      rows [32][OUT_W], wm half in its own stage buffer; then the whole
    //      workgroup stores the pass as 16-byte row chunks, adding the
    //      residual on the way.  Passes alternate between buffer pairs
    //      (0, 1) and (2, 3): a wave writing pass k+2 has passed the barrier
    //      every wave reaches only after storing pass k.
    constexpr int OUT_W = (EPI == Epi::PLAIN) ? BN : BN / 2;  // output columns of the tile
    constexpr int OSTRIDE = OUT_W * 2 + 16;                   // bytes per LDS row (+ bank padding)
    constexpr int CPRO = OUT_W / 8;                           // 16-byte chunks per output row
    static_assert(32 * OSTRIDE <= C::STAGE, "32 output rows fit one stage buffer");
    const int outN = (EPI == Epi::PLAIN) ? a.N : (a.N >> 1);
    __syncthreads();   // every wave has finished reading the stage buffers (and the flags)
    int pass = 0;
#pragma unroll
    for (int ms = 0; ms < C::MSUB; ++ms) {
        if (!(todo & (1u << ms))) continue;   // uniform
        uint8_t* const pair0 = (pass & 1) ? lds2 : lds0;
        uint8_t* const pair1 = (pass & 1) ? lds3 : lds1;
        ++pass;
        const int m = m0 + wm * 96 + ms * 32 + l32;
        uint8_t* orow = (wm ? pair1 : pair0) + l32 * OSTRIDE;
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
                                           ein[ns][rq], sa);
                }
            } else {
#pragma unroll
                for (int ns = 0; ns < C::NSUB / 2; ++ns) {
                    const int nl = wn * (C::WN / 2) + ns * 32 + nrow;
                    const int n = g * OUT_W + nl;        // gate column
                    if (n >= outN) continue;
                    const Acc& vg = acc[ns][ms];
                    const Acc& vu = acc[ns + C::NSUB / 2][ms];
                    uint2 gq, uq;
                    *reinterpret_cast<uint2*>(orow + nl * 2) =
                        epi_gelu4(f32x4_t{vg[4 * rq], vg[4 * rq + 1], vg[4 * rq + 2], vg[4 * rq + 3]},
                                  f32x4_t{vu[4 * rq], vu[4 * rq + 1], vu[4 * rq + 2], vu[4 * rq + 3]},
                                  ein[ns][rq], a.bias != nullptr, gq, uq);
                    if (a.gu && m < a.M) {
                        *reinterpret_cast<uint2*>(a.gu + static_cast<int64_t>(m) * a.N + n) = gq;
                        *reinterpret_cast<uint2*>(a.gu + static_cast<int64_t>(m) * a.N + outN + n) = uq;
                    }
                }
            }
        }
        // LDS writes done, then a bare barrier: __syncthreads() would add a
        // release fence that waits for the previous pass's global stores
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        // LDS rows -> 16-byte streaming stores (the output is not read again
        // by this kernel).  Only calls with a residual load anything here, so
        // the plain path issues stores back to back with no vmcnt wait.
        auto store_pass = [&](auto WITH_RESID) __attribute__((always_inline)) {
#pragma unroll
            for (int c = tid; c < 64 * CPRO; c += C::THREADS) {
                const int row = c / CPRO, ch = c % CPRO;
                const int gm = m0 + (row >> 5) * 96 + ms * 32 + (row & 31);
                const int n = g * OUT_W + ch * 8;
                if (gm >= a.M || n >= outN) continue;
                const uint8_t* src = ((row >> 5) ? pair1 : pair0) + (row & 31) * OSTRIDE + ch * 16;
                uint4 v = *reinterpret_cast<const uint4*>(src);
                if constexpr (decltype(WITH_RESID)::value) {
                    if (a.ypre)
                        *reinterpret_cast<uint4*>(a.ypre + static_cast<int64_t>(gm) * a.N + n) = v;
                    const uint4 r = *reinterpret_cast<const uint4*>(a.resid + static_cast<int64_t>(gm) * a.N + n);
                    v.x = add_resid2(v.x, r.x);
                    v.y = add_resid2(v.y, r.y);
                    v.z = add_resid2(v.z, r.z);
                    v.w = add_resid2(v.w, r.w);
                }
                __builtin_nontemporal_store(u32x4_t{v.x, v.y, v.z, v.w},
                                            reinterpret_cast<u32x4_t*>(a.Y + static_cast<int64_t>(gm) * outN + n));
            }
        };
        if (EPI == Epi::PLAIN && a.resid) store_pass(std::true_type{});
        else store_pass(std::false_type{});
    }
}

}  // namespace

size_t wide_part_bytes(const GemmPlan& p) {
    // p.nt = BN; per thread NSUB x MSUB x 4 f32x4, NSUB = BN / wnw / 32, MSUB = 3
    const int nsub = p.nt / p.wnw / 32, msub = 3;
    return static_cast<size_t>(p.ksplit) * p.mblocks * p.groups * (p.waves * 64) * (nsub * msub * 4) * 16;
}

// Wide tilings compiled in, per operand class: (BN, waves along N, K per stage).
#define VLA_WIDE_GELU(X) X(256, 4, 64)
#define VLA_WIDE_BF16W(X) X(128, 4, 64)
#define VLA_WIDE_FP8A(X) X(256, 4, 64) X(128, 4, 128)
#define VLA_WIDE_BF16A(X) X(256, 4, 64) X(128, 4, 64)
#define VLA_WIDE_FP4W(X) X(256, 4, 64) X(128, 4, 64)

template <AType AT, WType WT, Epi EPI>
hipError_t launch_wide(const gemm_detail::KArgs& ka, const GemmPlan& p, hipStream_t s) {
    const dim3 grid(p.groups, p.mblocks, p.ksplit);
#define VLA_WIDE(BN_, WNW_, BK_)                                                        \
    if (p.nt == BN_ && p.wnw == WNW_ && p.waves == 2 * WNW_ && p.steps == BK_) {         \
        wide_gemm_kernel<AT, WT, EPI, BN_, WNW_, BK_><<<grid, 128 * WNW_, 0, s>>>(ka);  \
        return hipGetLastError();                                                       \
    }
    if constexpr (EPI == Epi::GELU_MUL) {
        VLA_WIDE_GELU(VLA_WIDE)
    } else if constexpr (WT == WType::BF16) {
        VLA_WIDE_BF16W(VLA_WIDE)
    } else if constexpr (WT == WType::FP4) {
        VLA_WIDE_FP4W(VLA_WIDE)
    } else if constexpr (AT == AType::FP8) {
        VLA_WIDE_FP8A(VLA_WIDE)
    } else {
        VLA_WIDE_BF16A(VLA_WIDE)
    }
#undef VLA_WIDE
    return hipErrorInvalidValue;
}

bool wide_dispatchable(const GemmPlan& p, AType at, WType wt, Epi epi) {
#define VLA_WIDE(BN_, WNW_, BK_) \
    if (p.nt == BN_ && p.wnw == WNW_ && p.waves == 2 * WNW_ && p.steps == BK_) return true;
    if (epi == Epi::GELU_MUL) {
        if (at != AType::BF16 || wt != WType::FP8) return false;
        VLA_WIDE_GELU(VLA_WIDE)
    } else if (wt == WType::BF16) {
        if (at != AType::BF16) return false;
        VLA_WIDE_BF16W(VLA_WIDE)
    } else if (wt == WType::FP4) {
        if (at != AType::BF16) return false;
        VLA_WIDE_FP4W(VLA_WIDE)
    } else if (at == AType::FP8) {
        VLA_WIDE_FP8A(VLA_WIDE)
    } else {
        VLA_WIDE_BF16A(VLA_WIDE)
    }
#undef VLA_WIDE
    return false;
}

template hipError_t launch_wide<AType::BF16, WType::FP8, Epi::PLAIN>(const gemm_detail::KArgs&, const GemmPlan&, hipStream_t);
template hipError_t launch_wide<AType::BF16, WType::FP8, Epi::GELU_MUL>(const gemm_detail::KArgs&, const GemmPlan&, hipStream_t);
template hipError_t launch_wide<AType::BF16, WType::BF16, Epi::PLAIN>(const gemm_detail::KArgs&, const GemmPlan&, hipStream_t);
template hipError_t launch_wide<AType::FP8, WType::FP8, Epi::PLAIN>(const gemm_detail::KArgs&, const GemmPlan&, hipStream_t);
template hipError_t launch_wide<AType::BF16, WType::FP4, Epi::PLAIN>(const gemm_detail::KArgs&, const GemmPlan&, hipStream_t);

}  // namespace vla
