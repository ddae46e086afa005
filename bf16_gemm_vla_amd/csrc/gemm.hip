// Skinny GEMM (M <= 64) for gfx950 on v_mfma_f32_16x16x32_bf16, the GEMM
// planner and the dispatch for both GEMM kernels (the wide kernel lives in
// gemm_wide.hip).
//
// Orientation: the packed weight fragment (16 output channels x 32 K) is
// the MFMA "A" operand and the activation fragment (16 rows x 32 K) the "B"
// operand, so each lane's accumulator holds 4 consecutive output channels
// of one activation row and stores 8 contiguous bytes of Y.
//
// Every wave loads all of its weight fragments up front (8 or 16 bytes per
// lane each, coalesced 512/1024-byte blocks), the bf16 activation chunk is
// staged through LDS with direct global->LDS loads, and the epilogue's
// scales/bias/residual are prefetched, so a workgroup has its whole share
// in flight before the first MFMA; the waves split K and reduce through LDS
// with one barrier.  Workgroups split the output columns, then the
// activation rows (blocks of 16-row tiles, no exchange needed), and only
// then K: when K is split across workgroups, each workgroup writes fp32
// partials and counts its arrival; the last to arrive sums the partials in
// split order (bitwise repeatable) and runs the epilogue.
#include <algorithm>
#include <mutex>

#include "gemm_common.h"

namespace vla {
namespace {

using namespace gemm_detail;

// ------------------------------------------------------------ skinny GEMM

template <WType WT>
struct WFragT;
template <>
struct WFragT<WType::FP8> { using type = u32x2_t; };
template <>
struct WFragT<WType::BF16> { using type = u32x4_t; };
template <>
struct WFragT<WType::FP4> { using type = uint32_t; };

template <AType AT>
struct AFragT;
template <>
struct AFragT<AType::FP8> { using type = u32x2_t; };
template <>
struct AFragT<AType::BF16> { using type = u32x4_t; };

template <WType WT>
__device__ __forceinline__ bf16x8_t w_operand(typename WFragT<WT>::type f) {
    if constexpr (WT == WType::FP8) return ocp8_to_bf16x8(f);
    else return as_bf16x8(f);
}
template <AType AT>
__device__ __forceinline__ bf16x8_t a_operand(typename AFragT<AT>::type f) {
    if constexpr (AT == AType::FP8) return ocp8_to_bf16x8(f);
    else return as_bf16x8(f);
}

// Tile index (16-column block of weight rows) of local tile j of group g.
template <Epi EPI, int NT>
__device__ __forceinline__ int skinny_tile(int g, int j, int N) {
    if constexpr (EPI == Epi::PLAIN) {
        return g * NT + j;
    } else {
        constexpr int H = NT / 2;
        return j < H ? g * H + j : (N >> 5) + g * H + (j - H);
    }
}

// ALDS: stage the (row-major bf16) activation chunk through LDS with direct
// global->LDS loads, one contiguous KiB per wave instruction, instead of
// loading MFMA fragments (16 rows x 64 B per instruction) from global memory.
template <int WAVES, int S, int MT>
struct SkinnyLds {
    static constexpr int CH = WAVES * S;             // K steps per workgroup chunk
    static constexpr int RB = CH * 64;               // bf16 bytes of one row's chunk
    static constexpr int RS = RB + 16;               // LDS row stride (bank spread)
    static constexpr int BYTES = MT * 16 * RS;       // the workgroup's rows
};

// One workgroup: NT 16-column weight tiles x MT 16-row activation tiles
// (rows m0 .. m0 + 16*MT - 1, m0 = 16*MT*blockIdx.z) x one K chunk
// (blockIdx.y) of WAVES * S MFMA steps, each wave S steps of it.
template <AType AT, WType WT, Epi EPI, int NT, int S, int WAVES, bool ALDS, int MT>
__global__ __launch_bounds__(WAVES * 64) void skinny_gemm_kernel(KArgs a) {
    using WF = typename WFragT<WT>::type;
    using AF = typename AFragT<AT>::type;
    constexpr int WB = (WT == WType::FP8) ? 8 : (WT == WType::FP4 ? 4 : 16);   // weight bytes per lane per fragment
    constexpr int AB = (AT == AType::FP8) ? 1 : 2;    // activation bytes per element
    constexpr int JO = (EPI == Epi::PLAIN) ? NT : NT / 2;   // output tiles per group
    constexpr int PAIRS = JO * MT;                           // (output tile, m-tile) fragments
    constexpr int R = (PAIRS + WAVES - 1) / WAVES;           // fragments finished per wave

    using L = SkinnyLds<WAVES, S, MT>;
    constexpr int RED_BYTES = WAVES * NT * MT * 64 * 16;
    // the reduction area follows the activation chunk when both fit, so the
    // partial sums need not wait for every wave to finish its LDS reads
    constexpr bool SEPARATE = ALDS && (L::BYTES + RED_BYTES <= 160 * 1024);
    constexpr int LDS_BYTES = SEPARATE ? L::BYTES + RED_BYTES : ((ALDS && L::BYTES > RED_BYTES) ? L::BYTES : RED_BYTES);
    static_assert(LDS_BYTES <= 160 * 1024 && L::BYTES % 16 == 0, "the workgroup's LDS fits");
    __shared__ __attribute__((aligned(16))) uint8_t lds[LDS_BYTES];
    auto red = reinterpret_cast<f32x4_t(*)[NT][MT][64]>(lds + (SEPARATE ? L::BYTES : 0));

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = blockIdx.x, split = blockIdx.y, mh = blockIdx.z;
    const int m0 = mh * MT * 16;                      // first activation row of the workgroup
    const int mrows = min(a.M - m0, MT * 16);         // rows of the workgroup (> 0)
    const int ksteps = a.K >> 5;
    const int kbase = split * WAVES * S + wave * S;
    const int mt_count = (mrows + 15) >> 4;
    const int ntiles = a.N >> 4;
    const int mrow = lane & 15, q = lane >> 4;

    // Loads, in this order: the epilogue inputs of the fragments this wave
    // finishes, the activation chunk (straight into LDS, ALDS), then exactly
    // S*NT weight-fragment loads (out-of-range ones read fragment 0 and are
    // zeroed).  vmcnt retires in order, so waiting until only the weight
    // loads are outstanding means the activations have landed: the barrier
    // and the LDS operand reads then overlap the weights' HBM latency.
    // 1. epilogue inputs
    EpiIn ein[R];
    const float sa = (AT == AType::FP8) ? *a.s_a : 1.0f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int pair = wave + r * WAVES, jo = pair / MT, mt = pair % MT;
        const int tile = skinny_tile<EPI, NT>(g, jo < JO ? jo : 0, a.N);
        const int row = mt * 16 + mrow;
        if (pair < PAIRS && tile < ntiles && row < mrows)
            ein[r] = load_epi<WT, EPI>(a, m0 + row, tile * 16 + 4 * q, a.ksplit == 1);
    }
    // 2. activation fragments: row m0 + mt*16 + lane%16, 8 K values at 8*(lane/16)
    AF af[S][MT];
    if constexpr (ALDS) {
        // issue this wave's share of the chunk's row pieces (1 KiB each)
        const int kstep0 = split * L::CH;
        constexpr int PIECES = (L::RB + 1023) / 1024;
        const int kel_row = kstep0 * 32;                       // first K element of the chunk
        for (int piece = wave; piece < mrows * PIECES; piece += WAVES) {
            const int row = piece / PIECES, p = piece % PIECES;    // row within the workgroup
            const int byte = p * 1024 + lane * 16;             // within the row chunk
            const int kel = kel_row + byte / 2;
            if (byte < L::RB && kel < a.K) {
                const uint8_t* src = static_cast<const uint8_t*>(a.A) + (static_cast<int64_t>(m0 + row) * a.K + kel) * 2;
                __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(lds + row * L::RS + p * 1024), 16, 0, 0);
            }
        }
    } else {
#pragma unroll
        for (int s = 0; s < S; ++s) {
            const bool ok = kbase + s < ksteps;
            const int64_t k = static_cast<int64_t>(kbase + s) * 32 + 8 * q;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int row = mt * 16 + mrow;
                if (ok && row < mrows)
                    af[s][mt] = *reinterpret_cast<const AF*>(static_cast<const uint8_t*>(a.A) +
                                                             (static_cast<int64_t>(m0 + row) * a.K + k) * AB);
                else
                    af[s][mt] = AF{};
            }
        }
    }
    // 3. all weight fragments of this wave in flight.  MXFP4: first the E8M0
    //    scales of the lane's row for the wave's S K steps, one aligned load
    //    per tile (rows of P bytes after the N*K/2 code bytes; kbase is a
    //    multiple of S, which divides 8, so the load stays inside the row)
    WF wf[S][NT];
    float wsc[S][NT];
    if constexpr (WT == WType::FP4) {
        static_assert(S == 1 || S == 2 || S == 4 || S == 8, "scale loads of 1, 2, 4 or 8 bytes");
        const int64_t P = mxfp4_scale_row_bytes(a.K);
        const uint8_t* const wscale = static_cast<const uint8_t*>(a.W) + static_cast<int64_t>(a.N) * a.K / 2;
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const int tile = skinny_tile<EPI, NT>(g, j, a.N);
            const bool valid = tile < ntiles && kbase < ksteps;
            const uint8_t* p = wscale + (valid ? (static_cast<int64_t>(tile) * 16 + (lane & 15)) * P + kbase : 0);
            uint32_t b[2] = {0, 0};
            if constexpr (S == 8) {
                const uint2 v = *reinterpret_cast<const uint2*>(p);
                b[0] = v.x; b[1] = v.y;
            } else if constexpr (S == 4) {
                b[0] = *reinterpret_cast<const uint32_t*>(p);
            } else if constexpr (S == 2) {
                b[0] = *reinterpret_cast<const uint16_t*>(p);
            } else {
                b[0] = *p;
            }
#pragma unroll
            for (int s = 0; s < S; ++s) {
                const uint32_t e = (b[s >> 2] >> (8 * (s & 3))) & 0xFFu;
                wsc[s][j] = (valid && kbase + s < ksteps) ? e8m0_to_f32(e) : 0.0f;
            }
        }
    }
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const bool ok = kbase + s < ksteps;
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const int tile = skinny_tile<EPI, NT>(g, j, a.N);
            const bool valid = ok && tile < ntiles;
            const int64_t fi = valid ? static_cast<int64_t>(tile) * ksteps + kbase + s : 0;
            const WF w = *reinterpret_cast<const WF*>(static_cast<const uint8_t*>(a.W) + (fi * 64 + lane) * WB);
            wf[s][j] = valid ? w : WF{};
        }
    }
    if constexpr (ALDS) {
        // the activations (and epilogue inputs) have landed once at most the
        // S*NT weight loads (and the NT scale loads) are outstanding; then
        // read the LDS fragments.  Capped at the field's 63: a lower count
        // only waits for a few more loads.
        constexpr int NW0 = S * NT + (WT == WType::FP4 ? NT : 0);
        constexpr int NW = NW0 < 63 ? NW0 : 63;
        __builtin_amdgcn_s_waitcnt((NW & 15) | ((NW >> 4) << 14) | 0x0F70);
        // a bare barrier: __syncthreads() would add a release fence that
        // waits for the weight loads too
        __builtin_amdgcn_s_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
#pragma unroll
        for (int s = 0; s < S; ++s) {
            const bool ok = kbase + s < ksteps;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int row = mt * 16 + mrow;
                if (ok && row < mrows)
                    af[s][mt] = *reinterpret_cast<const AF*>(lds + row * L::RS + ((wave * S + s) * 32 + 8 * q) * 2);
                else
                    af[s][mt] = AF{};
            }
        }
    }
    // 4. MFMA
    f32x4_t acc[NT][MT];
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[j][mt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < S; ++s) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            if (mt >= mt_count) break;
            const bf16x8_t bop = a_operand<AT>(af[s][mt]);
#pragma unroll
            for (int j = 0; j < NT; ++j)
                if constexpr (WT == WType::FP4)
                    acc[j][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp4_to_bf16x8(wf[s][j], wsc[s][j]), bop, acc[j][mt], 0, 0, 0);
                else
                    acc[j][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w_operand<WT>(wf[s][j]), bop, acc[j][mt], 0, 0, 0);
        }
    }
    if constexpr (ALDS && !SEPARATE) __syncthreads();   // activation reads done before LDS is reused
    // 5. cross-wave reduction through LDS with one barrier: every wave
    //    publishes its K slice, then wave w sums fragments w, w+WAVES, ...
    //    over all waves in wave order (bitwise repeatable)
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            if (mt < mt_count) red[wave][j][mt][lane] = acc[j][mt];
    __syncthreads();
    auto total = [&](int j, int mt) {
        f32x4_t v = red[0][j][mt][lane];
#pragma unroll
        for (int w = 1; w < WAVES; ++w) v += red[w][j][mt][lane];
        return v;
    };
    auto finish = [&](int r, int jo, int mt, f32x4_t v, f32x4_t u) {
        const int tile = skinny_tile<EPI, NT>(g, jo, a.N);
        const int row = mt * 16 + mrow;
        if (tile >= ntiles || row >= mrows) return;
        if constexpr (EPI == Epi::PLAIN) store_plain<AT, WT>(a, m0 + row, tile * 16 + 4 * q, v, ein[r], sa);
        else store_gelu(a, m0 + row, tile * 16 + 4 * q, v, u, ein[r]);
    };
    constexpr int JU = (EPI == Epi::PLAIN) ? 0 : NT / 2;     // offset of the matching up tile
    if (a.ksplit == 1) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int pair = wave + r * WAVES, jo = pair / MT, mt = pair % MT;
            if (pair >= PAIRS || mt >= mt_count) continue;
            finish(r, jo, mt, total(jo, mt), JU ? total(jo + JU, mt) : f32x4_t{});
        }
        return;
    }
    // 6. cross-workgroup split-K.  Partial layout [split][m split][group][NT][MT][64 lanes]
    //    of f32x4; every wave stores and later finishes its own fragments.
    const Coherent part(a.part, a.part_bytes);
    const int slot = mh * a.groups + g;
    auto off = [&](int sp, int j, int mt) {
        return static_cast<uint32_t>((((static_cast<int64_t>(sp) * a.msplit * a.groups + slot) * NT + j) * MT + mt) * 64 + lane) * 16u;
    };
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int pair = wave + r * WAVES, jo = pair / MT, mt = pair % MT;
        if (pair >= PAIRS || mt >= mt_count) continue;
        part.store(off(split, jo, mt), total(jo, mt));
        if (JU) part.store(off(split, jo + JU, mt), total(jo + JU, mt));
    }
    if (!splitk_arrive_last(a.tickets, slot, a.ksplit)) return;
    // the residual was not prefetched (only the last workgroup needs it)
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int pair = wave + r * WAVES, jo = pair / MT, mt = pair % MT;
        const int tile = skinny_tile<EPI, NT>(g, jo < JO ? jo : 0, a.N);
        const int row = mt * 16 + mrow;
        if (EPI == Epi::PLAIN && a.resid && pair < PAIRS && tile < ntiles && row < mrows)
            ein[r].resid = *reinterpret_cast<const uint2*>(a.resid + static_cast<int64_t>(m0 + row) * a.N + tile * 16 + 4 * q);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int pair = wave + r * WAVES, jo = pair / MT, mt = pair % MT;
        if (pair >= PAIRS || mt >= mt_count) continue;
        f32x4_t v = part.load(off(0, jo, mt));
        f32x4_t u = JU ? part.load(off(0, jo + JU, mt)) : f32x4_t{};
        for (int sp = 1; sp < a.ksplit; ++sp) {
            v += part.load(off(sp, jo, mt));
            if (JU) u += part.load(off(sp, jo + JU, mt));
        }
        finish(r, jo, mt, v, u);
    }
    splitk_reset(a.tickets, slot);
}

// ------------------------------------------------------------- dispatch

// Skinny tilings compiled in: (tiles per workgroup, K steps per wave, waves,
// 16-row activation tiles per workgroup).
#define VLA_SKINNY_CONFIGS(X)                                                                        \
    X(1, 1, 16, 4) X(1, 2, 16, 4) X(1, 4, 16, 4) X(1, 2, 8, 4) X(1, 4, 8, 4) X(1, 8, 8, 4) X(1, 8, 4, 4) \
    X(2, 1, 16, 4) X(2, 2, 16, 4) X(2, 2, 8, 4) X(2, 4, 8, 4) X(2, 4, 4, 4) X(2, 8, 4, 4)                \
    X(4, 1, 8, 4) X(4, 2, 8, 4) X(4, 2, 4, 4) X(4, 4, 4, 4)                                              \
    X(1, 2, 8, 1) X(1, 4, 8, 1) X(1, 4, 16, 1) X(1, 8, 16, 1)                                            \
    X(2, 2, 8, 1) X(2, 4, 8, 1) X(2, 4, 16, 1) X(2, 8, 16, 1)                                            \
    X(2, 4, 8, 2) X(4, 4, 8, 2) X(4, 4, 8, 1) X(8, 4, 8, 1) X(2, 2, 16, 2)

template <AType AT, WType WT, Epi EPI>
hipError_t launch_skinny(const KArgs& ka, const GemmPlan& p, hipStream_t s) {
    const dim3 grid(p.groups, p.ksplit, p.mblocks);
#define VLA_CASE(NT_, S_, W_, MT_)                                                                 \
    if (p.nt == NT_ && p.steps == S_ && p.waves == W_ && p.mt == MT_) {                            \
        if constexpr (EPI == Epi::GELU_MUL && NT_ < 2) {                                           \
            return hipErrorInvalidValue;                                                           \
        } else if constexpr (AT == AType::BF16 && SkinnyLds<W_, S_, MT_>::BYTES <= 160 * 1024) {   \
            if (p.alds) skinny_gemm_kernel<AT, WT, EPI, NT_, S_, W_, true, MT_><<<grid, W_ * 64, 0, s>>>(ka); \
            else skinny_gemm_kernel<AT, WT, EPI, NT_, S_, W_, false, MT_><<<grid, W_ * 64, 0, s>>>(ka);  \
        } else {                                                                                   \
            skinny_gemm_kernel<AT, WT, EPI, NT_, S_, W_, false, MT_><<<grid, W_ * 64, 0, s>>>(ka);      \
        }                                                                                          \
        return hipGetLastError();                                                                  \
    }
    VLA_SKINNY_CONFIGS(VLA_CASE)
#undef VLA_CASE
    return hipErrorInvalidValue;
}

template <AType AT, WType WT, Epi EPI>
hipError_t launch_typed(const KArgs& ka, const GemmPlan& p, hipStream_t s) {
    if (p.kernel == 0) return launch_skinny<AT, WT, EPI>(ka, p, s);
    if constexpr (WT == WType::FP4 && (AT != AType::BF16 || EPI != Epi::PLAIN)) return hipErrorInvalidValue;
    else return launch_wide<AT, WT, EPI>(ka, p, s);
}

// Skinny plan for a given tiling: groups of `nt` tiles, activation row
// blocks of `mt` 16-row tiles, K chunks of waves * steps MFMA steps.
GemmPlan skinny_plan(int64_t M, int64_t N, int64_t K, Epi epi, int nt, int steps, int waves, int mt,
                     bool alds = false) {
    GemmPlan p{};
    p.kernel = 0;
    p.nt = nt;
    p.steps = steps;
    p.waves = waves;
    p.mt = mt;
    p.alds = alds && static_cast<int64_t>(mt) * 16 * (static_cast<int64_t>(waves) * steps * 64 + 16) <= 160 * 1024;
    const int64_t tiles = N / 16, ksteps = K / 32;
    p.groups = static_cast<int>(std::max<int64_t>(1, epi == Epi::GELU_MUL ? (tiles / 2) / (nt / 2) : (tiles + nt - 1) / nt));
    p.ksplit = static_cast<int>((ksteps + static_cast<int64_t>(waves) * steps - 1) / (static_cast<int64_t>(waves) * steps));
    p.mblocks = static_cast<int>((M + 16 * mt - 1) / (16 * mt));
    // split-K: one counter per output group, and partials the kernel
    // addresses with 32-bit byte offsets
    const uint64_t part = static_cast<uint64_t>(p.ksplit) * p.mblocks * p.groups * nt * mt * 64 * 16;
    p.ok = p.ksplit == 1 || (static_cast<int64_t>(p.groups) * p.mblocks <= kMaxCounters && part < kMaxPartBytes);
    return p;
}

}  // namespace

GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K, AType at, WType wt, Epi epi) {
    const int64_t ksteps = K / 32;
    const int64_t tiles = N / 16;
    if (M <= 64) {
        // One 16-column tile (a gate/up pair for the fused epilogue) per
        // workgroup.  With at least ~256 such groups every workgroup takes
        // all rows and K chunks of at most 32 MFMA steps (1024 K).  With
        // fewer (the 4096 -> 1024 down-projection: 64 groups) the rows are
        // split first, one 16-row tile per workgroup, which needs no
        // exchange between workgroups (workgroups sharing a weight tile
        // sit on the same XCD, grid x being a multiple of 8 there, so the
        // tile streams from HBM once); K is split across workgroups only
        // for what remains.  Tilings measured on MI355X at M = 50: FP8
        // weights 8 waves x 4 steps, BF16 weights 16 waves x 2 steps;
        // bf16 activations staged through LDS.
        const int nt = (epi == Epi::GELU_MUL) ? 2 : 1;
        const int64_t groups = std::max<int64_t>(1, (epi == Epi::GELU_MUL) ? tiles / 2 : tiles);
        const int64_t mt_total = (M + 15) / 16;
        const int64_t want = groups >= 256 ? 1 : (256 + groups - 1) / groups;   // splits wanted
        // MXFP4 weights take the FP8 tilings (fewer weight bytes per fragment)
        // one 16-row tile and too few column groups, FP8 weights: no K split
        // up to 128 MFMA steps (K = 4096) — one 16-wave workgroup per tile
        // beats the cross-workgroup exchange (the 10-row 4096 -> 1024
        // down-projection: 6.30 -> 5.31 us against four K splits)
        if (want > 1 && mt_total == 1 && wt != WType::BF16 && epi == Epi::PLAIN && ksteps > 16 && ksteps <= 128)
            return skinny_plan(M, N, K, epi, nt, ksteps <= 64 ? 4 : 8, 16, 1, at == AType::BF16);
        if (want > 1 && mt_total > 1) {
            const int64_t ksplit = (want + mt_total - 1) / mt_total;
            const int64_t chunk = (ksteps + ksplit - 1) / ksplit;               // K steps per workgroup
            int steps, waves;
            if (chunk <= 16) { waves = 8; steps = 2; }
            else if (chunk <= 32) { waves = 8; steps = 4; }
            else if (chunk <= 64) { waves = 16; steps = 4; }
            else { waves = 16; steps = 8; }
            return skinny_plan(M, N, K, epi, nt, steps, waves, 1, at == AType::BF16);
        }
        const int64_t chunk = (ksteps + want - 1) / want;   // K steps per workgroup
        int steps, waves;
        if (wt == WType::BF16) {
            waves = 16;
            steps = chunk <= 16 ? 1 : 2;
        } else {
            waves = 8;
            steps = chunk <= 16 ? 2 : 4;
        }
        // FP8 weights, more than 32 rows: two 16-column tiles (two gate/up
        // pairs for the fused epilogue) x two row halves per workgroup read
        // 36% fewer bytes per CU than one tile (pair) x all rows (the
        // 1024 -> 4096 up-projection: 5.4 -> 5.1 us); BF16 weights the same
        // with their 16 waves x 2 steps.  The fused epilogue needs an even
        // number of gate tiles (a group never straddles the gate/up halves).
        if (mt_total > 2 && ((wt != WType::BF16 && steps == 4) || (wt == WType::BF16 && steps == 2)) &&
            (epi == Epi::PLAIN || (tiles / 2) % 2 == 0))
            return skinny_plan(M, N, K, epi, 2 * nt, steps, waves, 2, at == AType::BF16);
        return skinny_plan(M, N, K, epi, nt, steps, waves, 4, at == AType::BF16);
    }
    // Wide kernel: 192-row blocks; 256-column tiles when they give enough
    // workgroups, else 128-column tiles and K split until ~256 workgroups
    // (each split keeps at least 8 pipeline stages).  Wave layout: 8 waves
    // of 96 x BN/4; 64 K per stage, 128 for FP8 x FP8 on 128-column tiles
    // (FP8 x FP8 on 256-column tiles: 2048 -> 16384 at M = 768, 35.0 ->
    // 29.7 us against 4 waves of 96 x 128).  MXFP4 weights follow FP8's
    // choice (bf16 activations, codes converted with their block scales).
    // BF16 weights always take 128-column tiles (a 256-column stage would
    // not fit the four-stage LDS ring).  The buffer resources address A and
    // W with 32-bit offsets.
    GemmPlan p{};
    p.kernel = 1;
    p.mblocks = static_cast<int>((M + 191) / 192);
    if (epi == Epi::GELU_MUL) {
        p.nt = 256;
        p.groups = static_cast<int>(std::max<int64_t>(1, (tiles / 2 + 7) / 8));
    } else {
        const int64_t g256 = (tiles + 15) / 16;
        if (wt != WType::BF16 && g256 * p.mblocks >= 192) {
            p.nt = 256;
            p.groups = static_cast<int>(g256);
        } else {
            p.nt = 128;
            p.groups = static_cast<int>((tiles + 7) / 8);
        }
    }
    p.waves = 8;
    p.steps = (at == AType::FP8 && p.nt == 128) ? 128 : 64;   // K values per pipeline stage
    p.wnw = p.waves / 2;
    const int64_t kt_total = (K + p.steps - 1) / p.steps;
    const int64_t base = static_cast<int64_t>(p.groups) * p.mblocks;
    // the largest K split that keeps the grid within one workgroup per CU
    // (256) and at least 8 stages per split: a grid past 256 runs a second,
    // partial wave of workgroups (571 rows, 2048 -> 16384: 66 -> 46 us for
    // one split against two)
    int ks = 1;
    while (base * (ks + 1) <= 256 && kt_total / (ks + 1) >= 8) ++ks;
    p.ksplit = ks;
    const int64_t a_bytes = M * K * (at == AType::FP8 ? 1 : 2);
    const int64_t w_bytes = (wt == WType::FP4) ? N * K / 2 + N * (((K >> 5) + 7) & ~int64_t(7))
                                               : N * K * (wt == WType::FP8 ? 1 : 2);
    // split-K counters: kWideCounters per output tile; partials addressed
    // with 32-bit byte offsets
    p.ok = base * kWideCounters <= kMaxCounters && a_bytes < (int64_t(1) << 31) && w_bytes < (int64_t(1) << 31) &&
           (p.ksplit == 1 || wide_part_bytes(p) < kMaxPartBytes);
    return p;
}

size_t gemm_ws_bytes(const GemmPlan& p, int64_t M, int64_t N) {
    (void)N;
    (void)M;
    if (p.ksplit <= 1) return kCounterBytes;
    size_t part;
    if (p.kernel == 0)
        part = static_cast<size_t>(p.ksplit) * p.mblocks * p.groups * p.nt * p.mt * 64 * 16;
    else
        part = wide_part_bytes(p);
    return kCounterBytes + part;
}

hipError_t launch_gemm_plan(const GemmProblem& pr, const GemmPlan& p, hipStream_t s) {
    KArgs ka{};
    ka.A = pr.A; ka.s_a = pr.s_a; ka.W = pr.W; ka.s_w = pr.s_w;
    ka.bias = pr.bias; ka.resid = pr.resid; ka.Y = pr.Y; ka.gu = pr.gu; ka.ypre = pr.ypre;
    ka.M = static_cast<int>(pr.M); ka.N = static_cast<int>(pr.N); ka.K = static_cast<int>(pr.K);
    ka.ksplit = p.ksplit;
    ka.groups = p.groups;
    ka.msplit = p.mblocks;
    ka.tickets = static_cast<uint32_t*>(pr.ws);
    ka.err = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(pr.ws) + kStatusOffset);
    ka.wait_polls = wait_polls();
    ka.part = reinterpret_cast<float*>(static_cast<uint8_t*>(pr.ws) + kCounterBytes);
    // below 2^32 for every plan marked ok (plan_gemm checks it)
    ka.part_bytes = static_cast<uint32_t>(gemm_ws_bytes(p, pr.M, pr.N) - kCounterBytes);

    if (pr.epi == Epi::GELU_MUL) return launch_typed<AType::BF16, WType::FP8, Epi::GELU_MUL>(ka, p, s);
    if (pr.wtype == WType::BF16) return launch_typed<AType::BF16, WType::BF16, Epi::PLAIN>(ka, p, s);
    if (pr.wtype == WType::FP4) return launch_typed<AType::BF16, WType::FP4, Epi::PLAIN>(ka, p, s);
    if (pr.atype == AType::FP8) return launch_typed<AType::FP8, WType::FP8, Epi::PLAIN>(ka, p, s);
    return launch_typed<AType::BF16, WType::FP8, Epi::PLAIN>(ka, p, s);
}

hipError_t launch_gemm(const GemmProblem& pr, hipStream_t s) {
    return launch_gemm_plan(pr, plan_gemm(pr.M, pr.N, pr.K, pr.atype, pr.wtype, pr.epi), s);
}

bool plan_dispatchable(const GemmPlan& p, AType at, WType wt, Epi epi) {
    if (!p.ok) return false;
    if (p.kernel != 0) return wide_dispatchable(p, at, wt, epi);
#define VLA_CASE(NT_, S_, W_, MT_) \
    if (p.nt == NT_ && p.steps == S_ && p.waves == W_ && p.mt == MT_) return !(epi == Epi::GELU_MUL && NT_ < 2);
    VLA_SKINNY_CONFIGS(VLA_CASE)
#undef VLA_CASE
    return false;
}

// ------------------------------------------------ library-owned workspace

namespace {

// The workspace of vla_gemm_fp8w_noalloc: one per GPU, in the code object's
// device memory, held until the process ends.  In host code `scratch` is
// only a stand-in for the symbol: its device address comes from
// hipGetSymbolAddress, once per device, and only that address is passed to
// kernels.
static __device__ __align__(256) uint8_t scratch[kNoAllocWorkspaceBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
bool g_scratch_clear[kMaxDevices] = {};

__global__ void zero_words_kernel(uint32_t* p, int n) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0;
}

}  // namespace

hipError_t noalloc_workspace(hipStream_t s, void** ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    if (!g_scratch_clear[dev]) {
        // the split-K counters and the status word must start at zero (every
        // completed call leaves the counters at zero again); cleared by a
        // kernel, not a memset, so a capturing caller records a kernel node
        zero_words_kernel<<<16, 256, 0, s>>>(static_cast<uint32_t*>(g_scratch_ptr[dev]),
                                             static_cast<int>(kCounterBytes / 4));
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        e = hipStreamIsCapturing(s, &cs);
        if (e != hipSuccess) return e;
        // under capture the clear runs only when the graph does: keep clearing
        // until a call runs eagerly
        if (cs == hipStreamCaptureStatusNone) g_scratch_clear[dev] = true;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace vla
