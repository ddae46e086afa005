// BF16/FP8-weight GEMMs for gfx950, built on v_mfma_f32_16x16x32_bf16 and
// v_mfma_f32_16x16x32_fp8_fp8 (OCP E4M3 on gfx950).
//
// Orientation: the packed weight fragment (16 output channels x 32 K) is
// the MFMA "A" operand and the activation fragment (16 rows x 32 K) the "B"
// operand, so each lane's accumulator holds 4 consecutive output channels
// of one activation row and stores 8 contiguous bytes of Y.
//
// Skinny kernel (M <= 64): every wave loads all of its weight fragments up
// front (8 or 16 bytes per lane each, coalesced 512/1024-byte blocks) and
// its activation fragments straight into registers, so a workgroup has its
// whole share in flight before the first MFMA; the waves split K and reduce
// through LDS.  When K is split across workgroups too, each workgroup
// writes fp32 partials and counts its arrival; the last to arrive sums the
// partials in split order (bitwise repeatable) and runs the epilogue.
//
// Cross-workgroup protocol: partials are written and read only with
// device-coherent (agent-scope atomic) accesses, which gfx950 serves from
// the coherent level of the hierarchy, and every wave waits for its stores
// to complete before the workgroup's arrival is counted.  This is the
// ordering a release/acquire pair provides, without the L2 write-back and
// invalidate that a device-scope fence issues (they cost ~20 us per call
// here, against a ~1 us kernel).
//
// Wide kernel (M > 64): 128 x 128 output tile per 256-thread workgroup,
// BK = 64, global -> LDS double buffering, both operands stored in LDS in
// MFMA fragment order (conflict-free 8/16-byte lane reads).
#include <algorithm>

#include "vla_device.h"
#include "vla_internal.h"

namespace vla {
namespace {

constexpr int kThreads = 256;

struct KArgs {
    const void* A;
    const float* s_a;
    const void* W;
    const float* s_w;
    const uint16_t* bias;
    const uint16_t* resid;
    uint16_t* Y;
    uint16_t* gu;
    uint32_t* tickets;
    float* part;
    uint32_t part_bytes;
    int M, N, K;
    int ksplit;
    int groups;
};

// ------------------------------------------------------------- epilogue

// Epilogue inputs of one output fragment (row m, output columns n..n+3),
// loaded early so their latency overlaps the weight stream.
struct EpiIn {
    float4 s;       // weight scales (gate scales for the fused gate/up epilogue)
    float4 su;      // up scales (fused gate/up epilogue)
    uint2 bias;
    uint2 resid;
};

__device__ __forceinline__ uint16_t lo16(uint32_t w) { return static_cast<uint16_t>(w & 0xFFFFu); }
__device__ __forceinline__ uint16_t hi16(uint32_t w) { return static_cast<uint16_t>(w >> 16); }
__device__ __forceinline__ uint2 pack4(const uint16_t* x) {
    return make_uint2(x[0] | (static_cast<uint32_t>(x[1]) << 16), x[2] | (static_cast<uint32_t>(x[3]) << 16));
}

template <WType WT, Epi EPI>
__device__ __forceinline__ EpiIn load_epi(const KArgs& a, int m, int n, bool with_resid) {
    EpiIn e;
    e.s = make_float4(1.0f, 1.0f, 1.0f, 1.0f);
    e.su = e.s;
    e.bias = make_uint2(0, 0);
    e.resid = make_uint2(0, 0);
    if (WT == WType::FP8) e.s = *reinterpret_cast<const float4*>(a.s_w + n);
    if (EPI == Epi::GELU_MUL) {
        e.su = *reinterpret_cast<const float4*>(a.s_w + (a.N >> 1) + n);
    } else {
        if (a.bias) e.bias = *reinterpret_cast<const uint2*>(a.bias + n);
        if (a.resid && with_resid) e.resid = *reinterpret_cast<const uint2*>(a.resid + static_cast<int64_t>(m) * a.N + n);
    }
    return e;
}

// y = v * scale (+ bias) -> bf16, then bf16(residual + y); four columns.
template <AType AT, WType WT>
__device__ __forceinline__ void store_plain(const KArgs& a, int m, int n, f32x4_t v, const EpiIn& e, float sa) {
    const float sc[4] = {e.s.x * sa, e.s.y * sa, e.s.z * sa, e.s.w * sa};
    const uint16_t b[4] = {lo16(e.bias.x), hi16(e.bias.x), lo16(e.bias.y), hi16(e.bias.y)};
    uint16_t o[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        float y = (WT == WType::FP8 || AT == AType::FP8) ? v[r] * sc[r] : v[r];
        if (a.bias) y += bf16_to_f32(b[r]);
        o[r] = f32_to_bf16(y);
    }
    if (a.resid) {
        const uint16_t rv[4] = {lo16(e.resid.x), hi16(e.resid.x), lo16(e.resid.y), hi16(e.resid.y)};
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = f32_to_bf16(bf16_to_f32(rv[r]) + bf16_to_f32(o[r]));
    }
    *reinterpret_cast<uint2*>(a.Y + static_cast<int64_t>(m) * a.N + n) = pack4(o);
}

// Gate values vg and up values vu for row m, gate columns n..n+3 (n < I).
__device__ __forceinline__ void store_gelu(const KArgs& a, int m, int n, f32x4_t vg, f32x4_t vu, const EpiIn& e) {
    const int I = a.N >> 1;
    const float sgv[4] = {e.s.x, e.s.y, e.s.z, e.s.w}, suv[4] = {e.su.x, e.su.y, e.su.z, e.su.w};
    uint16_t g[4], u[4], o[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        g[r] = f32_to_bf16(vg[r] * sgv[r]);
        u[r] = f32_to_bf16(vu[r] * suv[r]);
        o[r] = f32_to_bf16(gelu_tanh(bf16_to_f32(g[r])) * bf16_to_f32(u[r]));
    }
    *reinterpret_cast<uint2*>(a.Y + static_cast<int64_t>(m) * I + n) = pack4(o);
    if (a.gu) {
        *reinterpret_cast<uint2*>(a.gu + static_cast<int64_t>(m) * a.N + n) = pack4(g);
        *reinterpret_cast<uint2*>(a.gu + static_cast<int64_t>(m) * a.N + I + n) = pack4(u);
    }
}

// Device-coherent 16-byte partial stores / loads.  They use the cache
// policy of agent-scope atomic accesses (sc1), served at the level of the
// hierarchy every XCD sees, through a buffer resource bounded to the
// partial region (out-of-range offsets read zero and drop writes).
constexpr int kCpolSC1 = 16;                 // cache-policy bit SC1
constexpr int kRsrcWord3 = 0x00020000;       // raw buffer, 32-bit data format

struct Coherent {
    __amdgpu_buffer_rsrc_t r;
    __device__ Coherent(void* base, uint32_t bytes) : r(__builtin_amdgcn_make_buffer_rsrc(base, 0, bytes, kRsrcWord3)) {}
    __device__ void store(uint32_t off, f32x4_t v) const {
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, off, 0, kCpolSC1);
    }
    __device__ f32x4_t load(uint32_t off) const {
        return __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCpolSC1));
    }
};

// Split-K arrival, called by every thread after storing its partials with
// Coherent::store.  Returns true in the one workgroup that arrives last for
// `slot`; that workgroup then reads every partial with Coherent::load and
// must call splitk_reset when done.
__device__ __forceinline__ bool splitk_arrive_last(uint32_t* tickets, int slot, int ksplit) {
    __shared__ int s_last;
    // wait until this wave's partial stores have completed (gfx9 counts
    // stores in vmcnt); the barrier then orders every wave's stores before
    // the arrival below
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t prev = __hip_atomic_fetch_add(tickets + slot, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = (prev == static_cast<uint32_t>(ksplit - 1)) ? 1 : 0;
    }
    __syncthreads();
    return s_last != 0;
}

__device__ __forceinline__ void splitk_reset(uint32_t* tickets, int slot) {
    if (threadIdx.x == 0) __hip_atomic_store(tickets + slot, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------ skinny GEMM

template <WType WT>
struct WFragT;
template <>
struct WFragT<WType::FP8> { using type = u32x2_t; };
template <>
struct WFragT<WType::BF16> { using type = u32x4_t; };

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
template <int WAVES, int S>
struct SkinnyLds {
    static constexpr int CH = WAVES * S;             // K steps per workgroup chunk
    static constexpr int RB = CH * 64;               // bf16 bytes of one row's chunk
    static constexpr int RS = RB + 16;               // LDS row stride (bank spread)
    static constexpr int BYTES = 64 * RS;            // up to 64 rows
};

template <AType AT, WType WT, Epi EPI, int NT, int S, int WAVES, bool ALDS>
__global__ __launch_bounds__(WAVES * 64) void skinny_gemm_kernel(KArgs a) {
    using WF = typename WFragT<WT>::type;
    using AF = typename AFragT<AT>::type;
    constexpr int WB = (WT == WType::FP8) ? 8 : 16;   // weight bytes per lane per fragment
    constexpr int AB = (AT == AType::FP8) ? 1 : 2;    // activation bytes per element
    constexpr int JO = (EPI == Epi::PLAIN) ? NT : NT / 2;   // output tiles per group
    constexpr int PAIRS = JO * 4;                            // (output tile, m-tile) fragments
    constexpr int R = (PAIRS + WAVES - 1) / WAVES;           // fragments finished per wave

    using L = SkinnyLds<WAVES, S>;
    constexpr int RED_BYTES = WAVES * NT * 4 * 64 * 16;
    constexpr int LDS_BYTES = (ALDS && L::BYTES > RED_BYTES) ? L::BYTES : RED_BYTES;
    __shared__ __attribute__((aligned(16))) uint8_t lds[LDS_BYTES];
    auto red = reinterpret_cast<f32x4_t(*)[NT][4][64]>(lds);

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = blockIdx.x, split = blockIdx.y;
    const int ksteps = a.K >> 5;
    const int kbase = split * WAVES * S + wave * S;
    const int mt_count = (a.M + 15) >> 4;
    const int ntiles = a.N >> 4;
    const int mrow = lane & 15, q = lane >> 4;

    // 1. all weight fragments of this wave in flight
    WF wf[S][NT];
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const bool ok = kbase + s < ksteps;
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const int tile = skinny_tile<EPI, NT>(g, j, a.N);
            const int64_t fi = static_cast<int64_t>(tile) * ksteps + kbase + s;
            const uint8_t* p = static_cast<const uint8_t*>(a.W) + (fi * 64 + lane) * WB;
            if (ok && tile < ntiles) wf[s][j] = *reinterpret_cast<const WF*>(p);
            else wf[s][j] = WF{};
        }
    }
    // 2. activation fragments: row mt*16 + lane%16, 8 K values at 8*(lane/16)
    AF af[S][4];
    if constexpr (ALDS) {
        // issue this wave's share of the chunk's row pieces (1 KiB each)
        const int kstep0 = split * L::CH;
        constexpr int PIECES = (L::RB + 1023) / 1024;
        const int kel_row = kstep0 * 32;                       // first K element of the chunk
        for (int piece = wave; piece < a.M * PIECES; piece += WAVES) {
            const int row = piece / PIECES, p = piece % PIECES;
            const int byte = p * 1024 + lane * 16;             // within the row chunk
            const int kel = kel_row + byte / 2;
            if (byte < L::RB && kel < a.K) {
                const uint8_t* src = static_cast<const uint8_t*>(a.A) + (static_cast<int64_t>(row) * a.K + kel) * 2;
                __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(lds + row * L::RS + p * 1024), 16, 0, 0);
            }
        }
    } else {
#pragma unroll
        for (int s = 0; s < S; ++s) {
            const bool ok = kbase + s < ksteps;
            const int64_t k = static_cast<int64_t>(kbase + s) * 32 + 8 * q;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const int row = mt * 16 + mrow;
                if (ok && row < a.M)
                    af[s][mt] = *reinterpret_cast<const AF*>(static_cast<const uint8_t*>(a.A) +
                                                             (static_cast<int64_t>(row) * a.K + k) * AB);
                else
                    af[s][mt] = AF{};
            }
        }
    }
    // 3. epilogue inputs of the fragments this wave finishes (overlaps the loads)
    EpiIn ein[R];
    const float sa = (AT == AType::FP8) ? *a.s_a : 1.0f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int pair = wave + r * WAVES, jo = pair >> 2, mt = pair & 3;
        const int tile = skinny_tile<EPI, NT>(g, jo < JO ? jo : 0, a.N);
        const int m = mt * 16 + mrow;
        if (pair < PAIRS && tile < ntiles && m < a.M)
            ein[r] = load_epi<WT, EPI>(a, m, tile * 16 + 4 * q, a.ksplit == 1);
    }
    if constexpr (ALDS) {
        // every wave's direct-to-LDS loads have landed, then read fragments
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
#pragma unroll
        for (int s = 0; s < S; ++s) {
            const bool ok = kbase + s < ksteps;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const int row = mt * 16 + mrow;
                if (ok && row < a.M)
                    af[s][mt] = *reinterpret_cast<const AF*>(lds + row * L::RS + ((wave * S + s) * 32 + 8 * q) * 2);
                else
                    af[s][mt] = AF{};
            }
        }
    }
    // 4. MFMA
    f32x4_t acc[NT][4];
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) acc[j][mt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < S; ++s) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            if (mt >= mt_count) break;
            const bf16x8_t bop = a_operand<AT>(af[s][mt]);
#pragma unroll
            for (int j = 0; j < NT; ++j)
                acc[j][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w_operand<WT>(wf[s][j]), bop, acc[j][mt], 0, 0, 0);
        }
    }
    if constexpr (ALDS) __syncthreads();   // activation reads done before LDS is reused
    // 5. cross-wave reduction through LDS with one barrier: every wave
    //    publishes its K slice, then wave w sums fragments w, w+WAVES, ...
    //    over all waves in wave order (bitwise repeatable)
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
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
        const int m = mt * 16 + mrow;
        if (tile >= ntiles || m >= a.M) return;
        if constexpr (EPI == Epi::PLAIN) store_plain<AT, WT>(a, m, tile * 16 + 4 * q, v, ein[r], sa);
        else store_gelu(a, m, tile * 16 + 4 * q, v, u, ein[r]);
    };
    constexpr int JU = (EPI == Epi::PLAIN) ? 0 : NT / 2;     // offset of the matching up tile
    if (a.ksplit == 1) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int pair = wave + r * WAVES, jo = pair >> 2, mt = pair & 3;
            if (pair >= PAIRS || mt >= mt_count) continue;
            finish(r, jo, mt, total(jo, mt), JU ? total(jo + JU, mt) : f32x4_t{});
        }
        return;
    }
    // 6. cross-workgroup split-K.  Partial layout [split][group][NT][4 mt][64 lanes]
    //    of f32x4; every wave stores and later finishes its own fragments.
    const Coherent part(a.part, a.part_bytes);
    auto off = [&](int sp, int j, int mt) {
        return static_cast<uint32_t>((((static_cast<int64_t>(sp) * a.groups + g) * NT + j) * 4 + mt) * 64 + lane) * 16u;
    };
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int pair = wave + r * WAVES, jo = pair >> 2, mt = pair & 3;
        if (pair >= PAIRS || mt >= mt_count) continue;
        part.store(off(split, jo, mt), total(jo, mt));
        if (JU) part.store(off(split, jo + JU, mt), total(jo + JU, mt));
    }
    if (!splitk_arrive_last(a.tickets, g, a.ksplit)) return;
    // the residual was not prefetched (only the last workgroup needs it)
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int pair = wave + r * WAVES, jo = pair >> 2, mt = pair & 3;
        const int tile = skinny_tile<EPI, NT>(g, jo < JO ? jo : 0, a.N);
        const int m = mt * 16 + mrow;
        if (EPI == Epi::PLAIN && a.resid && pair < PAIRS && tile < ntiles && m < a.M)
            ein[r].resid = *reinterpret_cast<const uint2*>(a.resid + static_cast<int64_t>(m) * a.N + tile * 16 + 4 * q);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int pair = wave + r * WAVES, jo = pair >> 2, mt = pair & 3;
        if (pair >= PAIRS || mt >= mt_count) continue;
        f32x4_t v = part.load(off(0, jo, mt));
        f32x4_t u = JU ? part.load(off(0, jo + JU, mt)) : f32x4_t{};
        for (int sp = 1; sp < a.ksplit; ++sp) {
            v += part.load(off(sp, jo, mt));
            if (JU) u += part.load(off(sp, jo + JU, mt));
        }
        finish(r, jo, mt, v, u);
    }
    splitk_reset(a.tickets, g);
}

// -------------------------------------------------------------- wide GEMM

constexpr int kBM = 128;   // x 128 columns; BK = 64 = two 32-wide MFMA K steps

template <Epi EPI>
__device__ __forceinline__ int wide_tile(int g, int lt, int N) {
    if constexpr (EPI == Epi::PLAIN) {
        return g * 8 + lt;
    } else {
        // wave column wn holds gate columns g*4 + wn*2 + {0,1} and the
        // matching up columns, so each lane has g and u of the same output
        const int wn = lt >> 2, j = lt & 3;
        const int c = g * 4 + wn * 2 + (j & 1);
        return j < 2 ? c : (N >> 5) + c;
    }
}

template <AType AT, WType WT, Epi EPI>
__global__ __launch_bounds__(kThreads) void wide_gemm_kernel(KArgs a) {
    constexpr int ALB = (AT == AType::FP8) ? 8 : 16;   // A bytes per lane per fragment
    constexpr int WLB = (WT == WType::FP8) ? 8 : 16;   // W bytes per lane per fragment
    constexpr int A_BUF = 8 * 2 * 64 * ALB;            // 8 m-tiles x 2 k-steps
    constexpr int W_BUF = 8 * 2 * 64 * WLB;            // 8 n-tiles x 2 k-steps
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * (A_BUF + W_BUF)];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int g = blockIdx.x, mb = blockIdx.y, split = blockIdx.z;
    const int m0 = mb * kBM;
    const int ksteps = a.K >> 5;
    const int ntiles16 = a.N >> 4;
    // K range of this split, in steps; chunks are multiples of 2 steps
    const int kt_total = (ksteps + 1) >> 1;
    const int kt_per = (kt_total + a.ksplit - 1) / a.ksplit;
    const int kt_begin = split * kt_per;
    const int kt_end = min(kt_total, kt_begin + kt_per);
    const int nkt = max(0, kt_end - kt_begin);

    constexpr int A_CHUNKS = (kBM * 64 * (AT == AType::FP8 ? 1 : 2)) / 16 / kThreads;   // 4 or 2
    constexpr int W_CHUNKS = W_BUF / 16 / kThreads;                                      // 2 or 4
    uint4 ra[A_CHUNKS], rw[W_CHUNKS];

    auto load_global = [&](int kt) {
        const int ks0 = kt * 2;
#pragma unroll
        for (int i = 0; i < A_CHUNKS; ++i) {
            const int c = tid + kThreads * i;
            int row, kbyte;
            if constexpr (AT == AType::FP8) { row = c >> 2; kbyte = (c & 3) * 16; }
            else { row = c >> 3; kbyte = (c & 7) * 16; }
            const int gm = m0 + row;
            const int64_t kel = static_cast<int64_t>(ks0) * 32 + kbyte / (AT == AType::FP8 ? 1 : 2);
            if (gm < a.M && kel < a.K)
                ra[i] = *reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(a.A) +
                                                         (static_cast<int64_t>(gm) * a.K) * (AT == AType::FP8 ? 1 : 2) +
                                                         kel * (AT == AType::FP8 ? 1 : 2));
            else
                ra[i] = make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < W_CHUNKS; ++i) {
            const int c = tid + kThreads * i;
            const int per_tile = 2 * 64 * WLB / 16;      // 16-byte chunks per tile strip
            const int lt = c / per_tile, off = (c % per_tile) * 16;
            const int tile = wide_tile<EPI>(g, lt, a.N);
            const int ks = ks0 + off / (64 * WLB);
            if (tile < ntiles16 && ks < ksteps)
                rw[i] = *reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(a.W) +
                                                         (static_cast<int64_t>(tile) * ksteps + ks0) * 64 * WLB + off);
            else
                rw[i] = make_uint4(0, 0, 0, 0);
        }
    };
    auto store_lds = [&](int buf) {
        uint8_t* sa = lds + buf * (A_BUF + W_BUF);
        uint8_t* sw = sa + A_BUF;
#pragma unroll
        for (int i = 0; i < A_CHUNKS; ++i) {
            const int c = tid + kThreads * i;
            if constexpr (AT == AType::FP8) {
                const int row = c >> 2, kc = c & 3;             // 16 fp8 = lanes k1, k1+1
                const int ks = kc >> 1, k1 = (kc & 1) * 2;
                uint8_t* d0 = sa + ((((row >> 4) * 2 + ks) * 64) + 16 * k1 + (row & 15)) * 8;
                *reinterpret_cast<uint2*>(d0) = make_uint2(ra[i].x, ra[i].y);
                *reinterpret_cast<uint2*>(d0 + 16 * 8) = make_uint2(ra[i].z, ra[i].w);
            } else {
                const int row = c >> 3, kc = c & 7;
                const int ks = kc >> 2, k1 = kc & 3;
                *reinterpret_cast<uint4*>(sa + ((((row >> 4) * 2 + ks) * 64) + 16 * k1 + (row & 15)) * 16) = ra[i];
            }
        }
#pragma unroll
        for (int i = 0; i < W_CHUNKS; ++i) {
            const int c = tid + kThreads * i;
            *reinterpret_cast<uint4*>(sw + c * 16) = rw[i];
        }
    };

    f32x4_t acc[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) acc[j][mt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

    if (nkt > 0) {
        load_global(kt_begin);
        store_lds(0);
        __syncthreads();
        for (int i = 0; i < nkt; ++i) {
            const int buf = i & 1;
            if (i + 1 < nkt) load_global(kt_begin + i + 1);
            const uint8_t* sa = lds + buf * (A_BUF + W_BUF);
            const uint8_t* sw = sa + A_BUF;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                if constexpr (AT == AType::FP8) {
                    long av[4], wv[4];
#pragma unroll
                    for (int mt = 0; mt < 4; ++mt)
                        av[mt] = *reinterpret_cast<const long*>(sa + ((((wm * 4 + mt) * 2 + ks) * 64) + lane) * 8);
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        wv[j] = *reinterpret_cast<const long*>(sw + ((((wn * 4 + j) * 2 + ks) * 64) + lane) * 8);
#pragma unroll
                    for (int j = 0; j < 4; ++j)
#pragma unroll
                        for (int mt = 0; mt < 4; ++mt)
                            acc[j][mt] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(wv[j], av[mt], acc[j][mt], 0, 0, 0);
                } else {
                    bf16x8_t av[4], wv[4];
#pragma unroll
                    for (int mt = 0; mt < 4; ++mt)
                        av[mt] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(sa + ((((wm * 4 + mt) * 2 + ks) * 64) + lane) * 16));
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint8_t* p = sw + ((((wn * 4 + j) * 2 + ks) * 64) + lane) * WLB;
                        if constexpr (WT == WType::FP8) wv[j] = ocp8_to_bf16x8(*reinterpret_cast<const u32x2_t*>(p));
                        else wv[j] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(p));
                    }
#pragma unroll
                    for (int j = 0; j < 4; ++j)
#pragma unroll
                        for (int mt = 0; mt < 4; ++mt)
                            acc[j][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wv[j], av[mt], acc[j][mt], 0, 0, 0);
                }
            }
            if (i + 1 < nkt) store_lds(buf ^ 1);
            __syncthreads();
        }
    }

    // Epilogue.  Lane holds, for local tile (wn*4 + j) and m-tile (wm*4 + mt),
    // rows m = m0 + (wm*4+mt)*16 + lane%16, columns 4*(lane/16) + 0..3.
    const int mrow = lane & 15, q = lane >> 4;
    if (a.ksplit > 1) {
        // partial layout: [split][mblock][group][16 fragments][256 threads] of f32x4
        const int64_t slot = static_cast<int64_t>(mb) * a.groups + g;
        const int64_t per = static_cast<int64_t>(kThreads) * 16;
        const int64_t sstride = static_cast<int64_t>(gridDim.y) * a.groups * per;
        const Coherent part(a.part, a.part_bytes);
        auto off = [&](int sp, int f) { return static_cast<uint32_t>((sp * sstride + slot * per + f * kThreads + tid) * 16); };
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) part.store(off(split, j * 4 + mt), acc[j][mt]);
        if (!splitk_arrive_last(a.tickets, static_cast<int>(slot), a.ksplit)) return;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                f32x4_t v = part.load(off(0, j * 4 + mt));
                for (int sp = 1; sp < a.ksplit; ++sp) v += part.load(off(sp, j * 4 + mt));
                acc[j][mt] = v;
            }
        splitk_reset(a.tickets, static_cast<int>(slot));
    }
    const float sa = (AT == AType::FP8) ? *a.s_a : 1.0f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        const int m = m0 + (wm * 4 + mt) * 16 + mrow;
        if (m >= a.M) continue;
        if constexpr (EPI == Epi::PLAIN) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int tile = wide_tile<EPI>(g, wn * 4 + j, a.N);
                if (tile < ntiles16) {
                    const int n = tile * 16 + 4 * q;
                    store_plain<AT, WT>(a, m, n, acc[j][mt], load_epi<WT, EPI>(a, m, n, true), sa);
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int tile = wide_tile<EPI>(g, wn * 4 + j, a.N);
                if (tile < (a.N >> 5)) {
                    const int n = tile * 16 + 4 * q;
                    store_gelu(a, m, n, acc[j][mt], acc[j + 2][mt], load_epi<WT, EPI>(a, m, n, false));
                }
            }
        }
    }
}

// ------------------------------------------------------------- dispatch

// Skinny tilings compiled in: (tiles per workgroup, K steps per wave, waves).
#define VLA_SKINNY_CONFIGS(X) \
    X(1, 1, 16) X(1, 2, 16) X(1, 4, 16) X(1, 2, 8) X(1, 4, 8) X(1, 8, 8) X(1, 8, 4) \
    X(2, 1, 16) X(2, 2, 16) X(2, 2, 8) X(2, 4, 8) X(2, 4, 4) X(2, 8, 4)             \
    X(4, 1, 8) X(4, 2, 8) X(4, 2, 4) X(4, 4, 4)

template <AType AT, WType WT, Epi EPI>
hipError_t launch_skinny(const KArgs& ka, const GemmPlan& p, hipStream_t s) {
    const dim3 grid(p.groups, p.ksplit);
#define VLA_CASE(NT_, S_, W_)                                                                      \
    if (p.nt == NT_ && p.steps == S_ && p.waves == W_) {                                           \
        if constexpr (EPI == Epi::GELU_MUL && NT_ < 2) {                                           \
            return hipErrorInvalidValue;                                                           \
        } else if constexpr (AT == AType::BF16 && W_ * S_ <= 32) {                                 \
            if (p.alds) skinny_gemm_kernel<AT, WT, EPI, NT_, S_, W_, true><<<grid, W_ * 64, 0, s>>>(ka); \
            else skinny_gemm_kernel<AT, WT, EPI, NT_, S_, W_, false><<<grid, W_ * 64, 0, s>>>(ka);  \
        } else {                                                                                   \
            skinny_gemm_kernel<AT, WT, EPI, NT_, S_, W_, false><<<grid, W_ * 64, 0, s>>>(ka);      \
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
    const dim3 grid(p.groups, p.mblocks, p.ksplit);
    wide_gemm_kernel<AT, WT, EPI><<<grid, kThreads, 0, s>>>(ka);
    return hipGetLastError();
}

// Skinny plan for a given tiling: groups of `nt` tiles, K chunks of
// waves * steps MFMA steps.
GemmPlan skinny_plan(int64_t N, int64_t K, Epi epi, int nt, int steps, int waves, bool alds = false) {
    GemmPlan p{};
    p.kernel = 0;
    p.alds = alds && waves * steps <= 32;
    p.nt = nt;
    p.steps = steps;
    p.waves = waves;
    const int64_t tiles = N / 16, ksteps = K / 32;
    p.groups = static_cast<int>(std::max<int64_t>(1, epi == Epi::GELU_MUL ? (tiles / 2) / (nt / 2) : (tiles + nt - 1) / nt));
    p.ksplit = static_cast<int>((ksteps + static_cast<int64_t>(waves) * steps - 1) / (static_cast<int64_t>(waves) * steps));
    p.mblocks = 1;
    p.ok = p.ksplit == 1 || p.groups <= kMaxCounters;
    return p;
}

}  // namespace

GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K, AType at, WType wt, Epi epi) {
    const int64_t ksteps = K / 32;
    const int64_t tiles = N / 16;
    if (M <= 64) {
        // One 16-column tile (a gate/up pair for the fused epilogue) per
        // workgroup and K chunks of at most 32 MFMA steps (1024 K), split
        // over workgroups only as far as needed to reach ~256 workgroups.
        // Tilings measured on MI355X at M = 50: FP8 weights 8 waves x 4
        // steps, BF16 weights 16 waves x 2 steps; bf16 activations staged
        // through LDS (1.2-1.4 us faster per call than fragment loads).
        const int nt = (epi == Epi::GELU_MUL) ? 2 : 1;
        const int64_t groups = std::max<int64_t>(1, (epi == Epi::GELU_MUL) ? tiles / 2 : tiles);
        const int64_t want_split = groups >= 256 ? 1 : (256 + groups - 1) / groups;
        const int64_t chunk = (ksteps + want_split - 1) / want_split;   // K steps per workgroup
        int steps, waves;
        if (wt == WType::BF16) {
            waves = 16;
            steps = chunk <= 16 ? 1 : 2;
        } else {
            waves = 8;
            steps = chunk <= 16 ? 2 : 4;
        }
        return skinny_plan(N, K, epi, nt, steps, waves, at == AType::BF16);
    }
    GemmPlan p{};
    p.kernel = 1;
    p.nt = 8;
    p.steps = 2;
    p.waves = 4;
    p.groups = static_cast<int>(std::max<int64_t>(1, epi == Epi::GELU_MUL ? (tiles / 2 + 3) / 4 : (tiles + 7) / 8));
    p.mblocks = static_cast<int>((M + kBM - 1) / kBM);
    const int64_t base = static_cast<int64_t>(p.groups) * p.mblocks;
    const int64_t kt_total = (ksteps + 1) / 2;
    int ks = 1;
    while (base * ks < 256 && ks * 2 <= kt_total / 8) ks *= 2;
    p.ksplit = ks;
    p.ok = p.ksplit == 1 || base <= kMaxCounters;
    return p;
}

size_t gemm_ws_bytes(const GemmPlan& p, int64_t M, int64_t N) {
    (void)N;
    if (p.ksplit <= 1) return kCounterBytes;
    size_t part;
    if (p.kernel == 0)
        part = static_cast<size_t>(p.ksplit) * p.groups * p.nt * 4 * 64 * 16;
    else
        part = static_cast<size_t>(p.ksplit) * p.mblocks * p.groups * kThreads * 16 * 16;
    return kCounterBytes + part;
}

hipError_t launch_gemm_plan(const GemmProblem& pr, const GemmPlan& p, hipStream_t s) {
    KArgs ka{};
    ka.A = pr.A; ka.s_a = pr.s_a; ka.W = pr.W; ka.s_w = pr.s_w;
    ka.bias = pr.bias; ka.resid = pr.resid; ka.Y = pr.Y; ka.gu = pr.gu;
    ka.M = static_cast<int>(pr.M); ka.N = static_cast<int>(pr.N); ka.K = static_cast<int>(pr.K);
    ka.ksplit = p.ksplit;
    ka.groups = p.groups;
    ka.tickets = static_cast<uint32_t*>(pr.ws);
    ka.part = reinterpret_cast<float*>(static_cast<uint8_t*>(pr.ws) + kCounterBytes);
    ka.part_bytes = static_cast<uint32_t>(gemm_ws_bytes(p, pr.M, pr.N) - kCounterBytes);

    if (pr.epi == Epi::GELU_MUL) return launch_typed<AType::BF16, WType::FP8, Epi::GELU_MUL>(ka, p, s);
    if (pr.wtype == WType::BF16) return launch_typed<AType::BF16, WType::BF16, Epi::PLAIN>(ka, p, s);
    if (pr.atype == AType::FP8) return launch_typed<AType::FP8, WType::FP8, Epi::PLAIN>(ka, p, s);
    return launch_typed<AType::BF16, WType::FP8, Epi::PLAIN>(ka, p, s);
}

hipError_t launch_gemm(const GemmProblem& pr, hipStream_t s) {
    return launch_gemm_plan(pr, plan_gemm(pr.M, pr.N, pr.K, pr.atype, pr.wtype, pr.epi), s);
}

}  // namespace vla
