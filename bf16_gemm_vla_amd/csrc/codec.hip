// Weight/activation codecs on gfx950: per-output-channel quantize + MFMA
// lane pack, FP8 byte pack, FNUZ -> OCP re-encode, per-tensor activation
// quantization.  These run once at load time (weights) or once per call
// (activations of the FP8 x FP8 GEMM) and are HBM-bound byte streams.
//
// Every fp32 operation here is a single IEEE operation (division is the
// correctly rounded __fdiv_rn; no contraction), so results match the
// reference quantizer bit for bit.
#pragma clang fp contract(off)

#include <algorithm>

#include "vla_device.h"
#include "vla_internal.h"

namespace vla {
namespace {

constexpr int kThreads = 256;

// Offset (in elements) of the 8-value slot `slot` of 16-row tile n0 in the
// given layout.  slot = k0 * 64 + lane, lane = 16 k1 + n1.
__device__ __forceinline__ int64_t slot_offset(int layout, int64_t n0, int64_t slot, int64_t K) {
    const int64_t k0 = slot >> 6, lane = slot & 63, k1 = lane >> 4, n1 = lane & 15;
    if (layout == 1) return (n0 * (K >> 5) * 64 + slot) * 8;          // MFMA layout
    return (n0 * 16 + n1) * K + k0 * 32 + k1 * 8;                     // row-major
}

// Codes of fp32(v / sc) for eight fp32 values, the quotient correctly
// rounded as IEEE division gives it, with rcp = RN(1 / sc): q = RN(v * rcp)
// is within 2 ulps of RN(v / sc), and the code only changes at midpoints
// between E4M3 values (fraction bits 19..0 == 0x80000 in the normal range),
// so unless q lies within 3 ulps of a midpoint, below the smallest normal
// value (but not zero) or is not finite, the code of q is the code of the
// exact quotient.  Those codes come from the hardware conversion (nearest
// even, signed zero kept), two per instruction, of q clamped to the largest
// finite value the conversion gets right, since the encoder saturates:
//   OCP:  |q| clamped to 448 (code 0x7E);
//   FNUZ: 2 min(|q|, 224) + 0 converted as OCP (an FNUZ byte decodes to half
//         the OCP value; + 0 turns -0 into +0, FNUZ having no -0), and the
//         low bit set above 232, the midpoint to 240 (0x7F = 0x7E | 1).
template <bool FNUZ>
__device__ __forceinline__ bool needs_exact(float q) {
    constexpr float lo = FNUZ ? 0x1p-7f : 0x1p-6f;              // smallest normal
    const bool below_normal = __builtin_fabsf(q) < lo && q != 0.0f;
    const bool not_finite = !(__builtin_fabsf(q) < __builtin_inff());
    // fraction bits 19..0 within [0x80000 - 3, 0x80000 + 3]: shifted to the
    // top of the word, the window is one unsigned compare
    const bool near_mid = (__float_as_uint(q) << 12) - (0x7FFFDu << 12) <= (6u << 12);
    return below_normal || not_finite || near_mid;
}

template <bool FNUZ>
__device__ __forceinline__ uint2 encode8_fast(const float q[8]) {
    constexpr float top = FNUZ ? 224.0f : 448.0f;
    uint32_t o[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        float c4[4];
        uint32_t hi_bit = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float qc = __builtin_amdgcn_fmed3f(q[4 * h + j], -top, top);
            c4[j] = FNUZ ? __builtin_fmaf(qc, 2.0f, 0.0f) : qc;
            if (FNUZ) hi_bit |= (__builtin_fabsf(q[4 * h + j]) > 232.0f ? 1u : 0u) << (8 * j);
        }
        int c = __builtin_amdgcn_cvt_pk_fp8_f32(c4[0], c4[1], 0, false);
        c = __builtin_amdgcn_cvt_pk_fp8_f32(c4[2], c4[3], c, true);
        o[h] = static_cast<uint32_t>(c) | hi_bit;
    }
    return make_uint2(o[0], o[1]);
}

// All eight codes: the hardware ones, the elements that need it re-encoded
// from the exact quotient in a branch.  Whether any of the eight needs it
// is decided from three running extremes of the bit patterns (one min/max
// per element each) rather than per-element flags: with a = |q| bits,
// 0 < |q| < smallest normal  <=>  min(a - 1) < lo - 1 (a = 0 wraps to the
// top), near a midpoint  <=>  min((u << 12) - (0x7FFFD << 12)) <= 6 << 12,
// not finite  <=>  max(a) >= 0x7F800000 — the same tests as needs_exact.
template <bool FNUZ>
__device__ __forceinline__ uint2 encode8_quotient(const float v[8], float sc, float rcp) {
    constexpr uint32_t lo = FNUZ ? 0x3C000000u : 0x3C800000u;   // 2^-7 / 2^-6
    float q[8];
    uint32_t wmin = 0xFFFFFFFFu, tmin = 0xFFFFFFFFu, amax = 0u;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        q[j] = v[j] * rcp;
        const uint32_t u = __float_as_uint(q[j]), a = u & 0x7FFFFFFFu;
        wmin = min(wmin, a - 1u);
        tmin = min(tmin, (u << 12) - (0x7FFFDu << 12));
        amax = max(amax, a);
    }
    const bool any = wmin < lo - 1u || tmin <= (6u << 12) || amax >= 0x7F800000u;
    const uint2 f = encode8_fast<FNUZ>(q);
    uint32_t o[2] = {f.x, f.y};
    if (__builtin_expect(any, 0)) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            // recomputed here: an opaque copy keeps the compiler from carrying
            // the eight flags across the branch in registers
            float qj = q[j];
            asm volatile("" : "+v"(qj));
            if (needs_exact<FNUZ>(qj)) {
                const uint32_t code = encode_e4m3<FNUZ>(__fdiv_rn(v[j], sc));
                o[j >> 2] = (o[j >> 2] & ~(0xFFu << (8 * (j & 3)))) | (code << (8 * (j & 3)));
            }
        }
    }
    return make_uint2(o[0], o[1]);
}

// One workgroup of NT threads per 16-row tile (any K; the second read of
// the tile mostly hits L2).  Phase 1: row absmax -> scale.  Phase 2: each
// thread encodes 8-value slots (reads 2 x 16 B, writes 8 B / 16 B).  NT =
// 1024 keeps 16 waves' loads in flight per tile: a 2048 x 16384 matrix has
// only 128 tiles.
template <int WFMT, int NT>
__global__ __launch_bounds__(NT) void quantize_pack_kernel(const float* __restrict__ W,
                                                           void* __restrict__ Wq,
                                                           float* __restrict__ scales,
                                                           int64_t K, int layout) {
    constexpr int TPR = NT / 16;                 // threads per row in phase 1
    __shared__ float s_scale[16];
    const int64_t n0 = blockIdx.x;
    const int t = threadIdx.x;
    const float* tile = W + n0 * 16 * K;

    if (WFMT != VLA_WFMT_BF16) {
        // TPR threads per row, float4 loads strided by 4 TPR floats
        const int r = t / TPR, c = t % TPR;
        const float* row = tile + static_cast<int64_t>(r) * K;
        float m = 0.0f;
#pragma unroll 4
        for (int64_t k = 4 * c; k < K; k += 4 * TPR) {
            float4 v = *reinterpret_cast<const float4*>(row + k);
            m = fmaxf(m, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
        }
        m = group_max<TPR>(m);
        if (c == 0) {
            const float maxv = (WFMT == VLA_WFMT_E4M3_FNUZ) ? 240.0f : 448.0f;
            const float sc = (m == 0.0f) ? 1.0f : __fdiv_rn(m, maxv);
            s_scale[r] = sc;
            scales[n0 * 16 + r] = sc;
        }
        __syncthreads();
    }

    const int64_t nslots = (K >> 5) * 64;
    // slot % 64 = t % 64: the thread's row n1 and its scale stay fixed
    const float sc = (WFMT == VLA_WFMT_BF16) ? 1.0f : s_scale[t & 15];
    const float rcp = __fdiv_rn(1.0f, sc);
    for (int64_t slot = t; slot < nslots; slot += NT) {
        const int64_t k0 = slot >> 6;
        const int lane = static_cast<int>(slot & 63), k1 = lane >> 4, n1 = lane & 15;
        const float* src = tile + static_cast<int64_t>(n1) * K + k0 * 32 + k1 * 8;
        const float4 a = *reinterpret_cast<const float4*>(src);
        const float4 b = *reinterpret_cast<const float4*>(src + 4);
        const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
        const int64_t off = slot_offset(layout, n0, slot, K);
        if (WFMT == VLA_WFMT_BF16) {
            uint32_t w[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                w[i] = f32x2_to_bf16x2(v[2 * i], v[2 * i + 1]);
            *reinterpret_cast<uint4*>(static_cast<uint16_t*>(Wq) + off) =
                make_uint4(w[0], w[1], w[2], w[3]);
        } else {
            *reinterpret_cast<uint2*>(static_cast<uint8_t*>(Wq) + off) =
                encode8_quotient<WFMT == VLA_WFMT_E4M3_FNUZ>(v, sc, rcp);
        }
    }
}

// MXFP4 (OCP Microscaling Formats v1.0): nearest E2M1 code of |v|, ties to
// the even code (mantissa bit 0), |v| >= 6 saturating; the sign bit is
// taken from v (so -0 stays 0x8).  Magnitudes: 0, .5, 1, 1.5, 2, 3, 4, 6.
__device__ __forceinline__ uint32_t encode_e2m1(float v) {
    const float a = fabsf(v);
    uint32_t c;
    if (a <= 0.25f) c = 0;
    else if (a < 0.75f) c = 1;
    else if (a <= 1.25f) c = 2;
    else if (a < 1.75f) c = 3;
    else if (a <= 2.5f) c = 4;
    else if (a < 3.5f) c = 5;
    else if (a <= 5.0f) c = 6;
    else c = 7;
    return c | ((__float_as_uint(v) >> 28) & 8u);
}

// MXFP4 quantize + pack, one workgroup per 16-row tile, one thread per
// 32-value block (one output channel x one 32-wide K step, which is exactly
// one packed MFMA fragment row).  Shared exponent floor(log2 max|w|) - 2,
// clamped to E8M0's range (an all-zero block takes 0); codes of w * 2^-e
// (exact: a power-of-two scale).  Codes go two per byte (even position in
// the low nibble) in the FP8 fragment order; the E8M0 scale bytes follow all
// codes, row-major with rows padded to P = K/32 rounded up to 8 bytes (pad
// bytes 127): byte N*K/2 + n * P + k0, so a wave's consecutive K steps of one
// row are one aligned load.  Blocks are independent, so a tile's blocks are
// shared among gridDim.y workgroups (enough workgroups for few, long rows).
__global__ __launch_bounds__(kThreads) void mxfp4_quantize_pack_kernel(const float* __restrict__ W,
                                                                       uint8_t* __restrict__ Wq, int64_t N,
                                                                       int64_t K) {
    const int64_t n0 = blockIdx.x;
    const int64_t ksteps = K >> 5;
    const int64_t P = mxfp4_scale_row_bytes(K);
    uint8_t* const sc_base = Wq + N * K / 2;
    for (int64_t b = blockIdx.y * static_cast<int64_t>(kThreads) + threadIdx.x; b < P * 16;
         b += static_cast<int64_t>(gridDim.y) * kThreads) {
        const int64_t k0 = b >> 4;
        const int n1 = static_cast<int>(b & 15);
        if (k0 >= ksteps) {   // row padding
            sc_base[(n0 * 16 + n1) * P + k0] = 127;
            continue;
        }
        const float* src = W + (n0 * 16 + n1) * K + k0 * 32;
        float v[32];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float4 f = *reinterpret_cast<const float4*>(src + 4 * i);
            v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
        }
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < 32; ++i) m = fmaxf(m, fabsf(v[i]));
        // floor(log2 m) from the exponent field; a subnormal m clamps to -127
        const int ebits = static_cast<int>((__float_as_uint(m) >> 23) & 0xFFu);
        const int se = (m == 0.0f) ? 0 : (ebits == 0 ? -127 : max(-127, ebits - 127 - 2));
        const float inv = __uint_as_float(static_cast<uint32_t>(127 - se) << 23);   // 2^-se, a normal float
#pragma unroll
        for (int k1 = 0; k1 < 4; ++k1) {
            uint32_t w = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) w |= encode_e2m1(v[8 * k1 + i] * inv) << (4 * i);
            const int64_t slot = (n0 * ksteps + k0) * 64 + 16 * k1 + n1;
            *reinterpret_cast<uint32_t*>(Wq + slot * 4) = w;
        }
        sc_base[(n0 * 16 + n1) * P + k0] = static_cast<uint8_t>(127 + se);
    }
}

// Register-resident FP8 quantize + pack of one 16-row tile by NT threads
// (the tile's 2K slots of 8 values, SPT = 2K / NT per thread): thread t owns
// slots t + NT i, which all belong to row t % 16 of the tile (slot % 16 is
// the row), so the weights are read from HBM once: every load is issued up
// front, the row maxima are reduced over the threads of each row (lanes
// l ^ 16, l ^ 32 in a wave, then the waves through LDS), and the codes are
// encoded from registers with the same encoder (encode8_quotient) as
// quantize_pack_kernel.  NT = 1024 keeps a thread's share at K / 64 values,
// so two tiles fit on a compute unit at K = 2048 and the grid drains in
// whole rounds.
template <int WFMT, int SPT, int NT>
__global__ __launch_bounds__(NT) void quantize_pack_reg_kernel(const float* __restrict__ W,
                                                               uint8_t* __restrict__ Wq,
                                                               float* __restrict__ scales, int64_t K,
                                                               int layout) {
    constexpr int NW = NT / kWave;
    __shared__ float red[NW][16];
    const int64_t n0 = blockIdx.x;
    const int t = threadIdx.x, n1 = t & 15, k1 = (t & 63) >> 4;
    const float* row = W + (n0 * 16 + n1) * K;
    float4 a[SPT], b[SPT];
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
        const int64_t k0 = (t >> 6) + NW * i;      // slot t + NT i: k0 = slot / 64
        const float* src = row + k0 * 32 + k1 * 8;
        a[i] = *reinterpret_cast<const float4*>(src);
        b[i] = *reinterpret_cast<const float4*>(src + 4);
    }
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < SPT; ++i)
        m = fmaxf(m, fmaxf(fmaxf(fmaxf(fabsf(a[i].x), fabsf(a[i].y)), fmaxf(fabsf(a[i].z), fabsf(a[i].w))),
                           fmaxf(fmaxf(fabsf(b[i].x), fabsf(b[i].y)), fmaxf(fabsf(b[i].z), fabsf(b[i].w)))));
    m = fmaxf(m, __shfl_xor(m, 16, kWave));
    m = fmaxf(m, __shfl_xor(m, 32, kWave));
    if ((t & 63) < 16) red[t >> 6][n1] = m;
    __syncthreads();
    float rm = red[0][n1];
#pragma unroll
    for (int w = 1; w < NW; ++w) rm = fmaxf(rm, red[w][n1]);
    const float maxv = (WFMT == VLA_WFMT_E4M3_FNUZ) ? 240.0f : 448.0f;
    const float sc = (rm == 0.0f) ? 1.0f : __fdiv_rn(rm, maxv);
    if (t < 16) scales[n0 * 16 + t] = sc;
    const float rcp = __fdiv_rn(1.0f, sc);
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
        const float v[8] = {a[i].x, a[i].y, a[i].z, a[i].w, b[i].x, b[i].y, b[i].z, b[i].w};
        *reinterpret_cast<uint2*>(Wq + slot_offset(layout, n0, t + NT * i, K)) =
            encode8_quotient<WFMT == VLA_WFMT_E4M3_FNUZ>(v, sc, rcp);
    }
}

// The same for the row-major layout with K a multiple of 512: wave w owns
// rows RPW w .. RPW w + RPW - 1 of the tile (RPW = 16 / waves), lane l the 8
// values at k = 512 c + 8 l of each, so every load and store of a wave is
// one contiguous run of the row (2 KiB of fp32 in, 512 bytes of codes out)
// and the row maxima are wave reductions.
template <int WFMT, int SPT, int NT>
__global__ __launch_bounds__(NT) void quantize_rows_reg_kernel(const float* __restrict__ W,
                                                               uint8_t* __restrict__ Wq,
                                                               float* __restrict__ scales, int64_t K) {
    constexpr int RPW = 16 / (NT / kWave);           // rows per wave
    constexpr int CPR = SPT / RPW;                   // 512-value chunks per row
    static_assert(SPT % RPW == 0, "K a multiple of 512");
    const int64_t n0 = blockIdx.x;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    float4 a[SPT], b[SPT];
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
        const int r = wave * RPW + i / CPR, c = i % CPR;
        const float* src = W + (n0 * 16 + r) * K + c * 512 + lane * 8;
        a[i] = *reinterpret_cast<const float4*>(src);
        b[i] = *reinterpret_cast<const float4*>(src + 4);
    }
    float sc[RPW];
#pragma unroll
    for (int q = 0; q < RPW; ++q) {
        float m = 0.0f;
#pragma unroll
        for (int c = 0; c < CPR; ++c) {
            const int i = q * CPR + c;
            m = fmaxf(m, fmaxf(fmaxf(fmaxf(fabsf(a[i].x), fabsf(a[i].y)), fmaxf(fabsf(a[i].z), fabsf(a[i].w))),
                               fmaxf(fmaxf(fabsf(b[i].x), fabsf(b[i].y)), fmaxf(fabsf(b[i].z), fabsf(b[i].w)))));
        }
        m = wave_max(m);
        const float maxv = (WFMT == VLA_WFMT_E4M3_FNUZ) ? 240.0f : 448.0f;
        sc[q] = (m == 0.0f) ? 1.0f : __fdiv_rn(m, maxv);
        if (lane == 0) scales[n0 * 16 + wave * RPW + q] = sc[q];
    }
    float rcp[RPW];
#pragma unroll
    for (int q = 0; q < RPW; ++q) rcp[q] = __fdiv_rn(1.0f, sc[q]);
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
        const int r = wave * RPW + i / CPR, c = i % CPR;
        const float v[8] = {a[i].x, a[i].y, a[i].z, a[i].w, b[i].x, b[i].y, b[i].z, b[i].w};
        *reinterpret_cast<uint2*>(Wq + (n0 * 16 + r) * K + c * 512 + lane * 8) =
            encode8_quotient<WFMT == VLA_WFMT_E4M3_FNUZ>(v, sc[i / CPR], rcp[i / CPR]);
    }
}

// The row mapping of quantize_rows_reg_kernel (one row per wave, 1024
// threads, K a multiple of 512 up to 4096) for the MFMA layout: each lane's
// 8 codes (row r, k = 512 c + 8 l) are one slot (k0 = k / 32, k1 = l % 4,
// n1 = r), placed in LDS in the tile's packed order with the row index
// XOR-ed by k0 % 16 (without it the 16 k0 slots a wave writes fall in two
// banks), and the tile then leaves as one contiguous block, each lane
// reading a 16-byte slot pair (n1 even, odd) and swapping its halves when
// the XOR reversed them.  Reads of the weights are contiguous runs of a row
// instead of 16 rows x 32 bytes per wave.
template <int WFMT, int SPT>
__global__ __launch_bounds__(1024) void quantize_rows_packed_kernel(const float* __restrict__ W,
                                                                    uint8_t* __restrict__ Wq,
                                                                    float* __restrict__ scales, int64_t K) {
    extern __shared__ __attribute__((aligned(16))) uint8_t ptile[];   // 16 K bytes
    const int64_t n0 = blockIdx.x;
    const int t = threadIdx.x, lane = t & 63, r = t >> 6;
    const float* row = W + (n0 * 16 + r) * K;
    float4 a[SPT], b[SPT];
#pragma unroll
    for (int c = 0; c < SPT; ++c) {
        a[c] = *reinterpret_cast<const float4*>(row + c * 512 + lane * 8);
        b[c] = *reinterpret_cast<const float4*>(row + c * 512 + lane * 8 + 4);
    }
    float m = 0.0f;
#pragma unroll
    for (int c = 0; c < SPT; ++c)
        m = fmaxf(m, fmaxf(fmaxf(fmaxf(fabsf(a[c].x), fabsf(a[c].y)), fmaxf(fabsf(a[c].z), fabsf(a[c].w))),
                           fmaxf(fmaxf(fabsf(b[c].x), fabsf(b[c].y)), fmaxf(fabsf(b[c].z), fabsf(b[c].w)))));
    m = wave_max(m);
    const float maxv = (WFMT == VLA_WFMT_E4M3_FNUZ) ? 240.0f : 448.0f;
    const float sc = (m == 0.0f) ? 1.0f : __fdiv_rn(m, maxv);
    if (lane == 0) scales[n0 * 16 + r] = sc;
    const float rcp = __fdiv_rn(1.0f, sc);
#pragma unroll
    for (int c = 0; c < SPT; ++c) {
        const float v[8] = {a[c].x, a[c].y, a[c].z, a[c].w, b[c].x, b[c].y, b[c].z, b[c].w};
        const int k0 = 16 * c + (lane >> 2), k1 = lane & 3;
        *reinterpret_cast<uint2*>(ptile + (k0 * 64 + 16 * k1 + (r ^ (k0 & 15))) * 8) =
            encode8_quotient<WFMT == VLA_WFMT_E4M3_FNUZ>(v, sc, rcp);
    }
    __syncthreads();
    uint8_t* dst = Wq + n0 * 16 * K;
    for (int x = t; x < K; x += 1024) {            // 16-byte output chunk x = slots 2x, 2x + 1
        const int slot = 2 * x, k0 = slot >> 6, k1 = (slot >> 4) & 3, n1 = slot & 15, sw = k0 & 15;
        uint4 v = *reinterpret_cast<const uint4*>(ptile + (k0 * 64 + 16 * k1 + ((n1 ^ sw) & ~1)) * 8);
        if (sw & 1) v = make_uint4(v.z, v.w, v.x, v.y);
        *reinterpret_cast<uint4*>(dst + static_cast<int64_t>(x) * 16) = v;
    }
}

// Row-major FP8 -> MFMA layout through LDS, one workgroup per 16-row tile
// (K <= 8192: the tile's 16 K bytes fit in LDS): 16-byte chunks are read
// with the row fastest across lanes (a wave covers 64 bytes of each of the
// 16 rows), each chunk's two 8-byte slots are written to their place in the
// tile's packed order in LDS (the 16 rows' slots of one K group are 128
// contiguous bytes, so these writes do not collide in banks), and the tile
// then leaves as one contiguous block.
// The tile occupies the same bytes in both layouts and every byte of it is
// read before any is written.
constexpr int kPackMaxK = 8192;

__global__ __launch_bounds__(kThreads) void pack_fp8_tile_kernel(const uint8_t* __restrict__ q,
                                                                 uint8_t* __restrict__ qp, int64_t K) {
    extern __shared__ __attribute__((aligned(16))) uint8_t tile[];   // 16 K bytes
    const int64_t n0 = blockIdx.x;
    const uint8_t* src = q + n0 * 16 * K;
    const int cpr = static_cast<int>(K >> 4);        // 16-byte chunks per row
    const int chunks = 16 * cpr;
    for (int c = threadIdx.x; c < chunks; c += kThreads) {
        const int n1 = c & 15, j = c >> 4;          // row, chunk along the row (k = 16 j ..)
        const uint4 v = *reinterpret_cast<const uint4*>(src + static_cast<int64_t>(n1) * K + j * 16);
        const int k0 = j >> 1, k1 = (j & 1) * 2;    // slots (k0, k1, n1) and (k0, k1 + 1, n1)
        const int o = ((k0 * 64 + 16 * k1 + n1) * 8);
        *reinterpret_cast<uint2*>(tile + o) = make_uint2(v.x, v.y);
        *reinterpret_cast<uint2*>(tile + o + 128) = make_uint2(v.z, v.w);
    }
    __syncthreads();
    uint8_t* dst = qp + n0 * 16 * K;
    for (int c = threadIdx.x; c < chunks; c += kThreads)
        *reinterpret_cast<uint4*>(dst + c * 16) = *reinterpret_cast<const uint4*>(tile + c * 16);
}

// Row-major FP8 -> MFMA layout: one thread per 8-byte slot (K > 8192).
__global__ __launch_bounds__(kThreads) void pack_fp8_kernel(const uint8_t* __restrict__ q,
                                                            uint8_t* __restrict__ qp, int64_t N,
                                                            int64_t K) {
    const int64_t total = N * K / 8;
    for (int64_t i = blockIdx.x * static_cast<int64_t>(kThreads) + threadIdx.x; i < total;
         i += static_cast<int64_t>(gridDim.x) * kThreads) {
        const int64_t per_tile = (K >> 5) * 64;
        const int64_t n0 = i / per_tile, slot = i % per_tile;
        const uint2 v = *reinterpret_cast<const uint2*>(q + slot_offset(0, n0, slot, K));
        *reinterpret_cast<uint2*>(qp + i * 8) = v;
    }
}

// FNUZ -> OCP, one workgroup per 16-row tile.  The tile's per-row flag
// "contains a +-240 code" picks j; the byte map for each j is built once
// per workgroup in LDS from the bit-level decoder/encoder.  Every byte is
// read in phase 1 before any is written in phase 2 by the same thread, so
// in-place use is safe.
__global__ __launch_bounds__(kThreads) void reencode_kernel(const uint8_t* q, const float* sc,
                                                            uint8_t* q2, float* sc2, int64_t K,
                                                            int layout) {
    __shared__ uint8_t lut[2][256];
    __shared__ int has240[16];
    const int64_t n0 = blockIdx.x;
    const int t = threadIdx.x;
    if (t < 16) has240[t] = 0;
    {
        // lut[j][b] = encode_ocp(2^j * decode_fnuz(b)); FNUZ NaN -> 0x7F
        const uint32_t b = static_cast<uint32_t>(t);
        if (b == 0x80u) {
            lut[0][b] = 0x7F;
            lut[1][b] = 0x7F;
        } else {
            const float v = decode_e4m3<true>(b);
            lut[0][b] = encode_e4m3<false>(v);
            lut[1][b] = encode_e4m3<false>(v * 2.0f);
        }
    }
    __syncthreads();
    const int64_t nslots = (K >> 5) * 64;
    for (int64_t slot = t; slot < nslots; slot += kThreads) {
        const int n1 = static_cast<int>(slot & 15);
        const uint2 v = *reinterpret_cast<const uint2*>(q + slot_offset(layout, n0, slot, K));
        bool hit = false;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t byte = ((i < 4 ? v.x : v.y) >> (8 * (i & 3))) & 0x7Fu;
            hit |= byte == 0x7Fu;
        }
        if (hit) atomicOr(&has240[n1], 1);
    }
    __syncthreads();
    for (int64_t slot = t; slot < nslots; slot += kThreads) {
        const int n1 = static_cast<int>(slot & 15);
        const int j = has240[n1] ? 0 : 1;
        const int64_t off = slot_offset(layout, n0, slot, K);
        const uint2 v = *reinterpret_cast<const uint2*>(q + off);
        uint32_t w[2] = {0, 0};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t byte = ((i < 4 ? v.x : v.y) >> (8 * (i & 3))) & 0xFFu;
            w[i >> 2] |= static_cast<uint32_t>(lut[j][byte]) << (8 * (i & 3));
        }
        *reinterpret_cast<uint2*>(q2 + off) = make_uint2(w[0], w[1]);
    }
    if (t < 16) sc2[n0 * 16 + t] = has240[t] ? sc[n0 * 16 + t] : sc[n0 * 16 + t] * 0.5f;
}

// Register-resident FNUZ -> OCP for K a multiple of 128 up to 2048: the same
// slot ownership as quantize_pack_reg_kernel, so every byte is read once
// (all reads precede any write of the tile, so in-place use stays safe) and
// the per-row "+-240 present" flag is an OR over the row's 16 threads.
template <int SPT>
__global__ __launch_bounds__(kThreads) void reencode_reg_kernel(const uint8_t* q, const float* sc, uint8_t* q2,
                                                                float* sc2, int64_t K, int layout) {
    __shared__ uint8_t lut[2][256];
    __shared__ int hitw[kThreads / kWave][16];
    const int64_t n0 = blockIdx.x;
    const int t = threadIdx.x, n1 = t & 15;
    uint2 v[SPT];
#pragma unroll
    for (int i = 0; i < SPT; ++i) v[i] = *reinterpret_cast<const uint2*>(q + slot_offset(layout, n0, t + kThreads * i, K));
    {
        // lut[j][b] = encode_ocp(2^j * decode_fnuz(b)); FNUZ NaN -> 0x7F
        const uint32_t b = static_cast<uint32_t>(t);
        if (b == 0x80u) {
            lut[0][b] = 0x7F;
            lut[1][b] = 0x7F;
        } else {
            const float x = decode_e4m3<true>(b);
            lut[0][b] = encode_e4m3<false>(x);
            lut[1][b] = encode_e4m3<false>(x * 2.0f);
        }
    }
    int hit = 0;
#pragma unroll
    for (int i = 0; i < SPT; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) hit |= ((((e < 4 ? v[i].x : v[i].y) >> (8 * (e & 3))) & 0x7Fu) == 0x7Fu) ? 1 : 0;
    hit |= __shfl_xor(hit, 16, kWave);
    hit |= __shfl_xor(hit, 32, kWave);
    if ((t & 63) < 16) hitw[t >> 6][n1] = hit;
    __syncthreads();
    int h = 0;
#pragma unroll
    for (int w = 0; w < kThreads / kWave; ++w) h |= hitw[w][n1];
    const int j = h ? 0 : 1;
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
        uint32_t w[2] = {0, 0};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t byte = ((e < 4 ? v[i].x : v[i].y) >> (8 * (e & 3))) & 0xFFu;
            w[e >> 2] |= static_cast<uint32_t>(lut[j][byte]) << (8 * (e & 3));
        }
        *reinterpret_cast<uint2*>(q2 + slot_offset(layout, n0, t + kThreads * i, K)) = make_uint2(w[0], w[1]);
    }
    if (t < 16) sc2[n0 * 16 + t] = h ? sc[n0 * 16 + t] : sc[n0 * 16 + t] * 0.5f;
}

// Row-major FNUZ -> OCP with K a multiple of 512: the row mapping of
// quantize_rows_reg_kernel (contiguous 512-byte runs per wave, the +-240
// flag of a row is a wave ballot).  All reads precede the writes.
template <int SPT>
__global__ __launch_bounds__(kThreads) void reencode_rows_reg_kernel(const uint8_t* q, const float* sc, uint8_t* q2,
                                                                     float* sc2, int64_t K) {
    constexpr int RPW = 16 / (kThreads / kWave);
    constexpr int CPR = SPT / RPW;
    static_assert(SPT % RPW == 0, "K a multiple of 512");
    __shared__ uint8_t lut[2][256];
    const int64_t n0 = blockIdx.x;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    uint2 v[SPT];
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
        const int r = wave * RPW + i / CPR, c = i % CPR;
        v[i] = *reinterpret_cast<const uint2*>(q + (n0 * 16 + r) * K + c * 512 + lane * 8);
    }
    // lane q < RPW carries the scale of the wave's row q
    const float s_my = (lane < RPW) ? sc[n0 * 16 + wave * RPW + lane] : 0.0f;
    {
        const uint32_t b = static_cast<uint32_t>(t);
        if (b == 0x80u) {
            lut[0][b] = 0x7F;
            lut[1][b] = 0x7F;
        } else {
            const float x = decode_e4m3<true>(b);
            lut[0][b] = encode_e4m3<false>(x);
            lut[1][b] = encode_e4m3<false>(x * 2.0f);
        }
    }
    int jr[RPW];
#pragma unroll
    for (int qr = 0; qr < RPW; ++qr) {
        bool hit = false;
#pragma unroll
        for (int c = 0; c < CPR; ++c)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                hit |= (((e < 4 ? v[qr * CPR + c].x : v[qr * CPR + c].y) >> (8 * (e & 3))) & 0x7Fu) == 0x7Fu;
        jr[qr] = __ballot(hit) ? 0 : 1;
    }
    __syncthreads();   // the byte maps are built
#pragma unroll
    for (int i = 0; i < SPT; ++i) {
        const int r = wave * RPW + i / CPR, c = i % CPR;
        const int j = jr[i / CPR];
        uint32_t w[2] = {0, 0};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t byte = ((e < 4 ? v[i].x : v[i].y) >> (8 * (e & 3))) & 0xFFu;
            w[e >> 2] |= static_cast<uint32_t>(lut[j][byte]) << (8 * (e & 3));
        }
        *reinterpret_cast<uint2*>(q2 + (n0 * 16 + r) * K + c * 512 + lane * 8) = make_uint2(w[0], w[1]);
    }
    if (lane < RPW) {
        int jm = jr[0];
#pragma unroll
        for (int qr = 1; qr < RPW; ++qr)
            if (lane == qr) jm = jr[qr];
        sc2[n0 * 16 + wave * RPW + lane] = jm ? s_my * 0.5f : s_my;
    }
}

// Activation quantization, pass 1: per-block absmax of 8-element chunks.
constexpr int kActBlocks = 512;

// Every thread keeps kActUnroll 16-byte loads in flight at a time.
constexpr int kActUnroll = 4;

// Chunks c0 .. c0 + n - 1 of an array (bytes_per_chunk each) as a buffer
// resource: loads past the window read zero, so the absmax pass needs no
// per-lane range branch (a branch around a load makes the compiler wait for
// every load in flight before the code after it; branch-free, the pass's
// loads stay in flight together: 768 x 16384 dynamic quantization 12.7 ->
// 12.1 us on MI355X, same GPU call).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t chunk_window(const void* base, int64_t c0, int64_t n, int bytes_per_chunk) {
    const int64_t m = n < 0 ? 0 : n;
    return __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(static_cast<const uint8_t*>(base)) + c0 * bytes_per_chunk, 0,
        static_cast<int>(m * bytes_per_chunk), 0x00020000);
}

__global__ __launch_bounds__(kThreads) void act_absmax_kernel(const uint16_t* __restrict__ A,
                                                              float* __restrict__ partial,
                                                              int64_t chunks) {
    __shared__ float red[kThreads / kWave];
    float m = 0.0f;
    constexpr int64_t kSpan = static_cast<int64_t>(kThreads) * kActUnroll;   // chunks per block and step
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kSpan;
    for (int64_t w0 = blockIdx.x * kSpan; w0 < chunks; w0 += stride) {
        const __amdgpu_buffer_rsrc_t r = chunk_window(A, w0, chunks - w0 < kSpan ? chunks - w0 : kSpan, 16);
        u32x4_t v[kActUnroll];
#pragma unroll
        for (int u = 0; u < kActUnroll; ++u)
            v[u] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (u * kThreads + threadIdx.x) * 16, 0, 0));
#pragma unroll
        for (int u = 0; u < kActUnroll; ++u) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                m = fmaxf(m, fabsf(bf16_to_f32(static_cast<uint16_t>(v[u][j] & 0xFFFFu))));
                m = fmaxf(m, fabsf(bf16_to_f32(static_cast<uint16_t>(v[u][j] >> 16))));
            }
        }
    }
    m = wave_max(m);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        float r = red[0];
        for (int i = 1; i < kThreads / kWave; ++i) r = fmaxf(r, red[i]);
        partial[blockIdx.x] = r;
    }
}

// OCP E4M3 codes of fp32(x / sc) for the 8 bf16 values of one dword quad,
// by the reasoning of encode8_quotient (hardware codes of x * RN(1/sc)
// unless within 3 ulps of a midpoint, outside the normal range or not
// finite) with one flag and branch per element and the range top [448, inf)
// flagged too: a per-tensor scale puts only the absmax element there, and
// this form measured faster than encode8_quotient's on activations
// (768 x 16384: 13.6 -> 11.9 us), the reverse of the weights, where every
// row's maximum reaches the top.
__device__ __forceinline__ uint2 act_codes8(const uint32_t w[4], float sc, float rcp) {
    float x[8], q[8];
    bool slow[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        x[j] = __uint_as_float((j & 1) ? (w[j >> 1] & 0xFFFF0000u) : (w[j >> 1] << 16));
        q[j] = x[j] * rcp;
        const uint32_t a = __float_as_uint(q[j]) & 0x7FFFFFFFu;
        const bool out_of_range = (a - 0x3C800000u) >= (0x43E00000u - 0x3C800000u);   // not in [2^-6, 448)
        const bool near_mid = ((a & 0xFFFFFu) - (0x80000u - 3u)) <= 6u;
        slow[j] = (out_of_range && a != 0u) || near_mid;
    }
    uint32_t o[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        int v = __builtin_amdgcn_cvt_pk_fp8_f32(q[4 * h], q[4 * h + 1], 0, false);
        v = __builtin_amdgcn_cvt_pk_fp8_f32(q[4 * h + 2], q[4 * h + 3], v, true);
        o[h] = static_cast<uint32_t>(v);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        if (__builtin_expect(slow[j], 0)) {
            const uint32_t code = encode_e4m3<false>(__fdiv_rn(x[j], sc));
            o[j >> 2] = (o[j >> 2] & ~(0xFFu << (8 * (j & 3)))) | (code << (8 * (j & 3)));
        }
    }
    return make_uint2(o[0], o[1]);
}

// Pass 2 (and the frozen-scale path): every wave forms the scale itself —
// dynamic: the same reduction of the pass-1 maxima in the same order on
// every wave, so all agree bit for bit; STATIC: the given, calibrated scale
// — and no wave waits for another.  Then a grid-stride loop over groups of
// U 16-byte chunks per thread that issues the next group's loads before it
// encodes the current one, so loads, encoding and stores of different
// groups overlap.
template <bool STATIC, int U>
__global__ __launch_bounds__(kThreads) void act_encode_kernel(const uint16_t* __restrict__ A,
                                                              const float* __restrict__ partial,
                                                              uint8_t* __restrict__ qa,
                                                              float* __restrict__ s_a,
                                                              int64_t chunks) {
    float sc;
    if constexpr (STATIC) {
        sc = *s_a;
    } else {
        static_assert(kActBlocks % kWave == 0, "partials split evenly over one wave");
        const int lane = threadIdx.x & (kWave - 1);
        float p[kActBlocks / kWave];
#pragma unroll
        for (int i = 0; i < kActBlocks / kWave; ++i) p[i] = partial[lane + i * kWave];
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < kActBlocks / kWave; ++i) m = fmaxf(m, p[i]);
        m = wave_max(m);
        sc = (m == 0.0f) ? 1.0f : __fdiv_rn(m, 448.0f);
        if (blockIdx.x == 0 && threadIdx.x == 0) *s_a = sc;
    }
    const float rcp = __fdiv_rn(1.0f, sc);
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads * U;
    int64_t base = blockIdx.x * static_cast<int64_t>(kThreads) * U + threadIdx.x;
    auto load = [&](int64_t b0, uint4 (&v)[U]) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = b0 + u * kThreads;
            v[u] = i < chunks ? *reinterpret_cast<const uint4*>(A + i * 8) : make_uint4(0, 0, 0, 0);
        }
    };
    uint4 v[U];
    load(base, v);
    while (base < chunks) {
        uint4 nv[U];
        load(base + stride, nv);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + u * kThreads;
            if (i >= chunks) continue;
            const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
            *reinterpret_cast<uint2*>(qa + i * 8) = act_codes8(w, sc, rcp);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = nv[u];
        base += stride;
    }
}

}  // namespace

// K / 128 slots per thread, 1 .. 16 (K a multiple of 128, at most 2048).
#define VLA_SPT_CASES(X) X(1) X(2) X(3) X(4) X(5) X(6) X(7) X(8) X(9) X(10) X(11) X(12) X(13) X(14) X(15) X(16)

hipError_t launch_quantize_pack(const float* W, void* Wq, float* scales, int64_t N, int64_t K,
                                int wfmt, int layout, hipStream_t s) {
    const dim3 grid(static_cast<unsigned>(N / 16));
    // K a multiple of 512 up to 4096: 1024 threads per tile, one row per
    // wave, K / 512 slots per thread (the MFMA layout through LDS)
    if (wfmt != VLA_WFMT_BF16 && K % 512 == 0 && K <= 4096) {
        const int spt = static_cast<int>(K / 512);
        uint8_t* q = static_cast<uint8_t*>(Wq);
#define VLA_Q1K(SPT_)                                                                                  \
        if (spt == SPT_) {                                                                             \
            if (layout == 0 && wfmt == VLA_WFMT_E4M3_OCP)                                              \
                quantize_rows_reg_kernel<VLA_WFMT_E4M3_OCP, SPT_, 1024><<<grid, 1024, 0, s>>>(W, q, scales, K); \
            else if (layout == 0)                                                                      \
                quantize_rows_reg_kernel<VLA_WFMT_E4M3_FNUZ, SPT_, 1024><<<grid, 1024, 0, s>>>(W, q, scales, K); \
            else if (wfmt == VLA_WFMT_E4M3_OCP)                                                        \
                quantize_rows_packed_kernel<VLA_WFMT_E4M3_OCP, SPT_><<<grid, 1024, 16 * K, s>>>(W, q, scales, K); \
            else                                                                                       \
                quantize_rows_packed_kernel<VLA_WFMT_E4M3_FNUZ, SPT_><<<grid, 1024, 16 * K, s>>>(W, q, scales, K); \
            return hipGetLastError();                                                                  \
        }
        VLA_Q1K(1) VLA_Q1K(2) VLA_Q1K(3) VLA_Q1K(4) VLA_Q1K(5) VLA_Q1K(6) VLA_Q1K(7) VLA_Q1K(8)
#undef VLA_Q1K
    }
    // other K, multiples of 128 up to 2048: 256 threads, K / 128 slots each
    if (wfmt != VLA_WFMT_BF16 && K % 128 == 0 && K <= 2048) {
        const int spt = static_cast<int>(K / 128);
        uint8_t* q = static_cast<uint8_t*>(Wq);
#define VLA_QP(SPT_)                                                                                   \
        if (spt == SPT_) {                                                                             \
            if (wfmt == VLA_WFMT_E4M3_OCP)                                                             \
                quantize_pack_reg_kernel<VLA_WFMT_E4M3_OCP, SPT_, kThreads><<<grid, kThreads, 0, s>>>(W, q, scales, K, layout); \
            else                                                                                       \
                quantize_pack_reg_kernel<VLA_WFMT_E4M3_FNUZ, SPT_, kThreads><<<grid, kThreads, 0, s>>>(W, q, scales, K, layout); \
            return hipGetLastError();                                                                  \
        }
        VLA_QP(1) VLA_QP(2) VLA_QP(3) VLA_QP(5) VLA_QP(6) VLA_QP(7) VLA_QP(9) VLA_QP(10) VLA_QP(11) VLA_QP(13)
        VLA_QP(14) VLA_QP(15)
#undef VLA_QP
    }
    switch (wfmt) {
        case VLA_WFMT_BF16:
            quantize_pack_kernel<VLA_WFMT_BF16, 1024><<<grid, 1024, 0, s>>>(W, Wq, scales, K, layout);
            break;
        case VLA_WFMT_E4M3_OCP:
            quantize_pack_kernel<VLA_WFMT_E4M3_OCP, 1024><<<grid, 1024, 0, s>>>(W, Wq, scales, K, layout);
            break;
        default:
            quantize_pack_kernel<VLA_WFMT_E4M3_FNUZ, 1024><<<grid, 1024, 0, s>>>(W, Wq, scales, K, layout);
            break;
    }
    return hipGetLastError();
}

hipError_t launch_mxfp4_quantize_pack(const float* W, uint8_t* Wq, int64_t N, int64_t K, hipStream_t s) {
    // split each tile's 16 P blocks over enough workgroups for ~1024 in all
    const int64_t tiles = N / 16;
    const int64_t per_tile = (mxfp4_scale_row_bytes(K) * 16 + kThreads - 1) / kThreads;
    const int64_t ys = std::max<int64_t>(1, std::min<int64_t>(per_tile, (1024 + tiles - 1) / tiles));
    mxfp4_quantize_pack_kernel<<<dim3(static_cast<unsigned>(tiles), static_cast<unsigned>(ys)), kThreads, 0, s>>>(
        W, Wq, N, K);
    return hipGetLastError();
}

hipError_t launch_pack_fp8(const uint8_t* q, uint8_t* qp, int64_t N, int64_t K, hipStream_t s) {
    if (K <= kPackMaxK) {
        pack_fp8_tile_kernel<<<static_cast<unsigned>(N / 16), kThreads, static_cast<size_t>(16 * K), s>>>(q, qp, K);
        return hipGetLastError();
    }
    const int64_t total = N * K / 8;
    const int64_t blocks = (total + kThreads - 1) / kThreads;
    const unsigned grid = static_cast<unsigned>(blocks < 65536 ? blocks : 65536);
    pack_fp8_kernel<<<grid, kThreads, 0, s>>>(q, qp, N, K);
    return hipGetLastError();
}

hipError_t launch_reencode(const uint8_t* q, const float* sc, uint8_t* q2, float* sc2, int64_t N,
                           int64_t K, int layout, hipStream_t s) {
    if (layout == 0 && K % 512 == 0 && K <= 2048) {
        const int spt = static_cast<int>(K / 128);
#define VLA_RR(SPT_)                                                                                                    \
        if (spt == SPT_) {                                                                                              \
            reencode_rows_reg_kernel<SPT_><<<static_cast<unsigned>(N / 16), kThreads, 0, s>>>(q, sc, q2, sc2, K);      \
            return hipGetLastError();                                                                                   \
        }
        VLA_RR(4) VLA_RR(8) VLA_RR(12) VLA_RR(16)
#undef VLA_RR
    }
    if (K % 128 == 0 && K <= 2048) {
        const int spt = static_cast<int>(K / 128);
#define VLA_RE(SPT_)                                                                                                  \
        if (spt == SPT_) {                                                                                            \
            reencode_reg_kernel<SPT_><<<static_cast<unsigned>(N / 16), kThreads, 0, s>>>(q, sc, q2, sc2, K, layout); \
            return hipGetLastError();                                                                                 \
        }
        VLA_SPT_CASES(VLA_RE)
#undef VLA_RE
    }
    reencode_kernel<<<static_cast<unsigned>(N / 16), kThreads, 0, s>>>(q, sc, q2, sc2, K, layout);
    return hipGetLastError();
}

size_t quantize_act_ws_bytes(int64_t, int64_t) { return kActBlocks * sizeof(float); }

// Encoder grid: U chunks per thread per group (4 with a dynamic scale,
// whose every wave also reads the pass-1 maxima, 2 with a frozen one) when
// that still gives at least two workgroups per compute unit, else one; at
// most 2048 / 4096 workgroups (one group per thread up to 768 x 16384), the
// groups split evenly over them.  Measured on MI355X at 768 x 16384: one
// group per thread beat two pipelined ones (13.6 against 15.8 us, frozen
// scale), and two chunks per thread beat four (10.7 against 11.9 us).
template <bool STATIC>
hipError_t launch_act_encode(const uint16_t* A, const float* partial, uint8_t* qa, float* s_a, int64_t chunks,
                             hipStream_t s) {
    constexpr int U = STATIC ? 2 : 4;
    constexpr int64_t kMaxBlocks = STATIC ? 4096 : 2048;
    const int64_t needU = (chunks + U * kThreads - 1) / (U * kThreads);
    const bool grouped = needU >= 512;
    const int64_t need = grouped ? needU : (chunks + kThreads - 1) / kThreads;
    const int64_t iters = (need + kMaxBlocks - 1) / kMaxBlocks;
    const unsigned grid = static_cast<unsigned>(std::max<int64_t>(1, (need + iters - 1) / iters));
    if (grouped) act_encode_kernel<STATIC, U><<<grid, kThreads, 0, s>>>(A, partial, qa, s_a, chunks);
    else act_encode_kernel<STATIC, 1><<<grid, kThreads, 0, s>>>(A, partial, qa, s_a, chunks);
    return hipGetLastError();
}

hipError_t launch_quantize_act(const uint16_t* A, uint8_t* qa, float* s_a, void* ws, int64_t M,
                               int64_t K, hipStream_t s) {
    const int64_t chunks = M * K / 8;
    float* partial = static_cast<float*>(ws);
    act_absmax_kernel<<<kActBlocks, kThreads, 0, s>>>(A, partial, chunks);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_act_encode<false>(A, partial, qa, s_a, chunks, s);
}

hipError_t launch_quantize_act_static(const uint16_t* A, const float* s_a, uint8_t* qa, int64_t M, int64_t K,
                                      hipStream_t s) {
    const int64_t chunks = M * K / 8;
    return launch_act_encode<true>(A, nullptr, qa, const_cast<float*>(s_a), chunks, s);
}

}  // namespace vla
