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

// One workgroup per 16-row tile.  Phase 1: row absmax -> scale.  Phase 2:
// each thread encodes 8-value slots (reads 2 x 16 B, writes 8 B / 16 B).
template <int WFMT>
__global__ __launch_bounds__(kThreads) void quantize_pack_kernel(const float* __restrict__ W,
                                                                 void* __restrict__ Wq,
                                                                 float* __restrict__ scales,
                                                                 int64_t K, int layout) {
    __shared__ float s_scale[16];
    const int64_t n0 = blockIdx.x;
    const int t = threadIdx.x;
    const float* tile = W + n0 * 16 * K;

    if (WFMT != VLA_WFMT_BF16) {
        // 16 threads per row, float4 loads strided by 64 floats
        const int r = t >> 4, c = t & 15;
        const float* row = tile + static_cast<int64_t>(r) * K;
        float m = 0.0f;
        for (int64_t k = 4 * c; k < K; k += 64) {
            float4 v = *reinterpret_cast<const float4*>(row + k);
            m = fmaxf(m, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
        }
        m = group_max<16>(m);
        if (c == 0) {
            const float maxv = (WFMT == VLA_WFMT_E4M3_FNUZ) ? 240.0f : 448.0f;
            const float sc = (m == 0.0f) ? 1.0f : __fdiv_rn(m, maxv);
            s_scale[r] = sc;
            scales[n0 * 16 + r] = sc;
        }
        __syncthreads();
    }

    const int64_t nslots = (K >> 5) * 64;
    for (int64_t slot = t; slot < nslots; slot += kThreads) {
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
            const float sc = s_scale[n1];
            uint32_t w[2] = {0, 0};
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float x = __fdiv_rn(v[i], sc);
                const uint32_t code = (WFMT == VLA_WFMT_E4M3_FNUZ) ? encode_e4m3<true>(x)
                                                                    : encode_e4m3<false>(x);
                w[i >> 2] |= code << (8 * (i & 3));
            }
            *reinterpret_cast<uint2*>(static_cast<uint8_t*>(Wq) + off) = make_uint2(w[0], w[1]);
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
// row are one aligned load.
__global__ __launch_bounds__(kThreads) void mxfp4_quantize_pack_kernel(const float* __restrict__ W,
                                                                       uint8_t* __restrict__ Wq, int64_t N,
                                                                       int64_t K) {
    const int64_t n0 = blockIdx.x;
    const int64_t ksteps = K >> 5;
    const int64_t P = mxfp4_scale_row_bytes(K);
    uint8_t* const sc_base = Wq + N * K / 2;
    for (int64_t b = threadIdx.x; b < P * 16; b += kThreads) {
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

// Row-major FP8 -> MFMA layout: one thread per 8-byte slot.
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

// Activation quantization, pass 1: per-block absmax of 8-element chunks.
constexpr int kActBlocks = 512;

// Every thread keeps kActUnroll 16-byte loads in flight at a time.
constexpr int kActUnroll = 4;

__global__ __launch_bounds__(kThreads) void act_absmax_kernel(const uint16_t* __restrict__ A,
                                                              float* __restrict__ partial,
                                                              int64_t chunks) {
    __shared__ float red[kThreads / kWave];
    float m = 0.0f;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads * kActUnroll;
    for (int64_t base = blockIdx.x * static_cast<int64_t>(kThreads) * kActUnroll + threadIdx.x; base < chunks;
         base += stride) {
        uint4 v[kActUnroll];
#pragma unroll
        for (int u = 0; u < kActUnroll; ++u) {
            const int64_t i = base + u * kThreads;
            v[u] = i < chunks ? *reinterpret_cast<const uint4*>(A + i * 8) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < kActUnroll; ++u) {
            const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                m = fmaxf(m, fabsf(bf16_to_f32(static_cast<uint16_t>(w[j] & 0xFFFFu))));
                m = fmaxf(m, fabsf(bf16_to_f32(static_cast<uint16_t>(w[j] >> 16))));
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
// the quotient correctly rounded as IEEE division gives it.  With rcp =
// RN(1/sc), q = RN(x * rcp) is within 2 fp32 ulps of RN(x / sc), and the
// code only changes at the midpoints between E4M3 values (fp32 fraction
// bits 19..0 == 0x80000 in the normal range), so the code of q is the code
// of the exact quotient unless q lies within 3 ulps of a midpoint, below the
// smallest normal E4M3 value (2^-6) but not zero, at/above 448, or is not
// finite.  Such q take the exact division and the bit-level encoder; all
// other q are zero or normal-range E4M3 values, which the hardware
// conversion (round to nearest even, gfx950's OCP format, signed zero kept)
// encodes two per instruction.
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

// Pass 2: every block loads its kActUnroll chunks per thread first, then
// reduces the partial maxima (same order everywhere), forms s_a and encodes.
// STATIC: s_a is a given (calibrated) scale, read instead of formed.
template <bool STATIC>
__global__ __launch_bounds__(kThreads) void act_encode_kernel(const uint16_t* __restrict__ A,
                                                              const float* __restrict__ partial,
                                                              uint8_t* __restrict__ qa,
                                                              float* __restrict__ s_a,
                                                              int64_t chunks) {
    __shared__ float s_sc;
    uint4 v[kActUnroll];
    const int64_t base = blockIdx.x * static_cast<int64_t>(kThreads) * kActUnroll + threadIdx.x;
#pragma unroll
    for (int u = 0; u < kActUnroll; ++u) {
        const int64_t i = base + u * kThreads;
        v[u] = i < chunks ? *reinterpret_cast<const uint4*>(A + i * 8) : make_uint4(0, 0, 0, 0);
    }
    if constexpr (STATIC) {
        if (threadIdx.x == 0) s_sc = *s_a;
    } else if (threadIdx.x < kWave) {
        // all partial maxima requested at once (one round trip, not one per load)
        static_assert(kActBlocks % kWave == 0, "partials split evenly over one wave");
        float p[kActBlocks / kWave];
#pragma unroll
        for (int i = 0; i < kActBlocks / kWave; ++i) p[i] = partial[threadIdx.x + i * kWave];
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < kActBlocks / kWave; ++i) m = fmaxf(m, p[i]);
        m = wave_max(m);
        if (threadIdx.x == 0) {
            const float sc = (m == 0.0f) ? 1.0f : __fdiv_rn(m, 448.0f);
            s_sc = sc;
            if (blockIdx.x == 0) *s_a = sc;
        }
    }
    __syncthreads();
    const float sc = s_sc;
    const float rcp = __fdiv_rn(1.0f, sc);
#pragma unroll
    for (int u = 0; u < kActUnroll; ++u) {
        const int64_t i = base + u * kThreads;
        if (i >= chunks) continue;
        const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
        *reinterpret_cast<uint2*>(qa + i * 8) = act_codes8(w, sc, rcp);
    }
}

}  // namespace

hipError_t launch_quantize_pack(const float* W, void* Wq, float* scales, int64_t N, int64_t K,
                                int wfmt, int layout, hipStream_t s) {
    const dim3 grid(static_cast<unsigned>(N / 16));
    switch (wfmt) {
        case VLA_WFMT_BF16:
            quantize_pack_kernel<VLA_WFMT_BF16><<<grid, kThreads, 0, s>>>(W, Wq, scales, K, layout);
            break;
        case VLA_WFMT_E4M3_OCP:
            quantize_pack_kernel<VLA_WFMT_E4M3_OCP><<<grid, kThreads, 0, s>>>(W, Wq, scales, K, layout);
            break;
        default:
            quantize_pack_kernel<VLA_WFMT_E4M3_FNUZ><<<grid, kThreads, 0, s>>>(W, Wq, scales, K, layout);
            break;
    }
    return hipGetLastError();
}

hipError_t launch_mxfp4_quantize_pack(const float* W, uint8_t* Wq, int64_t N, int64_t K, hipStream_t s) {
    mxfp4_quantize_pack_kernel<<<static_cast<unsigned>(N / 16), kThreads, 0, s>>>(W, Wq, N, K);
    return hipGetLastError();
}

hipError_t launch_pack_fp8(const uint8_t* q, uint8_t* qp, int64_t N, int64_t K, hipStream_t s) {
    const int64_t total = N * K / 8;
    const int64_t blocks = (total + kThreads - 1) / kThreads;
    const unsigned grid = static_cast<unsigned>(blocks < 65536 ? blocks : 65536);
    pack_fp8_kernel<<<grid, kThreads, 0, s>>>(q, qp, N, K);
    return hipGetLastError();
}

hipError_t launch_reencode(const uint8_t* q, const float* sc, uint8_t* q2, float* sc2, int64_t N,
                           int64_t K, int layout, hipStream_t s) {
    reencode_kernel<<<static_cast<unsigned>(N / 16), kThreads, 0, s>>>(q, sc, q2, sc2, K, layout);
    return hipGetLastError();
}

size_t quantize_act_ws_bytes(int64_t, int64_t) { return kActBlocks * sizeof(float); }

hipError_t launch_quantize_act(const uint16_t* A, uint8_t* qa, float* s_a, void* ws, int64_t M,
                               int64_t K, hipStream_t s) {
    const int64_t chunks = M * K / 8;
    float* partial = static_cast<float*>(ws);
    act_absmax_kernel<<<kActBlocks, kThreads, 0, s>>>(A, partial, chunks);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t per_block = static_cast<int64_t>(kThreads) * kActUnroll;
    const unsigned grid = static_cast<unsigned>(std::max<int64_t>(1, (chunks + per_block - 1) / per_block));
    act_encode_kernel<false><<<grid, kThreads, 0, s>>>(A, partial, qa, s_a, chunks);
    return hipGetLastError();
}

hipError_t launch_quantize_act_static(const uint16_t* A, const float* s_a, uint8_t* qa, int64_t M, int64_t K,
                                      hipStream_t s) {
    const int64_t chunks = M * K / 8;
    const int64_t per_block = static_cast<int64_t>(kThreads) * kActUnroll;
    const unsigned grid = static_cast<unsigned>(std::max<int64_t>(1, (chunks + per_block - 1) / per_block));
    act_encode_kernel<true><<<grid, kThreads, 0, s>>>(A, nullptr, qa, const_cast<float*>(s_a), chunks);
    return hipGetLastError();
}

}  // namespace vla
