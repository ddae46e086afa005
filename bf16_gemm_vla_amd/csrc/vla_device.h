// Device-side helpers shared by the gfx950 kernels: bit-level E4M3 and bf16
// conversions, MFMA operand types and wavefront reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vla {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;

constexpr int kWave = 64;

// ------------------------------------------------------------------- bf16

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// fp32 -> bf16 with gfx950's conversion instruction: round to nearest even
// (the default rounding mode), NaN stays a quiet NaN.
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Two fp32 -> two bf16 packed in one dword (lo in the low half), one instruction.
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float lo, float hi) {
    const bf16x2_t r = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
    return __builtin_bit_cast(uint32_t, r);
}

// ------------------------------------------------------------------- E4M3

// Dialect constants: OCP (bias 7, max 448 = 0x43E00000, smallest normal
// 2^-6) and FNUZ (bias 8, max 240 = 0x43700000, smallest normal 2^-7).
template <bool FNUZ>
struct E4M3 {
    static constexpr int bias = FNUZ ? 8 : 7;
    static constexpr uint32_t max_bits = FNUZ ? 0x43700000u : 0x43E00000u;
    static constexpr uint32_t min_normal_bits = FNUZ ? 0x3C000000u : 0x3C800000u;
    static constexpr uint8_t max_code = FNUZ ? 0x7F : 0x7E;
    // subnormal quantum is 2^(1 - bias - 3); its reciprocal as an fp32
    static constexpr float inv_quantum = FNUZ ? 1024.0f : 512.0f;
};

// fp32 -> E4M3 code: round to nearest even, saturate at +-max; NaN -> OCP
// 0x7F|sign or FNUZ 0x80; zero keeps its sign in OCP, is 0x00 in FNUZ.
template <bool FNUZ>
__device__ __forceinline__ uint8_t encode_e4m3(float x) {
    using F = E4M3<FNUZ>;
    const uint32_t u = __float_as_uint(x);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7FFFFFFFu;
    if (a > 0x7F800000u) return FNUZ ? 0x80 : static_cast<uint8_t>(0x7F | sign);
    if (a >= F::max_bits) return static_cast<uint8_t>(F::max_code | sign);
    uint32_t code;
    if (a >= F::min_normal_bits) {
        // keep 3 of the 23 fraction bits, ties to even, then rebias
        const uint32_t r = (a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20;
        code = r - static_cast<uint32_t>((127 - F::bias) << 3);
    } else {
        // subnormal range: count quanta, rintf rounds ties to even; the
        // scaling by a power of two is exact
        code = static_cast<uint32_t>(__builtin_rintf(__uint_as_float(a) * F::inv_quantum));
    }
    if (FNUZ && code == 0) return 0;
    return static_cast<uint8_t>(code | sign);
}

// E4M3 code -> fp32 (exact).  NaN codes give a quiet NaN.
template <bool FNUZ>
__device__ __forceinline__ float decode_e4m3(uint32_t b) {
    using F = E4M3<FNUZ>;
    const uint32_t mag = b & 0x7Fu;
    const bool neg = (b & 0x80u) != 0;
    if (FNUZ ? (b == 0x80u) : (mag == 0x7Fu)) return __uint_as_float(0x7FC00000u);
    const uint32_t e = mag >> 3, m = mag & 7u;
    float v;
    if (e == 0)
        v = static_cast<float>(m) * (1.0f / F::inv_quantum);
    else
        v = __uint_as_float(((e + 127u - F::bias) << 23) | (m << 20));
    return neg ? -v : v;
}

// Four OCP E4M3 codes (one dword) -> four bf16 (two dwords), exact: every
// E4M3 value (subnormals included) is a bf16 value, and gfx950 converts a
// pair of FP8 codes to a pair of bf16 in one instruction (unit scale).
__device__ __forceinline__ u32x2_t ocp4_to_bf16x4(uint32_t w) {
    const bf16x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
    const bf16x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
    u32x2_t r;
    r.x = __builtin_bit_cast(uint32_t, lo);
    r.y = __builtin_bit_cast(uint32_t, hi);
    return r;
}

// Eight OCP E4M3 codes -> eight bf16 as an MFMA operand.
__device__ __forceinline__ bf16x8_t ocp8_to_bf16x8(u32x2_t w) {
    u32x2_t a = ocp4_to_bf16x4(w.x), b = ocp4_to_bf16x4(w.y);
    u32x4_t v = {a.x, a.y, b.x, b.y};
    return __builtin_bit_cast(bf16x8_t, v);
}

// E8M0 block scale -> fp32 2^(e - 127) (e = 0 is the subnormal 2^-127).
__device__ __forceinline__ float e8m0_to_f32(uint32_t e) {
    return __uint_as_float(e ? (e << 23) : 0x00400000u);
}

// Eight E2M1 codes (one dword, element i in bits 4i..4i+3) times a block
// scale -> eight bf16 as an MFMA operand.  Exact: an E2M1 value times a
// power of two in bf16's range is a bf16 value; gfx950 converts a byte (two
// codes, low nibble first) to a pair of scaled bf16 in one instruction.
__device__ __forceinline__ bf16x8_t fp4_to_bf16x8(uint32_t w, float scale) {
    const bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0);
    const bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1);
    const bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2);
    const bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3);
    const u32x4_t v = {__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
                       __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3)};
    return __builtin_bit_cast(bf16x8_t, v);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

// --------------------------------------------------------- wave reductions

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
    return v;
}

// Max over aligned groups of `G` consecutive lanes (G a power of two <= 64).
template <int G>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
    for (int off = G / 2; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
    return v;
}

// GELU, tanh form, times u: 0.5 g (1 + tanh(z)) u, z = sqrt(2/pi) (g +
// 0.044715 g^3), evaluated as g / (1 + exp(-2z)) * u (the same function:
// 1 + tanh(z) = 2 / (1 + exp(-2z))), which keeps its relative accuracy for
// negative g, where 1 + tanh(z) cancels to a few ulps or to zero in fp32.
// exp and the reciprocal are gfx950's exp2 and reciprocal instructions
// (about 1 ulp of fp32 each): the result is rounded to bf16, 2^16 times
// coarser, so they move it by at most one bf16 ulp, and only next to a
// rounding boundary.
// For z < -40 (g below about -9.2) gelu(g) = g e^{2z} / (1 + e^{2z}) is
// below ~1e-34, where 1 + e^{2z} is 1 in fp32: the value is g u e^{2z},
// whose factors would overflow (g u) or leave the normal range (e^{2z},
// exp(-2z) overflowing near g = -10.1) while the product can still be a
// normal number when |u| is large.  It is formed with exact exponents:
// g = mg 2^eg, u = mu 2^eu (frexp), 2z log2(e) = ti + tf with ti an
// integer and tf in [0, 1), then (mg mu 2^tf) 2^(eg + eu + ti) with one
// rounding in ldexp.  Rare in practice (a wave takes the branch only if one
// of its lanes needs it).
__device__ __forceinline__ float gelu_mul(float g, float u) {
    const float c = 0.7978845608028654f;  // sqrt(2/pi)
    const float z = c * (g + 0.044715f * g * g * g);
    if (z > -40.0f) {
        const float e = __builtin_amdgcn_exp2f(-2.8853900817779268f * z);    // exp(-2z), -2 log2(e) z < 116
        return g * __builtin_amdgcn_rcpf(1.0f + e) * u;
    }
    const float t = fmaxf(2.0f * z * 1.4426950408889634f, -2048.0f);   // log2 e^{2z}; below -2048 all underflow
    const float ti = floorf(t);
    int eg, eu;
    const float mg = frexpf(g, &eg), mu = frexpf(u, &eu);
    return ldexpf(mg * mu * exp2f(t - ti), eg + eu + static_cast<int>(ti));
}

// bf16 bits -> fp64 (exact).
__device__ __forceinline__ double bf16_f64(uint32_t bits16) { return static_cast<double>(__uint_as_float(bits16 << 16)); }

// Nearest-even bf16 of an fp64 value with one rounding: truncate to fp32,
// set the lowest bit if that was inexact (round to odd keeps the 29 dropped
// bits' information in a sticky bit), then round the fp32 bits to bf16.
__device__ __forceinline__ uint32_t f64_to_bf16(double v) {
    const float t = __double2float_rz(v);
    uint32_t b = __float_as_uint(t);
    if (static_cast<double>(t) != v) b |= 1u;
    b += 0x7FFFu + ((b >> 16) & 1u);
    return b >> 16;
}

// Gated residual of the decoder boundary for one value: bf16(x + y * g),
// the product and sum exact in fp64 (bf16 significands) and rounded once.
__device__ __forceinline__ uint32_t gated_residual_bf16(uint32_t x16, uint32_t y16, uint32_t g16) {
    return f64_to_bf16(bf16_f64(x16) + bf16_f64(y16) * bf16_f64(g16));
}

}  // namespace vla
