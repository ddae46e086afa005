// Fused decoder boundary ("Real-time VLA inference on AMD hardware", section
// "Fusing the BF16 decoder boundary"): the gated residual update and the
// adaptive RMS norm of its result in one kernel,
//   r  = bf16(residual + out * gate)
//   h  = bf16(r / sqrt(mean(r^2) + eps) * (1 + scale) + shift)
//   ng = next gate,
// with (scale | shift | next gate) the D-wide blocks of a style row.
//
// One workgroup of 256 threads per row, 4 consecutive channels per thread
// per chunk (8-byte loads and stores), every load of the row issued before
// any arithmetic.  The arithmetic is fp64: out * gate and the sum with the
// residual are exact there (bf16 significands), and each bf16 result is
// rounded once from fp64 (round-to-odd to fp32, then nearest-even to bf16),
// so r is the correctly rounded sum bit for bit.  The sum of squares is
// reduced in a fixed order (thread, wave, then the four waves), so results
// are bitwise repeatable.  The kernel is bound by latency at decoder sizes
// (M = 50, D = 1024: 0.9 MB moved).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "vla_device.h"
#include "vla_internal.h"

namespace vla {
namespace {

constexpr int kBThreads = 256;

struct BArgs {
    const uint16_t* resid;
    const uint16_t* out;
    const uint16_t* gate;
    const uint16_t* style;
    uint16_t* r_out;
    uint16_t* h_out;
    uint16_t* ng_out;
    int64_t D;
    int style_per_row;
    float eps;
};

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

template <int CH>
__global__ __launch_bounds__(kBThreads) void gate_residual_ada_norm_kernel(BArgs a) {
    __shared__ double part[kBThreads / 64];
    const int tid = threadIdx.x;
    const int64_t nq = a.D >> 2;                                    // 4-channel chunks per row
    const int64_t row = static_cast<int64_t>(blockIdx.x) * a.D;
    const uint16_t* st = a.style + (a.style_per_row ? static_cast<int64_t>(blockIdx.x) * 3 * a.D : 0);

    // chunks past the row load chunk 0 (always present) and are never used,
    // so every load is unconditional
    uint2 xv[CH], yv[CH], gv[CH], sc[CH], sh[CH], ng[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const int64_t q0 = tid + static_cast<int64_t>(c) * kBThreads;
        const int64_t q = q0 < nq ? q0 : 0;
        xv[c] = *reinterpret_cast<const uint2*>(a.resid + row + 4 * q);
        yv[c] = *reinterpret_cast<const uint2*>(a.out + row + 4 * q);
        gv[c] = *reinterpret_cast<const uint2*>(a.gate + row + 4 * q);
        sc[c] = *reinterpret_cast<const uint2*>(st + 4 * q);
        sh[c] = *reinterpret_cast<const uint2*>(st + a.D + 4 * q);
        ng[c] = *reinterpret_cast<const uint2*>(st + 2 * a.D + 4 * q);
    }

    // gated residual, one rounding per value; sum of squares of the rounded r
    double r[CH][4];
    double ss = 0.0;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const int64_t q = tid + static_cast<int64_t>(c) * kBThreads;
        const uint32_t xw[2] = {xv[c].x, xv[c].y}, yw[2] = {yv[c].x, yv[c].y}, gw[2] = {gv[c].x, gv[c].y};
        uint32_t rw[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t b0 = gated_residual_bf16(xw[h] & 0xFFFFu, yw[h] & 0xFFFFu, gw[h] & 0xFFFFu);
            const uint32_t b1 = gated_residual_bf16(xw[h] >> 16, yw[h] >> 16, gw[h] >> 16);
            rw[h] = b0 | (b1 << 16);
            r[c][2 * h] = bf16_f64(b0);
            r[c][2 * h + 1] = bf16_f64(b1);
        }
        if (q < nq) {
            *reinterpret_cast<uint2*>(a.r_out + row + 4 * q) = make_uint2(rw[0], rw[1]);
#pragma unroll
            for (int e = 0; e < 4; ++e) ss += r[c][e] * r[c][e];
        }
    }
    ss = wave_sum(ss);
    if ((tid & 63) == 0) part[tid >> 6] = ss;
    __syncthreads();
    double total = part[0];
#pragma unroll
    for (int w = 1; w < kBThreads / 64; ++w) total += part[w];
    const double inv = 1.0 / sqrt(total / static_cast<double>(a.D) + static_cast<double>(a.eps));

    // adaptive norm: scale, shift, then one rounding to bf16
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const int64_t q = tid + static_cast<int64_t>(c) * kBThreads;
        if (q >= nq) continue;
        const uint32_t sw[2] = {sc[c].x, sc[c].y}, tw[2] = {sh[c].x, sh[c].y};
        uint32_t hw[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const double h0 = r[c][2 * h] * inv * (1.0 + bf16_f64(sw[h] & 0xFFFFu)) + bf16_f64(tw[h] & 0xFFFFu);
            const double h1 = r[c][2 * h + 1] * inv * (1.0 + bf16_f64(sw[h] >> 16)) + bf16_f64(tw[h] >> 16);
            hw[h] = f64_to_bf16(h0) | (f64_to_bf16(h1) << 16);
        }
        *reinterpret_cast<uint2*>(a.h_out + row + 4 * q) = make_uint2(hw[0], hw[1]);
        if (a.ng_out) *reinterpret_cast<uint2*>(a.ng_out + row + 4 * q) = ng[c];
    }
}

}  // namespace

hipError_t launch_gate_residual_ada_norm(const uint16_t* resid, const uint16_t* out, const uint16_t* gate,
                                         const uint16_t* style, int style_per_row, float eps, uint16_t* r_out,
                                         uint16_t* h_out, uint16_t* ng_out, int64_t M, int64_t D, hipStream_t s) {
    const BArgs a{resid, out, gate, style, r_out, h_out, ng_out, D, style_per_row, eps};
    const dim3 grid(static_cast<unsigned>(M));
    const int64_t ch = (D / 4 + kBThreads - 1) / kBThreads;
    if (ch <= 1) gate_residual_ada_norm_kernel<1><<<grid, kBThreads, 0, s>>>(a);
    else if (ch <= 2) gate_residual_ada_norm_kernel<2><<<grid, kBThreads, 0, s>>>(a);
    else if (ch <= 4) gate_residual_ada_norm_kernel<4><<<grid, kBThreads, 0, s>>>(a);
    else if (ch <= 8) gate_residual_ada_norm_kernel<8><<<grid, kBThreads, 0, s>>>(a);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

bool boundary_width_ok(int64_t D) { return D > 0 && D % 4 == 0 && D <= 4 * kBThreads * 8; }

}  // namespace vla
