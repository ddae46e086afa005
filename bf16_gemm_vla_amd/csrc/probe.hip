// Streaming-read probe: the time one launch takes to read a buffer from HBM
// and do nothing else.  It is the floor under a weight-streaming GEMM call
// of the same bytes (the decoder GEMMs of "Real-time VLA inference on AMD
// hardware" are bound by streaming their weights, section "FP8 helps the
// encoder and hurts the decoder"), so a call's time can be read against it.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "vla_device.h"
#include "vla_internal.h"

namespace vla {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 4;   // 16-byte loads in flight per thread

__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(const uint4* __restrict__ p, int64_t n,
                                                                    uint32_t* __restrict__ sink) {
    uint32_t acc = 0;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kProbeThreads * kProbeUnroll;
    for (int64_t base = blockIdx.x * static_cast<int64_t>(kProbeThreads) * kProbeUnroll + threadIdx.x; base < n;
         base += stride) {
        uint4 v[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) {
            const int64_t i = base + u * kProbeThreads;
            v[u] = i < n ? p[i] : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    // the loads must not be dropped; the store almost never happens
    if (acc == 0x9E3779B9u) sink[0] = acc;
}

}  // namespace

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, int blocks, hipStream_t s) {
    stream_read_kernel<<<blocks, kProbeThreads, 0, s>>>(static_cast<const uint4*>(src),
                                                        static_cast<int64_t>(bytes / 16), sink);
    return hipGetLastError();
}

}  // namespace vla

// ------------------------------------------------------------------------
// Matrix-core rate probe: every wave runs `iters` rounds of four independent
// MFMA chains on operands held in registers, so nothing but the matrix pipe
// limits it.  The operands come from a caller buffer (zeros, ones, random
// codes): the issue rate of these instructions depends on the data, and the
// ceiling a GEMM of these shapes can reach is the rate on operands like its
// own, not the published peak.  The four chains use four different operand
// sets, so the inputs change from one instruction to the next as they do in
// a GEMM.  Each lane writes the sum of its accumulators, which lets a test
// check that the launch did exactly the multiply-adds it is credited with.

namespace vla {
namespace {

constexpr int kRateChains = 4;
constexpr int kRateThreads = 256;
constexpr int kRateWordsPerLane = 64;   // four operand sets of A and B, 8 dwords each

typedef __attribute__((ext_vector_type(8))) int i32x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;

template <int FORM>
struct RateForm;
template <>
struct RateForm<VLA_MFMA_BF16_32X32X16> {
    typedef f32x16_t Acc;
    static __device__ __forceinline__ Acc step(const uint32_t* a, const uint32_t* b, Acc c) {
        const u32x4_t av = {a[0], a[1], a[2], a[3]}, bv = {b[0], b[1], b[2], b[3]};
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(av), as_bf16x8(bv), c, 0, 0, 0);
    }
};
template <>
struct RateForm<VLA_MFMA_BF16_16X16X32> {
    typedef f32x4_t Acc;
    static __device__ __forceinline__ Acc step(const uint32_t* a, const uint32_t* b, Acc c) {
        const u32x4_t av = {a[0], a[1], a[2], a[3]}, bv = {b[0], b[1], b[2], b[3]};
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av), as_bf16x8(bv), c, 0, 0, 0);
    }
};
template <>
struct RateForm<VLA_MFMA_FP8_32X32X64> {
    typedef f32x16_t Acc;
    static __device__ __forceinline__ Acc step(const uint32_t* a, const uint32_t* b, Acc c) {
        i32x8_t av, bv;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            av[i] = static_cast<int>(a[i]);
            bv[i] = static_cast<int>(b[i]);
        }
        // E4M3 x E4M3 (format 0 for both), unit E8M0 scales (127)
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c, 0, 0, 0, 127, 0, 127);
    }
};
template <>
struct RateForm<VLA_MFMA_FP8_16X16X128> {
    typedef f32x4_t Acc;
    static __device__ __forceinline__ Acc step(const uint32_t* a, const uint32_t* b, Acc c) {
        i32x8_t av, bv;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            av[i] = static_cast<int>(a[i]);
            bv[i] = static_cast<int>(b[i]);
        }
        return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 0, 0, 0, 127, 0, 127);
    }
};

template <int FORM>
__global__ __launch_bounds__(kRateThreads) void mfma_rate_kernel(const uint32_t* __restrict__ src, int iters,
                                                                 float* __restrict__ out, uint64_t* __restrict__ clocks) {
    typedef typename RateForm<FORM>::Acc Acc;
    uint32_t ops[kRateWordsPerLane];
    const uint32_t* p = src + threadIdx.x * kRateWordsPerLane;
#pragma unroll
    for (int i = 0; i < kRateWordsPerLane; ++i) ops[i] = p[i];
    // four named chains: with an array of vector accumulators the register
    // allocator rotates them through copies inside the loop
    Acc c0{}, c1{}, c2{}, c3{};
    static_assert(kRateChains == 4, "four chains");
    asm volatile("" : "+a"(c0), "+a"(c1), "+a"(c2), "+a"(c3));
    // shader-clock cycles and 100 MHz real-time ticks around the loop: their
    // ratio is the clock the instructions ran at
    const uint64_t t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
        c0 = RateForm<FORM>::step(ops + 0, ops + 8, c0);
        c1 = RateForm<FORM>::step(ops + 16, ops + 24, c1);
        c2 = RateForm<FORM>::step(ops + 32, ops + 40, c2);
        c3 = RateForm<FORM>::step(ops + 48, ops + 56, c3);
        // pins each chain to its own registers across iterations (no code)
        asm volatile("" : "+a"(c0), "+a"(c1), "+a"(c2), "+a"(c3));
    }
    const uint64_t t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
    if (clocks && threadIdx.x == 0) {
        clocks[2 * blockIdx.x] = t1 - t0;
        clocks[2 * blockIdx.x + 1] = r1 - r0;
    }
    float s = 0.0f;
#pragma unroll
    for (int e = 0; e < static_cast<int>(sizeof(Acc) / sizeof(float)); ++e) s += c0[e];
#pragma unroll
    for (int e = 0; e < static_cast<int>(sizeof(Acc) / sizeof(float)); ++e) s += c1[e];
#pragma unroll
    for (int e = 0; e < static_cast<int>(sizeof(Acc) / sizeof(float)); ++e) s += c2[e];
#pragma unroll
    for (int e = 0; e < static_cast<int>(sizeof(Acc) / sizeof(float)); ++e) s += c3[e];
    out[static_cast<int64_t>(blockIdx.x) * kRateThreads + threadIdx.x] = s;
}

}  // namespace

hipError_t launch_mfma_rate(int form, const uint32_t* src, int iters, float* out, uint64_t* clocks, int blocks,
                            hipStream_t s) {
    switch (form) {
        case VLA_MFMA_BF16_32X32X16:
            mfma_rate_kernel<VLA_MFMA_BF16_32X32X16><<<blocks, kRateThreads, 0, s>>>(src, iters, out, clocks);
            break;
        case VLA_MFMA_BF16_16X16X32:
            mfma_rate_kernel<VLA_MFMA_BF16_16X16X32><<<blocks, kRateThreads, 0, s>>>(src, iters, out, clocks);
            break;
        case VLA_MFMA_FP8_32X32X64:
            mfma_rate_kernel<VLA_MFMA_FP8_32X32X64><<<blocks, kRateThreads, 0, s>>>(src, iters, out, clocks);
            break;
        default:
            mfma_rate_kernel<VLA_MFMA_FP8_16X16X128><<<blocks, kRateThreads, 0, s>>>(src, iters, out, clocks);
            break;
    }
    return hipGetLastError();
}

}  // namespace vla
