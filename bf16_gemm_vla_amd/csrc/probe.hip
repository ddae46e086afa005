// Streaming-read probe: the time one launch takes to read a buffer from HBM
// and do nothing else.  It is the floor under a weight-streaming GEMM call
// of the same bytes (the decoder GEMMs of "Real-time VLA inference on AMD
// hardware" are bound by streaming their weights, section "FP8 helps the
// encoder and hurts the decoder"), so a call's time can be read against it.
#include <hip/hip_runtime.h>

#include <cstdint>

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
