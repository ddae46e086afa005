// Pieces shared by the GEMM kernels: kernel arguments, the fused epilogues
// (scale, bias, residual, GELU-tanh * up) and the cross-workgroup split-K
// protocol.
//
// Cross-workgroup protocol: partials are written and read only with
// device-coherent accesses (the sc1 cache policy of agent-scope atomic
// stores and loads on gfx950, served at the level of the hierarchy every
// XCD sees), and every wave waits for its stores to complete before the
// workgroup's arrival is counted with an agent-scope atomic.  That is the
// ordering a release/acquire pair provides for these accesses, without the
// L2 write-back and invalidate a device-scope fence issues (~20 us per call
// on MI355X, against a kernel of a few microseconds).
#pragma once

#include "vla_device.h"
#include "vla_internal.h"

namespace vla {
namespace gemm_detail {

struct KArgs {
    const void* A;
    const float* s_a;
    const void* W;
    const float* s_w;
    const uint16_t* bias;
    const uint16_t* resid;
    uint16_t* Y;
    uint16_t* gu;
    uint16_t* ypre;     // nullable: bf16(acc * scale + bias) before the residual add
    uint32_t* tickets;
    uint32_t* err;      // the workspace's status word (a bounded wait gave up)
    float* part;
    uint32_t part_bytes;
    uint32_t wait_polls;   // bound of every in-kernel wait, in polls
    int M, N, K;
    int ksplit;
    int groups;
    int msplit;     // skinny kernel: activation row blocks (grid z)
};

// s_waitcnt immediate that waits until at most n vector-memory operations
// are outstanding (lgkmcnt and expcnt left unconstrained).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }

// ------------------------------------------------------------- epilogue

// Epilogue inputs of one output fragment (row m, output columns n..n+3),
// loaded early so their latency overlaps the weight stream.
struct EpiIn {
    float4 s;       // weight scales (gate scales for the fused gate/up epilogue)
    float4 su;      // up scales (fused gate/up epilogue)
    uint2 bias;     // bias (gate bias for the fused gate/up epilogue)
    uint2 bu;       // up bias (fused gate/up epilogue)
    uint2 resid;
};

__device__ __forceinline__ uint16_t lo16(uint32_t w) { return static_cast<uint16_t>(w & 0xFFFFu); }
__device__ __forceinline__ uint16_t hi16(uint32_t w) { return static_cast<uint16_t>(w >> 16); }

template <WType WT, Epi EPI>
__device__ __forceinline__ EpiIn load_epi(const KArgs& a, int m, int n, bool with_resid) {
    EpiIn e;
    e.s = make_float4(1.0f, 1.0f, 1.0f, 1.0f);
    e.su = e.s;
    e.bias = make_uint2(0, 0);
    e.bu = make_uint2(0, 0);
    e.resid = make_uint2(0, 0);
    if (WT == WType::FP8) e.s = *reinterpret_cast<const float4*>(a.s_w + n);
    if (EPI == Epi::GELU_MUL) {
        e.su = *reinterpret_cast<const float4*>(a.s_w + (a.N >> 1) + n);
        if (a.bias) {
            e.bias = *reinterpret_cast<const uint2*>(a.bias + n);
            e.bu = *reinterpret_cast<const uint2*>(a.bias + (a.N >> 1) + n);
        }
    } else {
        if (a.bias) e.bias = *reinterpret_cast<const uint2*>(a.bias + n);
        if (a.resid && with_resid) e.resid = *reinterpret_cast<const uint2*>(a.resid + static_cast<int64_t>(m) * a.N + n);
    }
    return e;
}

// y = v * scale (+ bias) -> bf16 for four columns (before any residual).
template <AType AT, WType WT>
__device__ __forceinline__ uint2 epi_plain4(const KArgs& a, f32x4_t v, const EpiIn& e, float sa) {
    const bool scaled = (WT == WType::FP8 || AT == AType::FP8);
    float y[4] = {v[0], v[1], v[2], v[3]};
    if (scaled) {
        y[0] *= e.s.x * sa;
        y[1] *= e.s.y * sa;
        y[2] *= e.s.z * sa;
        y[3] *= e.s.w * sa;
    }
    if (a.bias) {
        y[0] += bf16_to_f32(lo16(e.bias.x));
        y[1] += bf16_to_f32(hi16(e.bias.x));
        y[2] += bf16_to_f32(lo16(e.bias.y));
        y[3] += bf16_to_f32(hi16(e.bias.y));
    }
    return make_uint2(f32x2_to_bf16x2(y[0], y[1]), f32x2_to_bf16x2(y[2], y[3]));
}

// bf16(residual + y) on two packed bf16 values.
__device__ __forceinline__ uint32_t add_resid2(uint32_t y, uint32_t r) {
    return f32x2_to_bf16x2(bf16_to_f32(lo16(r)) + bf16_to_f32(lo16(y)), bf16_to_f32(hi16(r)) + bf16_to_f32(hi16(y)));
}

// y = v * scale (+ bias) -> bf16, then bf16(residual + y); four columns.
template <AType AT, WType WT>
__device__ __forceinline__ void store_plain(const KArgs& a, int m, int n, f32x4_t v, const EpiIn& e, float sa) {
    uint2 o = epi_plain4<AT, WT>(a, v, e, sa);
    if (a.resid) {
        if (a.ypre) *reinterpret_cast<uint2*>(a.ypre + static_cast<int64_t>(m) * a.N + n) = o;
        o.x = add_resid2(o.x, e.resid.x);
        o.y = add_resid2(o.y, e.resid.y);
    }
    *reinterpret_cast<uint2*>(a.Y + static_cast<int64_t>(m) * a.N + n) = o;
}

// act = bf16(gelu_tanh(g) * u) with g = bf16(vg * sg (+ bg)), u = bf16(vu * su
// (+ bu)); four gate columns.  g and u are returned for the optional gate/up
// output.
__device__ __forceinline__ uint2 epi_gelu4(f32x4_t vg, f32x4_t vu, const EpiIn& e, bool bias, uint2& gp, uint2& up) {
    float g[4] = {vg[0] * e.s.x, vg[1] * e.s.y, vg[2] * e.s.z, vg[3] * e.s.w};
    float u[4] = {vu[0] * e.su.x, vu[1] * e.su.y, vu[2] * e.su.z, vu[3] * e.su.w};
    if (bias) {
        g[0] += bf16_to_f32(lo16(e.bias.x));
        g[1] += bf16_to_f32(hi16(e.bias.x));
        g[2] += bf16_to_f32(lo16(e.bias.y));
        g[3] += bf16_to_f32(hi16(e.bias.y));
        u[0] += bf16_to_f32(lo16(e.bu.x));
        u[1] += bf16_to_f32(hi16(e.bu.x));
        u[2] += bf16_to_f32(lo16(e.bu.y));
        u[3] += bf16_to_f32(hi16(e.bu.y));
    }
    gp = make_uint2(f32x2_to_bf16x2(g[0], g[1]), f32x2_to_bf16x2(g[2], g[3]));
    up = make_uint2(f32x2_to_bf16x2(u[0], u[1]), f32x2_to_bf16x2(u[2], u[3]));
    const float a0 = gelu_mul(bf16_to_f32(lo16(gp.x)), bf16_to_f32(lo16(up.x)));
    const float a1 = gelu_mul(bf16_to_f32(hi16(gp.x)), bf16_to_f32(hi16(up.x)));
    const float a2 = gelu_mul(bf16_to_f32(lo16(gp.y)), bf16_to_f32(lo16(up.y)));
    const float a3 = gelu_mul(bf16_to_f32(hi16(gp.y)), bf16_to_f32(hi16(up.y)));
    return make_uint2(f32x2_to_bf16x2(a0, a1), f32x2_to_bf16x2(a2, a3));
}

// Gate values vg and up values vu for row m, gate columns n..n+3 (n < I).
__device__ __forceinline__ void store_gelu(const KArgs& a, int m, int n, f32x4_t vg, f32x4_t vu, const EpiIn& e) {
    const int I = a.N >> 1;
    uint2 g, u;
    const uint2 o = epi_gelu4(vg, vu, e, a.bias != nullptr, g, u);
    *reinterpret_cast<uint2*>(a.Y + static_cast<int64_t>(m) * I + n) = o;
    if (a.gu) {
        *reinterpret_cast<uint2*>(a.gu + static_cast<int64_t>(m) * a.N + n) = g;
        *reinterpret_cast<uint2*>(a.gu + static_cast<int64_t>(m) * a.N + I + n) = u;
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

// Record that a bounded wait gave up (its output was not written): OR the
// cause bit into the workspace's status word, read back on the host by
// vla_workspace_status.
__device__ __forceinline__ void report_wait_timeout(uint32_t* err, uint32_t cause) {
    __hip_atomic_fetch_or(err, cause, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

}  // namespace gemm_detail

// Wide kernel (gemm_wide.hip).  For the wide kernel GemmPlan::nt holds the
// tile width BN (128 or 256).
template <AType AT, WType WT, Epi EPI>
hipError_t launch_wide(const gemm_detail::KArgs& ka, const GemmPlan& p, hipStream_t s);
size_t wide_part_bytes(const GemmPlan& p);
bool wide_dispatchable(const GemmPlan& p, AType at, WType wt, Epi epi);

}  // namespace vla
