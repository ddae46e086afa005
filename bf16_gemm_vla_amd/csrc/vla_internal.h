// Host-side declarations shared between the C ABI layer and the kernel
// launchers.  Launchers assume validated arguments and report launch errors
// through their hipError_t return value.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "vla.h"

namespace vla {

// ---------------------------------------------------------------- codec
hipError_t launch_quantize_pack(const float* W, void* Wq, float* scales, int64_t N, int64_t K,
                                int wfmt, int layout, hipStream_t s);
// MXFP4 block-scale bytes per weight row: K/32 rounded up to 8.
constexpr int64_t mxfp4_scale_row_bytes(int64_t K) { return ((K >> 5) + 7) & ~int64_t(7); }
hipError_t launch_mxfp4_quantize_pack(const float* W, uint8_t* Wq, int64_t N, int64_t K, hipStream_t s);
hipError_t launch_pack_fp8(const uint8_t* q, uint8_t* qp, int64_t N, int64_t K, hipStream_t s);
hipError_t launch_reencode(const uint8_t* q, const float* sc, uint8_t* q2, float* sc2, int64_t N,
                           int64_t K, int layout, hipStream_t s);
size_t quantize_act_ws_bytes(int64_t M, int64_t K);
hipError_t launch_quantize_act(const uint16_t* A, uint8_t* qa, float* s_a, void* ws, int64_t M,
                               int64_t K, hipStream_t s);
hipError_t launch_gate_residual_ada_norm(const uint16_t* resid, const uint16_t* out, const uint16_t* gate,
                                         const uint16_t* style, int style_per_row, float eps, uint16_t* r_out,
                                         uint16_t* h_out, uint16_t* ng_out, int64_t M, int64_t D, hipStream_t s);
bool boundary_width_ok(int64_t D);   // D a positive multiple of 4, at most 8192
hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, int blocks, hipStream_t s);
hipError_t launch_mfma_rate(int form, const uint32_t* src, int iters, float* out, uint64_t* clocks, int blocks,
                            hipStream_t s);
hipError_t launch_quantize_act_static(const uint16_t* A, const float* s_a, uint8_t* qa, int64_t M, int64_t K,
                                      hipStream_t s);

// ----------------------------------------------------------------- GEMM
enum class AType { BF16 = 0, FP8 = 1 };
enum class WType { BF16 = 0, FP8 = 1, FP4 = 2 };   // FP4: MXFP4 (E2M1 + E8M0 per 32 K)
enum class Epi { PLAIN = 0, GELU_MUL = 1 };

struct GemmProblem {
    const void* A;
    const float* s_a;       // device scalar for FP8 A, else nullptr
    const void* W;          // packed weights
    const float* s_w;       // per-row scales (FP8 weights), else nullptr
    const uint16_t* bias;   // nullable
    const uint16_t* resid;  // nullable
    uint16_t* Y;            // PLAIN: M x N; GELU_MUL: M x N/2
    uint16_t* gu;           // GELU_MUL debug output M x N, nullable
    uint16_t* ypre;         // PLAIN: output before the residual add, M x N, nullable
    void* ws;
    int64_t M, N, K;        // N = weight rows
    AType atype;
    WType wtype;
    Epi epi;
};

// Launch plan chosen for a problem (host-side, deterministic per shape).
struct GemmPlan {
    int kernel;     // 0 = skinny (M <= 64), 1 = wide
    int nt;         // skinny: 16-column tiles per workgroup; wide: tile width BN
    int steps;      // K steps (of 32) per wave per workgroup chunk (skinny)
    int waves;      // wavefronts per workgroup
    int wnw;        // wide: wavefronts along N (the rest are along M)
    int ksplit;     // number of K chunks across workgroups
    int groups;     // N groups (grid x)
    int mblocks;    // M blocks (wide: grid y of 192 rows; skinny: grid z of mt 16-row tiles)
    int mt;         // skinny: 16-row activation tiles per workgroup
    bool alds;      // skinny: stage activations through LDS
    bool ok;        // false when the shape exceeds the split-K counter or partial space
};

// The first kCounterBytes of every GEMM workspace hold the split-K arrival
// counters (one uint32 per skinny output group, kWideCounters per wide output
// tile: workgroups started, arrivals with handed-over slices, workgroups done),
// at the same place for every shape, so one zero-filled workspace can serve
// calls of different shapes.  Its last 4 KiB are not used.
constexpr size_t kCounterBytes = 65536;
constexpr size_t kZeroPageOffset = kCounterBytes - 4096;
constexpr int kMaxCounters = static_cast<int>(kZeroPageOffset / 4);
constexpr int kWideCounters = 4;   // three used, one pad
// The status word: the first 4 bytes of the page after the counters.  Zero
// until a bounded in-kernel wait gives up; each cause sets one bit.
constexpr size_t kStatusOffset = kZeroPageOffset;
constexpr uint32_t kStatusWideSplitK = 1u;   // wide split-K owner gave up waiting for partials
constexpr uint32_t kStatusChainBarrier = 2u;   // fused chain: a phase barrier gave up
// Split-K partial regions are addressed with 32-bit offsets.
constexpr uint64_t kMaxPartBytes = uint64_t(1) << 32;
// Default bound of every in-kernel wait, in polls (about 2 s of polling on
// MI355X; never reached by a grid that is resident).
constexpr uint32_t kDefaultWaitPolls = 1u << 22;
uint32_t wait_polls();                  // current bound (vla_set_wait_limit)

// vla_gemm_fp8w_noalloc's workspace: counters (64 KiB) + up to 32 MiB of
// split-K partials, enough for the encoder GEMMs at 768 rows.
constexpr size_t kNoAllocWorkspaceBytes = kCounterBytes + (size_t(32) << 20);
// Device address of the library's workspace on the current device (set up
// on first use per device; its counters are cleared by a kernel on `s`).
hipError_t noalloc_workspace(hipStream_t s, void** ptr);

// ------------------------------------------------------------ fused chain
// One persistent launch of kChainGrid workgroups runs every layer of the
// gated-MLP chain (chain.hip); the weight pointers travel in the kernel
// arguments, so at most kMaxChainLayers layers.
constexpr int kChainGrid = 256;
constexpr int kMaxChainLayers = 32;
// Barrier words of the fused chain (34 lines of 128 bytes), zero between
// launches; the chain scratch holds them after its GEMM workspace.
constexpr size_t kChainSyncBytes = 8192;

struct ChainLaunch {
    const uint8_t* const* wgu;     // host arrays of L device pointers
    const float* const* sgu;
    const uint8_t* const* wd;
    const float* const* sd;
    const uint16_t* x_in;
    uint16_t* x_out;
    uint16_t* xbuf;                // x after layers 0..L-2, xstride elements apart
    uint16_t* actbuf;              // act of layers 0..L-1, M * I elements apart
    uint16_t* gu_out;              // nullable per-layer stage outputs
    uint16_t* down_out;
    uint16_t* xlast;               // nullable second copy of the final x
    uint32_t* sync;
    uint32_t* err;
    int64_t xstride;
    int L;
    int64_t M, H, I;
    // decoder-block chain (style != nullptr): the boundary closes every layer
    const uint16_t* const* style = nullptr;   // host array of L device pointers
    int style_per_row = 0;
    float eps = 0.0f;
    const uint16_t* h_in = nullptr;
    const uint16_t* g_in = nullptr;
    uint16_t* h_out = nullptr;
    uint16_t* g_out = nullptr;
    uint16_t* hbuf = nullptr;                 // nullable per-layer stage output
    double* sspart = nullptr;                 // L x M x H/16 partial sums of squares
};
// Whether a compiled fused configuration covers (M, H, I, L); npa receives
// the gate/up pairs per workgroup.
bool chain_fused_plan(int64_t M, int64_t H, int64_t I, int L, int* npa);
// Whether the fused grid can be resident at once on the current device.
bool chain_fused_resident(int64_t H, int64_t I, int npa);
hipError_t launch_mlp_chain_fused(const ChainLaunch& c, hipStream_t s);

GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K, AType at, WType wt, Epi epi);
size_t gemm_ws_bytes(const GemmPlan& p, int64_t M, int64_t N);
hipError_t launch_gemm(const GemmProblem& pr, hipStream_t s);
// Whether the plan names a compiled kernel configuration (host only).
bool plan_dispatchable(const GemmPlan& p, AType at, WType wt, Epi epi);

}  // namespace vla
