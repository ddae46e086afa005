// Fused gated-MLP chain for gfx950: every layer of the chain in one
// persistent launch.
//
// The chain ("Real-time VLA inference on AMD hardware", sections "How
// FlashRT works", "Merging gate and up" and "Fusing the BF16 decoder
// boundary") is, per layer l,
//   phase A: [g | u] = x_l @ [Wgate_l; Wup_l]^T,  act_l = bf16(gelu(bf16 g) * bf16 u)
//   phase B: x_l+1  = bf16(x_l + bf16(act_l @ Wdown_l^T))
// with scales per output channel.  Replayed as a graph of 2L GEMM launches
// it costs a launch (and its cache flush and invalidate) per phase; here one
// grid of 256 workgroups - one per compute unit, all resident - runs every
// phase, and the workgroups of each 16-row tile meet at a barrier between
// phases.  The weights of a phase
// do not depend on the activations, so each workgroup loads its next
// phase's weight fragments into registers before it waits at the barrier:
// the weight stream overlaps the synchronisation and the activation fetch.
//
// Workgroup w (on XCD w % 8) owns one 16-row activation tile t and one
// column group of each phase, the four workgroups that share a column
// group (different t) sitting on the same XCD, so a weight tile streams
// from HBM once and the others read it from that XCD's L2:
//   phase A: NPA gate/up pairs (16 gate + 16 up channels each), all of K = H;
//   phase B: one 16-column tile of x, all of K = I.
// Eight compute waves split a phase's K range (phase A: WPA = 8 / NPA
// waves per pair) and reduce through LDS in wave order (bitwise
// repeatable); a ninth, control wave issues no weight loads, so it alone
// can poll the barrier counter (gfx9 counts loads and stores in one vmcnt
// that retires in order: a wave with weight loads in flight could not wait
// for a poll without waiting for them).
//
// Coherence without cache maintenance: every intermediate (act_l, x_l+1)
// has its own buffer, written once per launch with device-coherent stores
// (sc1: through to memory) that complete before the workgroup arrives at
// the barrier, and read only after it; a launch starts with no stale copy
// of them in any L2 (the preceding kernel boundary invalidates L2), so
// plain loads that miss fetch the new values and the 32 compute units of
// an XCD then share that XCD's copy.
//
// Every wait is bounded (the host-set poll limit): a workgroup that gives
// up sets the abort word, which releases every other waiter; all
// workgroups then write NaN over their slice of the output, the cause goes
// to the workspace's status word, and every workgroup exits normally.
//
// Decoder-block chain (DEC): the same phases with the decoder boundary
// ("Fusing the BF16 decoder boundary") split over them.  Phase B's epilogue
// forms the gated residual x_l+1 = bf16(x_l + d * g) exactly in fp64 and
// stores, per row and 16-column tile, the fp64 sum of squares of its new
// values; phase A of the next layer stages x_l+1 with the previous layer's
// scale and shift rows and the tile's partial sums, forms 1/rms per row
// and normalizes the staged rows in place before its MFMAs read them.  The
// first layer reads the given h; after the last, one more barrier lets the
// phase-B workgroups write h_out and the next gate for their tiles.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>

#include "gemm_common.h"

namespace vla {
namespace {

using namespace gemm_detail;

constexpr int kCW = 8;                       // compute waves per workgroup
constexpr int kThreads = 64 * (kCW + 1);     // + the control wave
// Sync words (uint32 index into ChainArgs::sync): counter (t, x) of row
// tile t and workgroup class x = w % 8 at (8 t + x) * kSyncStride, the
// abort word and the count of workgroups done on lines of their own.
constexpr int kSyncStride = 32;                 // 128 bytes
constexpr int kSyncAbort = 32 * kSyncStride;
constexpr int kSyncDone = 33 * kSyncStride;

struct ChainArgs {
    const uint8_t* wgu[kMaxChainLayers];
    const float* sgu[kMaxChainLayers];
    const uint8_t* wd[kMaxChainLayers];
    const float* sd[kMaxChainLayers];
    const uint16_t* x_in;     // M x H
    uint16_t* x_out;          // M x H
    uint16_t* xbuf;           // x after layers 0 .. L-2, each M x H, xstride apart
    uint16_t* actbuf;         // act of layers 0 .. L-1, each M x I
    uint16_t* gu_out;         // nullable: L x M x 2I
    uint16_t* down_out;       // nullable: L x M x H (before the residual)
    uint16_t* xlast;          // nullable: a second copy of x after the last layer
    uint32_t* sync;           // barrier counters, abort word, workgroups done (chain_sync_words)
    uint32_t* err;            // status word
    int64_t xstride;          // elements between consecutive xbuf layers
    uint32_t wait_polls;
    int L, M, MT;
    // decoder-block chain: the boundary closes every layer
    const uint16_t* style[kMaxChainLayers];   // per layer: rows of [scale | shift | next gate], 3H each
    const uint16_t* h_in;     // M x H: the first layer's normalized input
    const uint16_t* g_in;     // M x H: the first layer's gate
    uint16_t* h_out;          // M x H
    uint16_t* g_out;          // M x H
    uint16_t* hbuf;           // nullable: h after each layer, L x M x H
    double* sspart;           // per layer, row and 16-column tile: sum of squares of the residual, L x M x H/16
    float eps;
    int style_per_row;
};

// 8-byte store of four bf16 at element `elem` of a buffer of `n` elements
// starting at the wave-uniform `base` (a buffer store: a 32-bit per-lane
// offset, no 64-bit address kept live); the coherent form is written
// through to memory (device-coherent, sc1).
__device__ __forceinline__ void store_b64(uint16_t* base, int64_t n, int64_t elem, uint2 v) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(base, 0, static_cast<int>(n * 2), kRsrcWord3);
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2_t, v), r, static_cast<int>(elem * 2), 0, 0);
}
__device__ __forceinline__ void store_b64_coherent(uint16_t* base, int64_t n, int64_t elem, uint2 v) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(base, 0, static_cast<int>(n * 2), kRsrcWord3);
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2_t, v), r, static_cast<int>(elem * 2), 0, kCpolSC1);
}

template <int SA, int SB, int NPA, bool DEC>
__global__ __launch_bounds__(kThreads) void mlp_chain_kernel(ChainArgs a) {
    constexpr int WPA = kCW / NPA;           // compute waves per gate/up pair
    constexpr int H = SA * WPA * 32;         // phase A depth (hidden size)
    constexpr int I = SB * kCW * 32;         // phase B depth (intermediate size)
    constexpr int RSA = H * 2 + 16;          // LDS row strides (+16 B: bank spread)
    constexpr int RSB = I * 2 + 16;
    constexpr int ACT_A = 16 * RSA, ACT_B = 16 * RSB;
    constexpr int RED_A = kCW * 2 * 1024, RED_B = kCW * 1024;
    // phase A: gate and up scales of the NPA pairs after the reduction area;
    // phase B: the tile's 16 scales and its 16 x 16 residual block
    constexpr int SCL_A = ACT_A + RED_A, SCL_B = ACT_B + RED_B;
    constexpr int END_A0 = SCL_A + 2 * NPA * 64, END_B0 = SCL_B + 64 + 16 * 32;
    // decoder-block chain: phase A also holds the tile's style rows (scale |
    // shift, 4H bytes each) and the rows' 1/rms; phase B the tile's gate
    // block and (after the last layer) 1/rms again
    constexpr int RSS = 4 * H + 16;
    constexpr int G = H / 16;                // 16-column tiles of a row (sum-of-squares partials per row)
    constexpr int SSR = G * 8 + 16;          // LDS row stride of the partials (+16 B: rows on different banks)
    constexpr int SSP = 16 * SSR;            // the tile rows' partials
    constexpr int STY_A = END_A0, INV_A = STY_A + 16 * RSS, SSP_A = INV_A + 128 + 64 * 8;
    constexpr int GB_B = END_B0, INV_B = GB_B + 16 * 32;
    constexpr int END_A = DEC ? SSP_A + SSP : END_A0, END_B = DEC ? INV_B + 128 + 64 * 8 : END_B0;
    constexpr int LDS_BYTES = END_A > END_B ? END_A : END_B;
    static_assert(SSP <= ACT_B, "the last layer's partials fit the free phase-B activation area");
    static_assert(!DEC || 16 * 4 * 8 <= 128 + 64 * 8, "the phase-B row partial quarters fit the 1/rms area");
    static_assert(!DEC || (G <= 64 && G % 4 == 0), "a row's partials in one load and four quarters");
    static_assert(LDS_BYTES <= 160 * 1024, "a phase's activation rows and reduction fit the LDS");
    static_assert(2 * SA + 2 <= 63 && SB + 2 <= 63, "the prefetch counts fit the vmcnt field");
    __shared__ __attribute__((aligned(16))) uint8_t lds[LDS_BYTES];
    __shared__ int s_flag;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int mrow = lane & 15, q = lane >> 4;
    const int w = blockIdx.x, x8 = w & 7, r = w >> 3;
    const int t = r % a.MT;                             // 16-row activation tile
    const int grp = (r / a.MT) * 8 + x8;                // column group (same for the 4 tiles: same XCD)
    const bool va = grp < (I / 16) / NPA;               // owns a phase-A group
    const bool vb = grp < H / 16;                       // owns a phase-B tile
    const int m0 = t * 16;
    const int mrows = min(a.M - m0, 16);                // > 0: the host sizes MT from M
    const bool compute = wave < kCW;

    // phase-A fragment of this wave: pair p, K steps kh*SA .. +SA-1
    const int pa = grp * NPA + (compute ? wave / WPA : 0);
    const int kh = compute ? wave % WPA : 0;
    const bool fin_a = compute && (wave % WPA) == 0;     // finishes pair pa
    // phase-B: tile grp, K steps wave*SB .. +SB-1 (the epilogue waves: fin_b below)
    const int nb = grp * 16 + 4 * q;                     // the lane's 4 output columns in phase B

    u32x2_t wa[SA][2];          // gate / up weight fragments (FP8)
    u32x2_t wb[SB];

    auto xl_ptr = [&](int l) -> const uint16_t* {   // x input of layer l
        return l == 0 ? a.x_in : a.xbuf + (l - 1) * a.xstride;
    };
    // Weight fragments through buffer resources over the layer's packed
    // weight: the per-lane offset (lane * 8) is the same for every load and
    // the fragment's offset is wave-uniform (a scalar operand), so no
    // per-load 64-bit addresses stay live across the layer loop.
    const uint32_t vlane = static_cast<uint32_t>(lane) * 8;
    auto load_wa = [&](int l) __attribute__((always_inline)) {
        constexpr int kst = H / 32;
        const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint8_t*>(a.wgu[l]), 0, 2 * I * H, kRsrcWord3);
        const int gt = va ? pa : 0, ut = (I / 16) + gt;
#pragma unroll
        for (int s = 0; s < SA; ++s) {
            const int ks = kh * SA + s;
            wa[s][0] = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rw, vlane, (gt * kst + ks) * 512, 0));
            wa[s][1] = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rw, vlane, (ut * kst + ks) * 512, 0));
        }
    };
    auto load_wb = [&](int l) __attribute__((always_inline)) {
        constexpr int kst = I / 32;
        const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint8_t*>(a.wd[l]), 0, H * I, kRsrcWord3);
        const int tile = vb ? grp : 0;
#pragma unroll
        for (int s = 0; s < SB; ++s)
            wb[s] = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rw, vlane, (tile * kst + wave * SB + s) * 512, 0));
    };
    // The epilogue inputs go to LDS with the activation rows (direct
    // global -> LDS loads by the control wave), so they hold no registers
    // through the MFMA loop: phase A the NPA pairs' gate and up scales
    // (16 bytes per lane, NPA * 4 lanes each), phase B the tile's 16 scales
    // (4 lanes) and its residual block x_l[m0 .. m0+15][16 columns] (two
    // lanes per row).
    auto stage_epi_a = [&](int l) __attribute__((always_inline)) {
        if (wave == kCW && va) {
            const int n0 = grp * NPA * 16;                          // first gate channel of the group
            const bool up = lane >= NPA * 4;
            const int j = up ? lane - NPA * 4 : lane;
            const uint8_t* src = reinterpret_cast<const uint8_t*>(a.sgu[l] + (up ? I : 0) + n0 + 4 * j);
            if (lane < 2 * NPA * 4)
                __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(lds + SCL_A), 16, 0, 0);
        }
    };
    auto stage_epi_b = [&](int l) __attribute__((always_inline)) {
        if (wave == kCW && vb) {
            const uint8_t* sc = reinterpret_cast<const uint8_t*>(a.sd[l] + grp * 16 + 4 * lane);
            if (lane < 4)
                __builtin_amdgcn_global_load_lds(sc, (__attribute__((address_space(3))) void*)(lds + SCL_B), 16, 0, 0);
            const int row = (lane >> 1) - 2, half = lane & 1;           // lanes 4 .. 35: rows 0 .. 15
            const uint8_t* xr = reinterpret_cast<const uint8_t*>(xl_ptr(l) + static_cast<int64_t>(m0 + row) * H + grp * 16 + 8 * half);
            if (lane >= 4 && lane < 36 && row < mrows)
                __builtin_amdgcn_global_load_lds(xr, (__attribute__((address_space(3))) void*)(lds + SCL_B), 16, 0, 0);
            if constexpr (DEC) {
                // the layer's gate block: the given gate for layer 0, else
                // the previous layer's style (its third block)
                const int grow = lane >> 1, ghalf = lane & 1;            // lanes 0 .. 31: rows 0 .. 15
                const uint16_t* gbase = l == 0 ? a.g_in + static_cast<int64_t>(m0) * H
                                               : a.style[l - 1] + (a.style_per_row ? static_cast<int64_t>(m0) * 3 * H : 0) + 2 * H;
                const int gstride = (l == 0 || a.style_per_row) ? (l == 0 ? H : 3 * H) : 0;   // elements between rows
                const uint32_t goff = static_cast<uint32_t>((grow * gstride + grp * 16 + 8 * ghalf) * 2);
                if (lane < 32 && grow < mrows)
                    __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint8_t*>(gbase) + goff,
                                                     (__attribute__((address_space(3))) void*)(lds + GB_B), 16, 0, 0);
            }
        }
    };
    // The control wave loads no weights; giving its copies a value on its
    // path too ends the previous layer's fragments' live ranges at their
    // last use (otherwise they would be carried around the layer loop).
    auto clear_wa = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int s = 0; s < SA; ++s) wa[s][0] = wa[s][1] = u32x2_t{0, 0};
    };
    auto clear_wb = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int s = 0; s < SB; ++s) wb[s] = u32x2_t{0, 0};
    };
    // Stage activation rows m0 .. m0+mrows-1 (RB bytes each) of src into LDS
    // rows of stride RS with direct global -> LDS loads, 1 KiB per wave
    // instruction, shared by all nine waves.
    auto stage_rows = [&](const uint8_t* base, int64_t sstride, int nrows, int RB, int dst, int RS)
                          __attribute__((always_inline)) {
        const int pieces = (RB + 1023) / 1024;
        for (int pc = wave; pc < nrows * pieces; pc += kCW + 1) {
            const int row = pc / pieces, p = pc % pieces;
            const int byte = p * 1024 + lane * 16;
            if (byte < RB) {
                const uint8_t* g = base + (static_cast<int64_t>(row) * sstride + byte);
                __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)(lds + dst + row * RS + p * 1024),
                                                 16, 0, 0);
            }
        }
    };
    auto stage = [&](const uint16_t* src, int RB, int RS) __attribute__((always_inline)) {
        stage_rows(reinterpret_cast<const uint8_t*>(src) + static_cast<int64_t>(m0) * RB, RB, mrows, RB, 0, RS);
    };
    // Barrier number b (0-based) of this workgroup's row-tile group: phase A
    // of tile t reads only rows of tile t of x, which phase B of the same
    // tile wrote, and phase B reads only tile t's rows of act, so the 64-odd
    // workgroups of a tile synchronise among themselves.  Their arrivals
    // spread over eight device-coherent counters (one per w % 8, 128 bytes
    // apart), so no counter takes more than a dozen atomics per barrier; the
    // control wave (no loads in flight) reads the eight counters and the
    // abort word with one load per poll.  Every wave's stores completed
    // before the workgroup barrier that opens it.  Returns false on abort.
    const uint32_t group_count = static_cast<uint32_t>((31 - t) / a.MT + 1);   // workgroups per counter
    uint32_t* const my_ctr = a.sync + (t * 8 + x8) * kSyncStride;
    uint32_t* const abort_word = a.sync + kSyncAbort;
    auto group_barrier = [&](int b) __attribute__((always_inline)) -> bool {
        __builtin_amdgcn_s_barrier();
        if (wave == kCW) {
            if (lane == 0) __hip_atomic_fetch_add(my_ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const uint32_t target = static_cast<uint32_t>(b + 1) * group_count;
            uint32_t* const mine = lane < 8 ? a.sync + (t * 8 + lane) * kSyncStride : abort_word;
            int flag = 1;
            for (uint32_t it = 0;; ++it) {
                const uint32_t v = lane <= 8 ? __hip_atomic_load(mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0u;
                if (__builtin_amdgcn_ballot_w64(lane == 8 && v != 0) != 0) { flag = 0; break; }
                if (__builtin_amdgcn_ballot_w64(lane < 8 && v < target) == 0) break;
                if (it >= a.wait_polls) {
                    if (lane == 0) {
                        __hip_atomic_store(abort_word, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        report_wait_timeout(a.err, kStatusChainBarrier);
                    }
                    flag = 0;
                    break;
                }
            }
            if (lane == 0) s_flag = flag;
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        return s_flag != 0;
    };
    auto lds_barrier = [&]() __attribute__((always_inline)) {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
    };

    // ---- decoder boundary pieces (DEC) ----
    // The style rows (scale | shift) of layer lp for the tile's rows (one
    // shared row when the style is not per row) -> LDS at STY_A.
    auto stage_style = [&](int lp) __attribute__((always_inline)) {
        const uint8_t* base = reinterpret_cast<const uint8_t*>(a.style[lp] + (a.style_per_row ? static_cast<int64_t>(m0) * 3 * H : 0));
        stage_rows(base, static_cast<int64_t>(6) * H, a.style_per_row ? mrows : 1, 4 * H, STY_A, RSS);
    };
    // The G per-tile partial sums of squares of the tile's rows after layer
    // lp's residual update (written by other workgroups in this launch:
    // device-coherent loads) -> LDS at dst, by the control wave.
    auto stage_partials = [&](int lp, int dst) __attribute__((always_inline)) {
        if (wave == kCW) {
            // one load per row (G * 8 <= 512 bytes: lanes 0 .. G/2-1), rows SSR apart in LDS
            const uint8_t* base = reinterpret_cast<const uint8_t*>(a.sspart + (static_cast<int64_t>(lp) * a.M + m0) * G);
            for (int rr = 0; rr < mrows; ++rr)
                if (lane * 16 < G * 8)
                    __builtin_amdgcn_global_load_lds(base + rr * G * 8 + lane * 16,
                                                     (__attribute__((address_space(3))) void*)(lds + dst + rr * SSR), 16, 0,
                                                     kCpolSC1);
        }
    };
    // 1/rms of each staged row from its partials in LDS (src, rows SSR
    // apart), as fp64 values at LDS offset dst: lane 4 rr + k sums quarter k
    // of row rr's G partials in column order, then lane rr adds the four
    // quarters in order (a fixed order: bitwise repeatable).  The quarters
    // pass through LDS at dst + 128, read back by the same wave; fp64
    // shuffles would each cost a round trip through the LDS crossbar.
    auto row_inv = [&](int src, int dst) __attribute__((always_inline)) {
        constexpr int GQ = G / 4;
        const int rr = lane >> 2, k = lane & 3;
        double part = 0.0;
        if (rr < mrows) {
            const double* pp = reinterpret_cast<const double*>(lds + src + rr * SSR) + k * GQ;
#pragma unroll
            for (int j = 0; j < GQ; ++j) part += pp[j];
        }
        double* const quart = reinterpret_cast<double*>(lds + dst + 128);
        quart[lane] = part;
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_wave_barrier();
        if (lane < mrows) {
            const double tot = ((quart[4 * lane] + quart[4 * lane + 1]) + quart[4 * lane + 2]) + quart[4 * lane + 3];
            *reinterpret_cast<double*>(lds + dst + lane * 8) = 1.0 / sqrt(tot / static_cast<double>(H) + static_cast<double>(a.eps));
        }
    };
    // h = bf16(r * (1/rms) * (1 + scale) + shift), fp32, one output value
    auto norm1 = [](float r, float inv, float sc, float sh) __attribute__((always_inline)) {
        return r * inv * (1.0f + sc) + sh;
    };
    // Normalize the staged rows of x (the residual after layer lp) in place:
    // they become h, the next GEMM's input.
    auto normalize = [&](int lp) __attribute__((always_inline)) {
        (void)lp;
        constexpr int C8 = H / 8;                                   // 16-byte chunks per row
        if (!a.style_per_row) {
            // one style row: each compute-wave thread takes one 8-column
            // chunk and the rows 512 / C8 apart, converting the chunk's
            // 1 + scale and shift once (the same fp32 values norm1 forms)
            static_assert((kCW * 64) % C8 == 0, "whole rows per pass of the compute waves");
            if (wave < kCW) {
                const int k8 = tid % C8;
                const u32x4_t sc = *reinterpret_cast<const u32x4_t*>(lds + STY_A + k8 * 16);
                const u32x4_t sh = *reinterpret_cast<const u32x4_t*>(lds + STY_A + 2 * H + k8 * 16);
                float sa[8], sb[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    sa[2 * i] = 1.0f + bf16_to_f32(lo16(sc[i]));
                    sa[2 * i + 1] = 1.0f + bf16_to_f32(hi16(sc[i]));
                    sb[2 * i] = bf16_to_f32(lo16(sh[i]));
                    sb[2 * i + 1] = bf16_to_f32(hi16(sh[i]));
                }
                for (int row = tid / C8; row < mrows; row += kCW * 64 / C8) {
                    u32x4_t rv = *reinterpret_cast<const u32x4_t*>(lds + row * RSA + k8 * 16);
                    const float inv = static_cast<float>(*reinterpret_cast<const double*>(lds + INV_A + row * 8));
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        rv[i] = f32x2_to_bf16x2(bf16_to_f32(lo16(rv[i])) * inv * sa[2 * i] + sb[2 * i],
                                                bf16_to_f32(hi16(rv[i])) * inv * sa[2 * i + 1] + sb[2 * i + 1]);
                    *reinterpret_cast<u32x4_t*>(lds + row * RSA + k8 * 16) = rv;
                }
            }
            return;
        }
        for (int c = tid; wave <= kCW && c < mrows * C8; c += (kCW + 1) * 64) {
            const int row = c / C8, k8 = c % C8;
            const int srow = a.style_per_row ? row : 0;
            u32x4_t rv = *reinterpret_cast<const u32x4_t*>(lds + row * RSA + k8 * 16);
            const u32x4_t sc = *reinterpret_cast<const u32x4_t*>(lds + STY_A + srow * RSS + k8 * 16);
            const u32x4_t sh = *reinterpret_cast<const u32x4_t*>(lds + STY_A + srow * RSS + 2 * H + k8 * 16);
            const float inv = static_cast<float>(*reinterpret_cast<const double*>(lds + INV_A + row * 8));
#pragma unroll
            for (int i = 0; i < 4; ++i)
                rv[i] = f32x2_to_bf16x2(norm1(bf16_to_f32(lo16(rv[i])), inv, bf16_to_f32(lo16(sc[i])), bf16_to_f32(lo16(sh[i]))),
                                        norm1(bf16_to_f32(hi16(rv[i])), inv, bf16_to_f32(hi16(sc[i])), bf16_to_f32(hi16(sh[i]))));
            *reinterpret_cast<u32x4_t*>(lds + row * RSA + k8 * 16) = rv;
        }
    };
    // The staged h rows of layer lp -> hbuf (per-layer stage output).
    auto write_h = [&](int lp) __attribute__((always_inline)) {
        constexpr int C8 = H / 8;
        const __amdgpu_buffer_rsrc_t rh = __builtin_amdgcn_make_buffer_rsrc(
            a.hbuf + (static_cast<int64_t>(lp) * a.M + m0) * H, 0, mrows * H * 2, kRsrcWord3);
        for (int c = tid; wave <= kCW && c < mrows * C8; c += (kCW + 1) * 64) {
            const int row = c / C8, k8 = c % C8;
            __builtin_amdgcn_raw_buffer_store_b128(*reinterpret_cast<const u32x4_t*>(lds + row * RSA + k8 * 16), rh,
                                                   static_cast<uint32_t>((row * H + k8 * 8) * 2), 0, 0);
        }
    };

    auto red_a = reinterpret_cast<f32x4_t(*)[2][64]>(lds + ACT_A);
    auto red_b = reinterpret_cast<f32x4_t(*)[64]>(lds + ACT_B);

    // Activation fragment of step s, read from LDS D steps ahead of its MFMA
    // (bounded live ranges, the LDS latency covered); phase A with 16 steps
    // per wave holds 64 registers of weights and reads 2 ahead.
    constexpr int DA = SA >= 16 ? 2 : 4, DB = 4;
    if (compute) load_wa(0);
    else clear_wa();
    bool ok = true;
    int b = 0;
    // Request a phase's weights (compute waves; the others clear theirs) and
    // leave this wave's earlier stores complete: NL is the number of loads
    // `load` issues.
    auto prefetch_then_wait = [&](auto load, auto clear, auto NL) __attribute__((always_inline)) {
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (DEC) {
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
            __builtin_amdgcn_sched_barrier(0);
            if (compute) load();
            else clear();
        } else if (compute) {
            load();
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(decltype(NL)::value));
        } else {
            clear();
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    for (int l = 0; l < a.L; ++l) {
        const uint16_t* xl = xl_ptr(l);
        uint16_t* act = a.actbuf + static_cast<int64_t>(l) * a.M * I;
        // ---------------- phase A: gate/up GEMM + GELU * up (its weights
        // were requested before the barrier that opens it).  Decoder-block
        // chain: the input is h, the first layer's given, later the staged
        // residual normalized here with the previous layer's style.
        const bool norm_in = DEC && l > 0;
        stage((DEC && l == 0) ? a.h_in : xl, H * 2, RSA);
        stage_epi_a(l);
        if constexpr (DEC) {
            if (norm_in) {
                stage_style(l - 1);
                stage_partials(l - 1, SSP_A);
            }
        }
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        lds_barrier();
        if constexpr (DEC) {
            if (norm_in) {
                if (wave == kCW) row_inv(SSP_A, INV_A);
                lds_barrier();
                normalize(l - 1);
                lds_barrier();
                if (a.hbuf && grp == 0) write_h(l - 1);
            }
        }
        if (compute) {
            f32x4_t acc[2] = {f32x4_t{0, 0, 0, 0}, f32x4_t{0, 0, 0, 0}};
            const uint8_t* arow = lds + mrow * RSA + (kh * SA * 32 + 8 * q) * 2;
            u32x4_t ring[DA];
#pragma unroll
            for (int d = 0; d < DA; ++d)
                if (d < SA) ring[d] = *reinterpret_cast<const u32x4_t*>(arow + d * 64);
#pragma unroll
            for (int s = 0; s < SA; ++s) {
                const u32x4_t bc = ring[s % DA];
                if (s + DA < SA) ring[s % DA] = *reinterpret_cast<const u32x4_t*>(arow + (s + DA) * 64);
                acc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ocp8_to_bf16x8(wa[s][0]), as_bf16x8(bc), acc[0], 0, 0, 0);
                acc[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ocp8_to_bf16x8(wa[s][1]), as_bf16x8(bc), acc[1], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
            red_a[wave][0][lane] = acc[0];
            red_a[wave][1][lane] = acc[1];
        }
        lds_barrier();
        if (fin_a && va) {
            // every partial read first, then summed in wave order
            f32x4_t pg[WPA], pu[WPA];
#pragma unroll
            for (int i = 0; i < WPA; ++i) {
                pg[i] = red_a[wave + i][0][lane];
                pu[i] = red_a[wave + i][1][lane];
            }
            f32x4_t g = pg[0], u = pu[0];
#pragma unroll
            for (int i = 1; i < WPA; ++i) {
                g += pg[i];
                u += pu[i];
            }
            if (mrow < mrows) {
                EpiIn e{};
                const int pl = wave / WPA;                              // pair within the group
                e.s = *reinterpret_cast<const float4*>(lds + SCL_A + 64 * pl + 16 * q);
                e.su = *reinterpret_cast<const float4*>(lds + SCL_A + NPA * 64 + 64 * pl + 16 * q);
                uint2 gq, uq;
                const uint2 o = epi_gelu4(g, u, e, false, gq, uq);
                const int m = m0 + mrow, n = pa * 16 + 4 * q;
                store_b64_coherent(act, static_cast<int64_t>(a.M) * I, static_cast<int64_t>(m) * I + n, o);
                if (a.gu_out) {
                    uint16_t* gu = a.gu_out + static_cast<int64_t>(l) * a.M * 2 * I;
                    store_b64(gu, static_cast<int64_t>(a.M) * 2 * I, static_cast<int64_t>(m) * 2 * I + n, gq);
                    store_b64(gu, static_cast<int64_t>(a.M) * 2 * I, static_cast<int64_t>(m) * 2 * I + I + n, uq);
                }
            }
        }
        // phase B's weights are requested before the barrier (they stream
        // in during it and the staging of act), and this wave's stores are
        // complete before the arrival.  Gated-MLP chain: the loads go out
        // right behind the stores and the wait leaves only them outstanding
        // (vmcnt retires in order); decoder chain: the stores complete
        // first (measured faster there)
        prefetch_then_wait([&] { load_wb(l); }, [&] { clear_wb(); }, std::integral_constant<int, SB>{});
        ok = group_barrier(b++);
        if (!ok) break;
        // ---------------- phase B: down GEMM + residual
        const bool more = l + 1 < a.L;
        stage(act, I * 2, RSB);
        stage_epi_b(l);
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        lds_barrier();
        if (compute) {
            // two accumulators (even and odd steps), so consecutive MFMAs do
            // not wait for each other's result
            f32x4_t acc2[2] = {f32x4_t{0, 0, 0, 0}, f32x4_t{0, 0, 0, 0}};
            const uint8_t* arow = lds + mrow * RSB + (wave * SB * 32 + 8 * q) * 2;
            u32x4_t ring[DB];
#pragma unroll
            for (int d = 0; d < DB; ++d)
                if (d < SB) ring[d] = *reinterpret_cast<const u32x4_t*>(arow + d * 64);
#pragma unroll
            for (int s = 0; s < SB; ++s) {
                const u32x4_t bc = ring[s % DB];
                if (s + DB < SB) ring[s % DB] = *reinterpret_cast<const u32x4_t*>(arow + (s + DB) * 64);
                acc2[s & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ocp8_to_bf16x8(wb[s]), as_bf16x8(bc), acc2[s & 1], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
            red_b[wave][lane] = acc2[0] + acc2[1];
        }
        lds_barrier();
        // the tile's rows split over EPW waves (the 4 lanes of a row stay in
        // one wave), each summing the waves' partials in wave order: the
        // gated-MLP chain uses all compute waves, two rows each, so every
        // wave's few stores go out ahead of its weight loads; the decoder
        // chain's fp64 epilogue stays on wave 0 (every wave would run its
        // whole instruction stream for a few lanes)
        constexpr int EPW = DEC ? 1 : kCW;
        static_assert(16 % EPW == 0 && EPW <= kCW, "whole rows per epilogue wave");
        const bool fin_b = compute && mrow / (16 / EPW) == wave && vb && mrow < mrows;
        if (fin_b) {
            f32x4_t pv[kCW];
#pragma unroll
            for (int i = 0; i < kCW; ++i) pv[i] = red_b[i][lane];
            f32x4_t v = pv[0];
#pragma unroll
            for (int i = 1; i < kCW; ++i) v += pv[i];
            const float4 sdb = *reinterpret_cast<const float4*>(lds + SCL_B + 16 * q);
            const uint2 xres = *reinterpret_cast<const uint2*>(lds + SCL_B + 64 + mrow * 32 + 8 * q);
            const float y0 = v[0] * sdb.x, y1 = v[1] * sdb.y, y2 = v[2] * sdb.z, y3 = v[3] * sdb.w;
            const uint2 y = make_uint2(f32x2_to_bf16x2(y0, y1), f32x2_to_bf16x2(y2, y3));
            uint2 xn;
            if constexpr (DEC) {
                // gated residual bf16(x + y * gate), exact in fp64, rounded once
                const uint2 gt = *reinterpret_cast<const uint2*>(lds + GB_B + mrow * 32 + 8 * q);
                const uint32_t r0 = gated_residual_bf16(xres.x & 0xFFFFu, y.x & 0xFFFFu, gt.x & 0xFFFFu);
                const uint32_t r1 = gated_residual_bf16(xres.x >> 16, y.x >> 16, gt.x >> 16);
                const uint32_t r2 = gated_residual_bf16(xres.y & 0xFFFFu, y.y & 0xFFFFu, gt.y & 0xFFFFu);
                const uint32_t r3 = gated_residual_bf16(xres.y >> 16, y.y >> 16, gt.y >> 16);
                xn = make_uint2(r0 | (r1 << 16), r2 | (r3 << 16));
                // the row's sum of squares over these 16 columns (lanes
                // mrow + 16 q), in one fixed order, as this tile's partial
                double ss = 0.0;
                ss += bf16_f64(r0) * bf16_f64(r0);
                ss += bf16_f64(r1) * bf16_f64(r1);
                ss += bf16_f64(r2) * bf16_f64(r2);
                ss += bf16_f64(r3) * bf16_f64(r3);
                // through LDS (the row's four lanes' values, then summed in
                // q order by lane q == 0): cheaper than shuffle round trips
                double* const sq = reinterpret_cast<double*>(lds + INV_B);       // 16 x 4 doubles, free here
                sq[mrow * 4 + q] = ss;
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                __builtin_amdgcn_wave_barrier();
                const double rs = ((sq[mrow * 4] + sq[mrow * 4 + 1]) + sq[mrow * 4 + 2]) + sq[mrow * 4 + 3];
                if (q == 0) {
                    const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(
                        a.sspart + static_cast<int64_t>(l) * a.M * G, 0, a.M * G * 8, kRsrcWord3);
                    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2_t, rs), rp,
                                                          static_cast<int>(((m0 + mrow) * G + grp) * 8), 0, kCpolSC1);
                }
            } else {
                xn = make_uint2(add_resid2(y.x, xres.x), add_resid2(y.y, xres.y));
            }
            const int64_t e = static_cast<int64_t>(m0 + mrow) * H + nb;
            const int64_t mh = static_cast<int64_t>(a.M) * H;
            if (!more) {
                store_b64(a.x_out, mh, e, xn);
                if (a.xlast) store_b64(a.xlast, mh, e, xn);
            } else {
                store_b64_coherent(a.xbuf + static_cast<int64_t>(l) * a.xstride, mh, e, xn);
            }
            if (a.down_out) store_b64(a.down_out + static_cast<int64_t>(l) * mh, mh, e, y);
        }
        if (!more) {
            if constexpr (DEC) {
                // h and the next gate of the last layer: every partial of
                // the tile's rows is in after one more barrier
                __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
                ok = group_barrier(b++);
                if (ok) {
                    stage_partials(l, 0);
                    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
                    lds_barrier();
                    if (wave == kCW) row_inv(0, INV_B);
                    lds_barrier();
                    if (fin_b) {
                        // this lane's residual values, stored by this wave above (complete)
                        const int64_t mhb = static_cast<int64_t>(a.M) * H * 2;
                        const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(a.x_out, 0, static_cast<int>(mhb), kRsrcWord3);
                        const uint2 xn_keep = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(
                            rx, static_cast<uint32_t>(((m0 + mrow) * H + nb) * 2), 0, 0));
                        const float inv = static_cast<float>(*reinterpret_cast<const double*>(lds + INV_B + mrow * 8));
                        const __amdgpu_buffer_rsrc_t rst = __builtin_amdgcn_make_buffer_rsrc(
                            const_cast<uint16_t*>(a.style[l]), 0, (a.style_per_row ? a.M : 1) * 3 * H * 2, kRsrcWord3);
                        const uint32_t so = static_cast<uint32_t>(((a.style_per_row ? (m0 + mrow) * 3 * H : 0) + nb) * 2);
                        const uint2 sc = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rst, so, 0, 0));
                        const uint2 sh = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rst, so + 2 * H, 0, 0));
                        const uint2 ng = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rst, so + 4 * H, 0, 0));
                        const uint2 hv = make_uint2(
                            f32x2_to_bf16x2(norm1(bf16_to_f32(lo16(xn_keep.x)), inv, bf16_to_f32(lo16(sc.x)), bf16_to_f32(lo16(sh.x))),
                                            norm1(bf16_to_f32(hi16(xn_keep.x)), inv, bf16_to_f32(hi16(sc.x)), bf16_to_f32(hi16(sh.x)))),
                            f32x2_to_bf16x2(norm1(bf16_to_f32(lo16(xn_keep.y)), inv, bf16_to_f32(lo16(sc.y)), bf16_to_f32(lo16(sh.y))),
                                            norm1(bf16_to_f32(hi16(xn_keep.y)), inv, bf16_to_f32(hi16(sc.y)), bf16_to_f32(hi16(sh.y)))));
                        const int64_t e = static_cast<int64_t>(m0 + mrow) * H + nb;
                        const int64_t mh = static_cast<int64_t>(a.M) * H;
                        store_b64(a.h_out, mh, e, hv);
                        store_b64(a.g_out, mh, e, ng);
                        if (a.hbuf) store_b64(a.hbuf + static_cast<int64_t>(l) * mh, mh, e, hv);
                    }
                }
            }
            break;
        }
        // the next layer's phase-A weights are requested the same way
        // (phase B's weights are dead by now: the two phases' fragments
        // never hold registers at once)
        prefetch_then_wait([&] { load_wa(l + 1); }, [&] { clear_wa(); }, std::integral_constant<int, 2 * SA>{});
        ok = group_barrier(b++);
        if (!ok) break;
    }
    if (!ok && wave == 0 && vb && mrow < mrows) {
        // a barrier gave up: this workgroup's slice of the output reads NaN
        const uint2 nan2 = make_uint2(0x7FC07FC0u, 0x7FC07FC0u);
        const int64_t e = static_cast<int64_t>(m0 + mrow) * H + nb;
        store_b64(a.x_out, static_cast<int64_t>(a.M) * H, e, nan2);
        if (a.xlast) store_b64(a.xlast, static_cast<int64_t>(a.M) * H, e, nan2);
        if (DEC) {
            store_b64(a.h_out, static_cast<int64_t>(a.M) * H, e, nan2);
            store_b64(a.g_out, static_cast<int64_t>(a.M) * H, e, nan2);
        }
    }
    // the last workgroup out clears the counters and the abort word for the
    // next launch
    if (wave == kCW && lane == 0) {
        uint32_t* const done = a.sync + kSyncDone;
        if (__hip_atomic_fetch_add(done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == gridDim.x - 1) {
            for (int i = 0; i < 32; ++i) __hip_atomic_store(a.sync + i * kSyncStride, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(abort_word, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// Configurations compiled in: (SA, SB, NPA) = K steps per wave in phase A
// and B, gate/up pairs per workgroup; H = SA * (8 / NPA) * 32, I = SB * 256.
// The decoder shapes (H = 1024, I = 4096) for 1-16, 17-32 and 33-64 rows,
// and H = 256, I = 512 for small cases.
#define VLA_CHAIN_CONFIGS(X) \
    X(4, 16, 1) X(8, 16, 2) X(16, 16, 4) X(1, 2, 1)

template <int SA, int SB, int NPA>
struct ChainCfg {
    static constexpr int H = SA * (kCW / NPA) * 32;
    static constexpr int I = SB * kCW * 32;
};

std::mutex g_occ_mu;
int g_occ_ok[64] = {};   // per device: 0 unknown, 1 resident grid fits, -1 it does not

}  // namespace

bool chain_fused_plan(int64_t M, int64_t H, int64_t I, int L, int* npa_out) {
    if (M < 1 || M > 64 || L < 1 || L > kMaxChainLayers) return false;
    const int MT = static_cast<int>((M + 15) / 16);
    const int64_t pairs = I / 16;
    // smallest power of two of pairs per workgroup that fits the grid
    int npa = 1;
    while (npa < 4 && (pairs / npa) * MT > kChainGrid) npa *= 2;
    const int64_t slots = 8 * (32 / MT);                // column groups the grid covers for every tile
    if ((pairs % npa) != 0 || pairs / npa > slots || H / 16 > slots) return false;
    bool found = false;
#define VLA_CASE(SA_, SB_, NPA_) \
    if (NPA_ == npa && ChainCfg<SA_, SB_, NPA_>::H == H && ChainCfg<SA_, SB_, NPA_>::I == I) found = true;
    VLA_CHAIN_CONFIGS(VLA_CASE)
#undef VLA_CASE
    if (found && npa_out) *npa_out = npa;
    return found;
}

hipError_t launch_mlp_chain_fused(const ChainLaunch& c, hipStream_t s) {
    int npa = 0;
    if (!chain_fused_plan(c.M, c.H, c.I, c.L, &npa)) return hipErrorInvalidValue;
    ChainArgs a{};
    for (int l = 0; l < c.L; ++l) {
        a.wgu[l] = c.wgu[l];
        a.sgu[l] = c.sgu[l];
        a.wd[l] = c.wd[l];
        a.sd[l] = c.sd[l];
    }
    a.x_in = c.x_in; a.x_out = c.x_out; a.xbuf = c.xbuf; a.actbuf = c.actbuf;
    a.gu_out = c.gu_out; a.down_out = c.down_out; a.xlast = c.xlast;
    a.sync = c.sync; a.err = c.err; a.xstride = c.xstride;
    a.wait_polls = wait_polls();
    a.L = c.L; a.M = static_cast<int>(c.M); a.MT = static_cast<int>((c.M + 15) / 16);
    const bool dec = c.style != nullptr;
    if (dec) {
        for (int l = 0; l < c.L; ++l) a.style[l] = c.style[l];
        a.h_in = c.h_in; a.g_in = c.g_in; a.h_out = c.h_out; a.g_out = c.g_out; a.hbuf = c.hbuf;
        a.sspart = c.sspart; a.eps = c.eps; a.style_per_row = c.style_per_row;
    }
#define VLA_CASE(SA_, SB_, NPA_)                                                                                \
    if (NPA_ == npa && ChainCfg<SA_, SB_, NPA_>::H == c.H && ChainCfg<SA_, SB_, NPA_>::I == c.I) {              \
        if (dec) mlp_chain_kernel<SA_, SB_, NPA_, true><<<kChainGrid, kThreads, 0, s>>>(a);                    \
        else mlp_chain_kernel<SA_, SB_, NPA_, false><<<kChainGrid, kThreads, 0, s>>>(a);                       \
        return hipGetLastError();                                                                               \
    }
    VLA_CHAIN_CONFIGS(VLA_CASE)
#undef VLA_CASE
    return hipErrorInvalidValue;
}

// Whether the fused chain's grid can be resident all at once on the current
// device: at least kChainGrid compute units, each able to hold one of its
// workgroups (checked once per device and configuration class).
bool chain_fused_resident(int64_t H, int64_t I, int npa) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return false;
    std::lock_guard<std::mutex> lk(g_occ_mu);
    if (g_occ_ok[dev] == 0) {
        int cus = 0;
        bool ok = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
                  cus >= kChainGrid;
        // every compiled configuration must fit one workgroup per compute unit
#define VLA_CASE(SA_, SB_, NPA_)                                                                                \
    if (ok) {                                                                                                   \
        int n = 0, nd = 0;                                                                                      \
        ok = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, mlp_chain_kernel<SA_, SB_, NPA_, false>, kThreads, \
                                                          0) == hipSuccess && n >= 1 &&                         \
             hipOccupancyMaxActiveBlocksPerMultiprocessor(&nd, mlp_chain_kernel<SA_, SB_, NPA_, true>, kThreads, \
                                                          0) == hipSuccess && nd >= 1;                          \
    }
        VLA_CHAIN_CONFIGS(VLA_CASE)
#undef VLA_CASE
        g_occ_ok[dev] = ok ? 1 : -1;
    }
    (void)H; (void)I; (void)npa;
    return g_occ_ok[dev] == 1;
}

}  // namespace vla
