// C ABI of the library: argument validation, status codes and the
// gated-MLP chain handle (HIP graph capture / replay).  Kernels live in
// codec.hip and gemm.hip; nothing here allocates device memory.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <utility>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <new>
#include <unordered_set>
#include <vector>

#include "vla.h"
#include "vla_internal.h"

namespace {

thread_local char g_err[512] = "";
std::atomic<uint32_t> g_wait_polls{vla::kDefaultWaitPolls};

int fail(int code, const char* fn, const char* fmt, ...) {
    char msg[384];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(msg, sizeof(msg), fmt, ap);
    va_end(ap);
    snprintf(g_err, sizeof(g_err), "%s: %s", fn, msg);
    return code;
}

int hip_fail(const char* fn, const char* what, hipError_t e) {
    return fail(VLA_EHIP, fn, "%s failed: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define REQUIRE_PTR(p)                                                                   \
    do {                                                                                 \
        if ((p) == nullptr) return fail(VLA_EINVAL, fn, "%s is NULL", #p);               \
        if (!aligned16(p)) return fail(VLA_EALIGN, fn, "%s is not 16-byte aligned", #p); \
    } while (0)

#define OPTIONAL_PTR(p)                                                                  \
    do {                                                                                 \
        if ((p) != nullptr && !aligned16(p))                                             \
            return fail(VLA_EALIGN, fn, "%s is not 16-byte aligned", #p);                \
    } while (0)

int check_nk(const char* fn, int64_t N, int64_t K) {
    if (N <= 0 || K <= 0) return fail(VLA_EINVAL, fn, "N=%lld K=%lld must be positive", (long long)N, (long long)K);
    if (N % 16 != 0) return fail(VLA_ESHAPE, fn, "N=%lld is not a multiple of 16", (long long)N);
    if (K % 32 != 0) return fail(VLA_ESHAPE, fn, "K=%lld is not a multiple of 32", (long long)K);
    if (N > (int64_t(1) << 30) || K > (int64_t(1) << 30) || N * K > (int64_t(1) << 40))
        return fail(VLA_ESHAPE, fn, "N=%lld K=%lld too large", (long long)N, (long long)K);
    return VLA_OK;
}

int check_mnk(const char* fn, int64_t M, int64_t N, int64_t K) {
    if (M <= 0) return fail(VLA_EINVAL, fn, "M=%lld must be positive", (long long)M);
    if (M > (int64_t(1) << 24)) return fail(VLA_ESHAPE, fn, "M=%lld too large", (long long)M);
    return check_nk(fn, N, K);
}

int run_gemm(const char* fn, const vla::GemmProblem& pr, size_t ws_bytes, hipStream_t s) {
    const vla::GemmPlan p = vla::plan_gemm(pr.M, pr.N, pr.K, pr.atype, pr.wtype, pr.epi);
    if (!vla::plan_dispatchable(p, pr.atype, pr.wtype, pr.epi))
        return fail(VLA_ESHAPE, fn, "M=%lld N=%lld K=%lld exceeds the kernels' limits (split-K counters, 2 GiB operands)",
                    (long long)pr.M, (long long)pr.N, (long long)pr.K);
    const size_t need = vla::gemm_ws_bytes(p, pr.M, pr.N);
    if (ws_bytes < need)
        return fail(VLA_EWORKSPACE, fn, "workspace %zu bytes < required %zu", ws_bytes, need);
    hipError_t e = vla::launch_gemm(pr, s);
    if (e != hipSuccess) return hip_fail(fn, "kernel launch", e);
    return VLA_OK;
}

}  // namespace

uint32_t vla::wait_polls() { return g_wait_polls.load(std::memory_order_relaxed); }

struct vla_mlp_chain {
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
    int layers = 0;
};

namespace {
std::mutex g_chain_mu;
std::unordered_set<const vla_mlp_chain*> g_chains;

// Chain scratch: GEMM workspace (first, so its status word sits at the
// same offset as in a plain GEMM workspace) | the fused chain's barrier
// words | x | act.  The x and act areas
// hold one buffer per layer for up to kMaxChainLayers layers: the fused
// chain writes every intermediate once per launch (the graph of GEMMs uses
// the first of each).
struct ChainLayout {
    size_t ws_off, sync_off, x_off, act_off, total, ws_bytes, x_stride, act_stride;
};

size_t round256(size_t v) { return (v + 255) / 256 * 256; }

size_t chain_ws_bytes(int64_t M, int64_t H, int64_t I) {
    const auto pg = vla::plan_gemm(M, 2 * I, H, vla::AType::BF16, vla::WType::FP8, vla::Epi::GELU_MUL);
    const auto pd = vla::plan_gemm(M, H, I, vla::AType::BF16, vla::WType::FP8, vla::Epi::PLAIN);
    const size_t a = vla::gemm_ws_bytes(pg, M, 2 * I), b = vla::gemm_ws_bytes(pd, M, H);
    return round256(a > b ? a : b);
}

ChainLayout chain_layout(int64_t M, int64_t H, int64_t I) {
    ChainLayout c{};
    c.ws_off = 0;
    c.ws_bytes = chain_ws_bytes(M, H, I);
    c.x_stride = round256(static_cast<size_t>(M) * H * 2);
    c.act_stride = round256(static_cast<size_t>(M) * I * 2);
    c.sync_off = c.ws_bytes;
    c.x_off = c.sync_off + vla::kChainSyncBytes;
    c.act_off = c.x_off + (vla::kMaxChainLayers - 1) * c.x_stride;
    c.total = c.act_off + vla::kMaxChainLayers * c.act_stride;
    return c;
}

int check_chain(const char* fn, const uint8_t* const* wgu, const float* const* sgu,
                const uint8_t* const* wd, const float* const* sd, const uint16_t* x_in,
                uint16_t* x_out, void* scratch, size_t scratch_bytes, int L, int64_t M,
                int64_t H, int64_t I) {
    if (!wgu || !sgu || !wd || !sd) return fail(VLA_EINVAL, fn, "weight pointer arrays must not be NULL");
    if (L <= 0) return fail(VLA_EINVAL, fn, "L=%d must be positive", L);
    if (int rc = check_mnk(fn, M, 2 * I, H)) return rc;
    if (int rc = check_nk(fn, H, I)) return rc;
    if (I % 16 != 0) return fail(VLA_ESHAPE, fn, "I=%lld is not a multiple of 16", (long long)I);
    REQUIRE_PTR(x_in);
    REQUIRE_PTR(x_out);
    REQUIRE_PTR(scratch);
    for (int l = 0; l < L; ++l) {
        if (!wgu[l] || !sgu[l] || !wd[l] || !sd[l]) return fail(VLA_EINVAL, fn, "layer %d has a NULL weight", l);
        if (!aligned16(wgu[l]) || !aligned16(sgu[l]) || !aligned16(wd[l]) || !aligned16(sd[l]))
            return fail(VLA_EALIGN, fn, "layer %d weight not 16-byte aligned", l);
    }
    const ChainLayout c = chain_layout(M, H, I);
    if (scratch_bytes < c.total)
        return fail(VLA_EWORKSPACE, fn, "scratch %zu bytes < required %zu", scratch_bytes, c.total);
    const uint8_t* xo = reinterpret_cast<const uint8_t*>(x_out);
    const uint8_t* xi = reinterpret_cast<const uint8_t*>(x_in);
    const uint8_t* sc = static_cast<const uint8_t*>(scratch);
    const size_t xb = static_cast<size_t>(M) * H * 2;
    auto overlap = [](const uint8_t* a, size_t na, const uint8_t* b, size_t nb) { return a < b + nb && b < a + na; };
    if (overlap(xo, xb, xi, xb) || overlap(xo, xb, sc, c.total))
        return fail(VLA_EINVAL, fn, "x_out overlaps x_in or scratch");
    return VLA_OK;
}

// Per-layer stage outputs of the gated-MLP chain (each nullable): the merged
// gate/up GEMM result [g | u] (L x M x 2I), the activation (L x M x I), the
// down GEMM result before the residual add (L x M x H) and x after each
// layer (L x M x H).
struct ChainStages {
    uint16_t* gu = nullptr;
    uint16_t* act = nullptr;
    uint16_t* down = nullptr;
    uint16_t* x = nullptr;
};

int enqueue_chain(const char* fn, const uint8_t* const* wgu, const float* const* sgu,
                  const uint8_t* const* wd, const float* const* sd, const uint16_t* x_in,
                  uint16_t* x_out, void* scratch, int L, int64_t M, int64_t H, int64_t I,
                  const ChainStages& st, hipStream_t s) {
    const ChainLayout c = chain_layout(M, H, I);
    uint8_t* base = static_cast<uint8_t*>(scratch);
    uint16_t* xbuf = reinterpret_cast<uint16_t*>(base + c.x_off);
    uint16_t* act_buf = reinterpret_cast<uint16_t*>(base + c.act_off);
    void* ws = base + c.ws_off;
    const size_t mh = static_cast<size_t>(M) * H, mi = static_cast<size_t>(M) * I;
    // The fused launch writes each layer's intermediates to their own
    // buffers; no two layers' buffers may share a cache line (a line read for
    // one layer would hold the next layer's bytes before they are written),
    // so it needs 256-byte aligned buffers (every compiled configuration has
    // per-layer sizes that are multiples of 256 bytes).
    auto a256 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 255u) == 0; };
    const bool aligned = a256(scratch) && a256(st.gu) && a256(st.act) && a256(st.down) && a256(st.x) &&
                         (mh * 2) % 256 == 0 && (mi * 2) % 256 == 0;
    int npa = 0;
    if (aligned && vla::chain_fused_plan(M, H, I, L, &npa) && vla::chain_fused_resident(H, I, npa)) {
        // one persistent launch for every layer
        vla::ChainLaunch cl{};
        cl.wgu = wgu; cl.sgu = sgu; cl.wd = wd; cl.sd = sd;
        cl.x_in = x_in; cl.x_out = x_out;
        cl.xbuf = st.x ? st.x : xbuf;
        cl.xstride = st.x ? static_cast<int64_t>(mh) : static_cast<int64_t>(c.x_stride / 2);
        cl.xlast = st.x ? st.x + (L - 1) * mh : nullptr;
        cl.actbuf = st.act ? st.act : act_buf;
        // the kernel places act_l at actbuf + l * M * I; the scratch pads
        // each to 256 bytes, which M * I * 2 already is when M * I % 128 == 0
        cl.gu_out = st.gu; cl.down_out = st.down;
        cl.sync = reinterpret_cast<uint32_t*>(base + c.sync_off);
        cl.err = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(ws) + vla::kStatusOffset);
        cl.L = L; cl.M = M; cl.H = H; cl.I = I;
        hipError_t e = vla::launch_mlp_chain_fused(cl, s);
        return e == hipSuccess ? VLA_OK : hip_fail(fn, "fused chain launch", e);
    }
    const uint16_t* x = x_in;
    for (int l = 0; l < L; ++l) {
        uint16_t* act = st.act ? st.act + l * mi : act_buf;
        vla::GemmProblem g{};
        g.A = x; g.W = wgu[l]; g.s_w = sgu[l]; g.Y = act; g.ws = ws;
        g.gu = st.gu ? st.gu + l * 2 * mi : nullptr;
        g.M = M; g.N = 2 * I; g.K = H;
        g.atype = vla::AType::BF16; g.wtype = vla::WType::FP8; g.epi = vla::Epi::GELU_MUL;
        if (int rc = run_gemm(fn, g, c.ws_bytes, s)) return rc;
        // with per-layer x outputs every layer writes its own slot (the
        // last one is then copied to x_out); else x alternates between
        // scratch and x_out
        uint16_t* y = st.x ? st.x + l * mh : ((l == L - 1) ? x_out : xbuf);
        vla::GemmProblem d{};
        d.A = act; d.W = wd[l]; d.s_w = sd[l]; d.resid = x; d.Y = y; d.ws = ws;
        d.ypre = st.down ? st.down + l * mh : nullptr;
        d.M = M; d.N = H; d.K = I;
        d.atype = vla::AType::BF16; d.wtype = vla::WType::FP8; d.epi = vla::Epi::PLAIN;
        if (int rc = run_gemm(fn, d, c.ws_bytes, s)) return rc;
        x = y;
    }
    if (st.x) {
        hipError_t e = hipMemcpyAsync(x_out, x, mh * 2, hipMemcpyDeviceToDevice, s);
        if (e != hipSuccess) return hip_fail(fn, "hipMemcpyAsync", e);
    }
    return VLA_OK;
}

// Decoder-block chain scratch, laid out for both paths.  Graph of launches:
// GEMM workspace | (barrier words) | x | h | gate (two, alternating) | down
// output | act.
// Single launch: the gated-MLP chain's layout (GEMM workspace | barrier
// words | x per layer | act per layer) followed by the per-layer partial
// sums of squares (L x M x H/16 fp64).
struct DecoderLayout {
    size_t ws_off, x_off, h_off, g_off[2], d_off, act_off, ssp_off, total, ws_bytes;
};

DecoderLayout decoder_layout(int64_t M, int64_t H, int64_t I) {
    const size_t mh = round256(static_cast<size_t>(M) * H * 2);
    DecoderLayout c{};
    c.ws_off = 0;
    c.ws_bytes = chain_ws_bytes(M, H, I);
    // the graph path's buffers start past the single launch's barrier
    // words, which must stay zero between launches
    c.x_off = c.ws_bytes + vla::kChainSyncBytes;
    c.h_off = c.x_off + mh;
    c.g_off[0] = c.x_off + 2 * mh;
    c.g_off[1] = c.x_off + 3 * mh;
    c.d_off = c.x_off + 4 * mh;
    c.act_off = c.x_off + 5 * mh;
    const size_t graph_total = c.act_off + round256(static_cast<size_t>(M) * I * 2);
    const ChainLayout f = chain_layout(M, H, I);
    c.ssp_off = f.total;
    const size_t fused_total = c.ssp_off + round256(static_cast<size_t>(vla::kMaxChainLayers) * M * (H / 16) * 8);
    c.total = graph_total > fused_total ? graph_total : fused_total;
    return c;
}

int check_decoder(const char* fn, const uint8_t* const* wgu, const float* const* sgu, const uint8_t* const* wd,
                  const float* const* sd, const uint16_t* const* style, int style_per_row, float eps,
                  const uint16_t* x_in, const uint16_t* h_in, const uint16_t* gate_in, uint16_t* x_out,
                  uint16_t* h_out, uint16_t* gate_out, void* scratch, size_t scratch_bytes, int L, int64_t M,
                  int64_t H, int64_t I) {
    if (!wgu || !sgu || !wd || !sd || !style) return fail(VLA_EINVAL, fn, "pointer arrays must not be NULL");
    if (L <= 0) return fail(VLA_EINVAL, fn, "L=%d must be positive", L);
    if (int rc = check_mnk(fn, M, 2 * I, H)) return rc;
    if (int rc = check_nk(fn, H, I)) return rc;
    if (I % 16 != 0) return fail(VLA_ESHAPE, fn, "I=%lld is not a multiple of 16", (long long)I);
    if (!vla::boundary_width_ok(H)) return fail(VLA_ESHAPE, fn, "H=%lld must be at most 8192", (long long)H);
    if (!std::isfinite(eps) || eps < 0.0f) return fail(VLA_EINVAL, fn, "eps must be finite and >= 0");
    REQUIRE_PTR(x_in);
    REQUIRE_PTR(h_in);
    REQUIRE_PTR(gate_in);
    REQUIRE_PTR(x_out);
    REQUIRE_PTR(h_out);
    REQUIRE_PTR(gate_out);
    REQUIRE_PTR(scratch);
    for (int l = 0; l < L; ++l) {
        if (!wgu[l] || !sgu[l] || !wd[l] || !sd[l] || !style[l]) return fail(VLA_EINVAL, fn, "layer %d has a NULL pointer", l);
        if (!aligned16(wgu[l]) || !aligned16(sgu[l]) || !aligned16(wd[l]) || !aligned16(sd[l]) || !aligned16(style[l]))
            return fail(VLA_EALIGN, fn, "layer %d pointer not 16-byte aligned", l);
    }
    const DecoderLayout c = decoder_layout(M, H, I);
    if (scratch_bytes < c.total)
        return fail(VLA_EWORKSPACE, fn, "scratch %zu bytes < required %zu", scratch_bytes, c.total);
    const size_t mat = static_cast<size_t>(M) * H * 2;
    const size_t sty = static_cast<size_t>(style_per_row ? M : 1) * 3 * H * 2;
    auto overlap = [](const void* x, size_t nx, const void* y, size_t ny) {
        const uint8_t *a = static_cast<const uint8_t*>(x), *b = static_cast<const uint8_t*>(y);
        return a < b + ny && b < a + nx;
    };
    const void* outs[3] = {x_out, h_out, gate_out};
    const void* ins[3] = {x_in, h_in, gate_in};
    for (int i = 0; i < 3; ++i) {
        for (int j = i + 1; j < 3; ++j)
            if (overlap(outs[i], mat, outs[j], mat)) return fail(VLA_EINVAL, fn, "outputs %d and %d overlap", i, j);
        for (int j = 0; j < 3; ++j)
            if (overlap(outs[i], mat, ins[j], mat)) return fail(VLA_EINVAL, fn, "output %d overlaps input %d", i, j);
        if (overlap(outs[i], mat, scratch, c.total)) return fail(VLA_EINVAL, fn, "output %d overlaps scratch", i);
        for (int l = 0; l < L; ++l)
            if (overlap(outs[i], mat, style[l], sty)) return fail(VLA_EINVAL, fn, "output %d overlaps style %d", i, l);
    }
    for (int j = 0; j < 3; ++j)
        if (overlap(ins[j], mat, scratch, c.total)) return fail(VLA_EINVAL, fn, "input %d overlaps scratch", j);
    return VLA_OK;
}

// Per-layer stage outputs of the decoder-block chain (each nullable): those
// of the gated-MLP chain plus h after each layer (L x M x H).
struct DecoderStages {
    ChainStages mlp;
    uint16_t* h = nullptr;
};

// Whether the decoder-block chain of this shape takes the single launch
// (given aligned buffers): the gated-MLP chain's conditions, H at most 1024
// (a row's partial sums of squares fit one load), and, with a style row per
// activation row, at most one 16-row tile - beyond that every workgroup
// stages 16 rows of scale and shift per layer and the graph of launches
// measured faster.
bool decoder_fused(int64_t M, int64_t H, int64_t I, int L, int style_per_row) {
    int npa = 0;
    return H <= 1024 && !(style_per_row && M > 16) && vla::chain_fused_plan(M, H, I, L, &npa) &&
           vla::chain_fused_resident(H, I, npa);
}

int enqueue_decoder(const char* fn, const uint8_t* const* wgu, const float* const* sgu, const uint8_t* const* wd,
                    const float* const* sd, const uint16_t* const* style, int style_per_row, float eps,
                    const uint16_t* x_in, const uint16_t* h_in, const uint16_t* gate_in, uint16_t* x_out,
                    uint16_t* h_out, uint16_t* gate_out, void* scratch, int L, int64_t M, int64_t H, int64_t I,
                    const DecoderStages& st, hipStream_t s) {
    const DecoderLayout c = decoder_layout(M, H, I);
    uint8_t* base = static_cast<uint8_t*>(scratch);
    const size_t mh = static_cast<size_t>(M) * H, mi = static_cast<size_t>(M) * I;
    // One persistent launch for every layer (the gated-MLP chain's kernel
    // with the boundary after each layer) where decoder_fused allows it and
    // every buffer it writes is 256-byte aligned.
    auto a256 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 255u) == 0; };
    const ChainStages& ms = st.mlp;
    const bool aligned = a256(scratch) && a256(ms.gu) && a256(ms.act) && a256(ms.down) && a256(ms.x) && a256(st.h) &&
                         (mh * 2) % 256 == 0 && (mi * 2) % 256 == 0;
    if (aligned && decoder_fused(M, H, I, L, style_per_row)) {
        const ChainLayout f = chain_layout(M, H, I);
        vla::ChainLaunch cl{};
        cl.wgu = wgu; cl.sgu = sgu; cl.wd = wd; cl.sd = sd;
        cl.x_in = x_in; cl.x_out = x_out;
        cl.xbuf = ms.x ? ms.x : reinterpret_cast<uint16_t*>(base + f.x_off);
        cl.xstride = ms.x ? static_cast<int64_t>(mh) : static_cast<int64_t>(f.x_stride / 2);
        cl.xlast = ms.x ? ms.x + (L - 1) * mh : nullptr;
        cl.actbuf = ms.act ? ms.act : reinterpret_cast<uint16_t*>(base + f.act_off);
        cl.gu_out = ms.gu; cl.down_out = ms.down;
        cl.sync = reinterpret_cast<uint32_t*>(base + f.sync_off);
        cl.err = reinterpret_cast<uint32_t*>(base + c.ws_off + vla::kStatusOffset);
        cl.L = L; cl.M = M; cl.H = H; cl.I = I;
        cl.style = style; cl.style_per_row = style_per_row ? 1 : 0; cl.eps = eps;
        cl.h_in = h_in; cl.g_in = gate_in; cl.h_out = h_out; cl.g_out = gate_out; cl.hbuf = st.h;
        cl.sspart = reinterpret_cast<double*>(base + c.ssp_off);
        hipError_t e = vla::launch_mlp_chain_fused(cl, s);
        return e == hipSuccess ? VLA_OK : hip_fail(fn, "fused decoder chain launch", e);
    }
    uint16_t* xs = reinterpret_cast<uint16_t*>(base + c.x_off);
    uint16_t* hs = reinterpret_cast<uint16_t*>(base + c.h_off);
    uint16_t* gs[2] = {reinterpret_cast<uint16_t*>(base + c.g_off[0]), reinterpret_cast<uint16_t*>(base + c.g_off[1])};
    uint16_t* dbuf = reinterpret_cast<uint16_t*>(base + c.d_off);
    uint16_t* act = reinterpret_cast<uint16_t*>(base + c.act_off);
    void* ws = base + c.ws_off;
    const uint16_t *x = x_in, *h = h_in, *g = gate_in;
    for (int l = 0; l < L; ++l) {
        uint16_t* actl = ms.act ? ms.act + l * mi : act;
        uint16_t* dl = ms.down ? ms.down + l * mh : dbuf;
        vla::GemmProblem gp{};
        gp.A = h; gp.W = wgu[l]; gp.s_w = sgu[l]; gp.Y = actl; gp.ws = ws;
        gp.gu = ms.gu ? ms.gu + l * 2 * mi : nullptr;
        gp.M = M; gp.N = 2 * I; gp.K = H;
        gp.atype = vla::AType::BF16; gp.wtype = vla::WType::FP8; gp.epi = vla::Epi::GELU_MUL;
        if (int rc = run_gemm(fn, gp, c.ws_bytes, s)) return rc;
        vla::GemmProblem dp{};
        dp.A = actl; dp.W = wd[l]; dp.s_w = sd[l]; dp.Y = dl; dp.ws = ws;
        dp.M = M; dp.N = H; dp.K = I;
        dp.atype = vla::AType::BF16; dp.wtype = vla::WType::FP8; dp.epi = vla::Epi::PLAIN;
        if (int rc = run_gemm(fn, dp, c.ws_bytes, s)) return rc;
        const bool last = l == L - 1;
        // per-layer stage buffers when given (the last ones then copied
        // out), else x and h in place from the second layer on (this
        // layer's GEMM has read h already) and the gate alternating
        uint16_t* xo = ms.x ? ms.x + l * mh : (last ? x_out : xs);
        uint16_t* ho = st.h ? st.h + l * mh : (last ? h_out : hs);
        uint16_t* go = last ? gate_out : gs[l & 1];
        hipError_t e = vla::launch_gate_residual_ada_norm(x, dl, g, style[l], style_per_row ? 1 : 0, eps, xo, ho, go,
                                                          M, H, s);
        if (e != hipSuccess) return hip_fail(fn, "boundary launch", e);
        x = xo; h = ho; g = go;
    }
    for (auto [dst, src] : {std::pair<uint16_t*, const uint16_t*>{x_out, ms.x ? x : nullptr},
                            std::pair<uint16_t*, const uint16_t*>{h_out, st.h ? h : nullptr}}) {
        if (!src) continue;
        hipError_t e = hipMemcpyAsync(dst, src, mh * 2, hipMemcpyDeviceToDevice, s);
        if (e != hipSuccess) return hip_fail(fn, "hipMemcpyAsync", e);
    }
    return VLA_OK;
}

// Capture `enqueue` on capture_stream into a graph and instantiate it.
template <class F>
int capture_chain(const char* fn, void* capture_stream, int L, vla_mlp_chain** out, F&& enqueue) {
    hipStream_t s = static_cast<hipStream_t>(capture_stream);
    hipError_t e = hipStreamBeginCapture(s, hipStreamCaptureModeRelaxed);
    if (e != hipSuccess) return hip_fail(fn, "hipStreamBeginCapture", e);
    int rc = enqueue(s);
    hipGraph_t graph = nullptr;
    e = hipStreamEndCapture(s, &graph);
    if (rc != VLA_OK) {
        if (graph) (void)hipGraphDestroy(graph);
        return rc;
    }
    if (e != hipSuccess) return hip_fail(fn, "hipStreamEndCapture", e);
    hipGraphExec_t exec = nullptr;
    e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
    if (e != hipSuccess) {
        (void)hipGraphDestroy(graph);
        return hip_fail(fn, "hipGraphInstantiate", e);
    }
    vla_mlp_chain* h = new (std::nothrow) vla_mlp_chain;
    if (!h) {
        (void)hipGraphExecDestroy(exec);
        (void)hipGraphDestroy(graph);
        return fail(VLA_EINVAL, fn, "out of host memory");
    }
    h->graph = graph;
    h->exec = exec;
    h->layers = L;
    {
        std::lock_guard<std::mutex> lk(g_chain_mu);
        g_chains.insert(h);
    }
    *out = h;
    return VLA_OK;
}

}  // namespace

extern "C" {

const char* vla_status_string(int status) {
    switch (status) {
        case VLA_OK: return "ok";
        case VLA_EINVAL: return "invalid argument";
        case VLA_ESHAPE: return "unsupported shape";
        case VLA_EALIGN: return "misaligned pointer";
        case VLA_EWORKSPACE: return "workspace too small";
        case VLA_EHIP: return "HIP error";
        case VLA_ESTATE: return "invalid handle state";
        default: return "unknown status";
    }
}

const char* vla_last_error(void) { return g_err; }

void vla_set_wait_limit(uint32_t polls) {
    g_wait_polls.store(polls == 0 ? vla::kDefaultWaitPolls : polls, std::memory_order_relaxed);
}

int vla_workspace_status(void* ws, void* stream) {
    const char* fn = "vla_workspace_status";
    REQUIRE_PTR(ws);
    hipStream_t s = static_cast<hipStream_t>(stream);
    uint32_t* word = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(ws) + vla::kStatusOffset);
    uint32_t v = 0;
    static const uint32_t zero = 0;
    hipError_t e = hipMemcpyAsync(&v, word, 4, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e == hipSuccess && v != 0) e = hipMemcpyAsync(word, &zero, 4, hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(fn, "status word copy", e);
    if (v == 0) return VLA_OK;
    return fail(VLA_EHIP, fn, "an in-kernel wait gave up and left output unwritten (status 0x%x:%s%s)", v,
                (v & vla::kStatusWideSplitK) ? " wide split-K partials" : "",
                (v & vla::kStatusChainBarrier) ? " fused chain phase barrier" : "");
}

size_t vla_packed_bytes(int64_t N, int64_t K, int wfmt) {
    if (N <= 0 || K <= 0) return 0;
    if (wfmt == VLA_WFMT_MXFP4)
        return static_cast<size_t>(N) * K / 2 + static_cast<size_t>(N) * vla::mxfp4_scale_row_bytes(K);
    return static_cast<size_t>(N) * static_cast<size_t>(K) * (wfmt == VLA_WFMT_BF16 ? 2 : 1);
}

int vla_quantize_pack(const float* W, void* Wq, float* scales, int64_t N, int64_t K, int wfmt,
                      int layout, void* stream) {
    const char* fn = "vla_quantize_pack";
    if (wfmt < VLA_WFMT_BF16 || wfmt > VLA_WFMT_MXFP4) return fail(VLA_EINVAL, fn, "unknown wfmt %d", wfmt);
    if (layout != VLA_LAYOUT_ROWMAJOR && layout != VLA_LAYOUT_MFMA) return fail(VLA_EINVAL, fn, "unknown layout %d", layout);
    if (int rc = check_nk(fn, N, K)) return rc;
    REQUIRE_PTR(W);
    REQUIRE_PTR(Wq);
    if (wfmt == VLA_WFMT_MXFP4) {
        if (scales != nullptr) return fail(VLA_EINVAL, fn, "scales must be NULL for MXFP4 (they are packed into Wq)");
        if (layout != VLA_LAYOUT_MFMA) return fail(VLA_EINVAL, fn, "MXFP4 is packed in VLA_LAYOUT_MFMA only");
        hipError_t e = vla::launch_mxfp4_quantize_pack(W, static_cast<uint8_t*>(Wq), N, K, static_cast<hipStream_t>(stream));
        return e == hipSuccess ? VLA_OK : hip_fail(fn, "kernel launch", e);
    }
    if (wfmt == VLA_WFMT_BF16) {
        if (scales != nullptr) return fail(VLA_EINVAL, fn, "scales must be NULL for BF16");
    } else {
        REQUIRE_PTR(scales);
    }
    hipError_t e = vla::launch_quantize_pack(W, Wq, scales, N, K, wfmt, layout, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? VLA_OK : hip_fail(fn, "kernel launch", e);
}

int vla_pack_fp8(const uint8_t* q_rowmajor, uint8_t* q_packed, int64_t N, int64_t K, void* stream) {
    const char* fn = "vla_pack_fp8";
    if (int rc = check_nk(fn, N, K)) return rc;
    REQUIRE_PTR(q_rowmajor);
    REQUIRE_PTR(q_packed);
    const size_t nb = static_cast<size_t>(N) * K;
    const uint8_t *a = q_rowmajor, *b = q_packed;
    if (a < b + nb && b < a + nb) return fail(VLA_EINVAL, fn, "input and output overlap");
    hipError_t e = vla::launch_pack_fp8(q_rowmajor, q_packed, N, K, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? VLA_OK : hip_fail(fn, "kernel launch", e);
}

int vla_reencode_fnuz_to_ocp(const uint8_t* q_fnuz, const float* s_fnuz, uint8_t* q_ocp,
                             float* s_ocp, int64_t N, int64_t K, int layout, void* stream) {
    const char* fn = "vla_reencode_fnuz_to_ocp";
    if (layout != VLA_LAYOUT_ROWMAJOR && layout != VLA_LAYOUT_MFMA) return fail(VLA_EINVAL, fn, "unknown layout %d", layout);
    if (int rc = check_nk(fn, N, K)) return rc;
    REQUIRE_PTR(q_fnuz);
    REQUIRE_PTR(s_fnuz);
    REQUIRE_PTR(q_ocp);
    REQUIRE_PTR(s_ocp);
    const size_t nb = static_cast<size_t>(N) * K;
    auto partial = [](const void* x, const void* y, size_t n) {
        const uint8_t *a = static_cast<const uint8_t*>(x), *b = static_cast<const uint8_t*>(y);
        return a != b && a < b + n && b < a + n;
    };
    if (partial(q_fnuz, q_ocp, nb) || partial(s_fnuz, s_ocp, static_cast<size_t>(N) * 4))
        return fail(VLA_EINVAL, fn, "outputs partially overlap inputs");
    hipError_t e = vla::launch_reencode(q_fnuz, s_fnuz, q_ocp, s_ocp, N, K, layout, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? VLA_OK : hip_fail(fn, "kernel launch", e);
}

size_t vla_quantize_act_workspace_bytes(int64_t M, int64_t K) { return vla::quantize_act_ws_bytes(M, K); }

int vla_quantize_act(const uint16_t* A, uint8_t* qa, float* s_a, void* ws, size_t ws_bytes,
                     int64_t M, int64_t K, void* stream) {
    const char* fn = "vla_quantize_act";
    if (int rc = check_mnk(fn, M, 16, K)) return rc;
    if (M * K > (int64_t(1) << 40)) return fail(VLA_ESHAPE, fn, "M*K=%lld too large", (long long)(M * K));
    REQUIRE_PTR(A);
    REQUIRE_PTR(qa);
    REQUIRE_PTR(s_a);
    REQUIRE_PTR(ws);
    const size_t need = vla::quantize_act_ws_bytes(M, K);
    if (ws_bytes < need) return fail(VLA_EWORKSPACE, fn, "workspace %zu bytes < required %zu", ws_bytes, need);
    hipError_t e = vla::launch_quantize_act(A, qa, s_a, ws, M, K, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? VLA_OK : hip_fail(fn, "kernel launch", e);
}

int vla_quantize_act_static(const uint16_t* A, const float* s_a, uint8_t* qa, int64_t M, int64_t K, void* stream) {
    const char* fn = "vla_quantize_act_static";
    if (int rc = check_mnk(fn, M, 16, K)) return rc;
    if (M * K > (int64_t(1) << 40)) return fail(VLA_ESHAPE, fn, "M*K=%lld too large", (long long)(M * K));
    REQUIRE_PTR(A);
    REQUIRE_PTR(s_a);
    REQUIRE_PTR(qa);
    hipError_t e = vla::launch_quantize_act_static(A, s_a, qa, M, K, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? VLA_OK : hip_fail(fn, "kernel launch", e);
}

int vla_gate_residual_ada_norm(const uint16_t* residual, const uint16_t* out, const uint16_t* gate,
                               const uint16_t* style, int style_per_row, float eps, uint16_t* residual_out,
                               uint16_t* normalized, uint16_t* next_gate, int64_t M, int64_t D, void* stream) {
    const char* fn = "vla_gate_residual_ada_norm";
    REQUIRE_PTR(residual);
    REQUIRE_PTR(out);
    REQUIRE_PTR(gate);
    REQUIRE_PTR(style);
    REQUIRE_PTR(residual_out);
    REQUIRE_PTR(normalized);
    OPTIONAL_PTR(next_gate);
    if (M <= 0 || D <= 0) return fail(VLA_EINVAL, fn, "M=%lld D=%lld must be positive", (long long)M, (long long)D);
    if (M > (int64_t(1) << 24)) return fail(VLA_ESHAPE, fn, "M=%lld too large", (long long)M);
    if (!vla::boundary_width_ok(D)) return fail(VLA_ESHAPE, fn, "D=%lld must be a multiple of 4, at most 8192", (long long)D);
    if (!std::isfinite(eps) || eps < 0.0f) return fail(VLA_EINVAL, fn, "eps must be finite and >= 0");
    // residual_out may be residual itself; no other output may overlap anything
    const size_t mat = static_cast<size_t>(M) * D * 2;
    const size_t sty = static_cast<size_t>(style_per_row ? M : 1) * 3 * D * 2;
    struct Range { const void* p; size_t n; };
    const Range ins[4] = {{residual, mat}, {out, mat}, {gate, mat}, {style, sty}};
    const Range outs[3] = {{residual_out, mat}, {normalized, mat}, {next_gate, next_gate ? mat : 0}};
    auto overlap = [](const Range& x, const Range& y) {
        const uint8_t *a = static_cast<const uint8_t*>(x.p), *b = static_cast<const uint8_t*>(y.p);
        return x.n && y.n && a < b + y.n && b < a + x.n;
    };
    for (int i = 0; i < 3; ++i) {
        for (int j = 0; j < 4; ++j)
            if (overlap(outs[i], ins[j]) && !(i == 0 && j == 0 && outs[i].p == ins[j].p))
                return fail(VLA_EINVAL, fn, "output %d overlaps input %d", i, j);
        for (int j = i + 1; j < 3; ++j)
            if (overlap(outs[i], outs[j])) return fail(VLA_EINVAL, fn, "outputs %d and %d overlap", i, j);
    }
    hipError_t e = vla::launch_gate_residual_ada_norm(residual, out, gate, style, style_per_row ? 1 : 0, eps,
                                                      residual_out, normalized, next_gate, M, D,
                                                      static_cast<hipStream_t>(stream));
    return e == hipSuccess ? VLA_OK : hip_fail(fn, "kernel launch", e);
}

int vla_probe_stream_read(const void* src, size_t bytes, uint32_t* sink, int blocks, void* stream) {
    const char* fn = "vla_probe_stream_read";
    REQUIRE_PTR(src);
    REQUIRE_PTR(sink);
    if (bytes == 0 || bytes % 16 != 0) return fail(VLA_ESHAPE, fn, "bytes=%zu must be a positive multiple of 16", bytes);
    if (blocks <= 0 || blocks > 65536) return fail(VLA_EINVAL, fn, "blocks=%d outside 1..65536", blocks);
    hipError_t e = vla::launch_stream_read(src, bytes, sink, blocks, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? VLA_OK : hip_fail(fn, "kernel launch", e);
}

int vla_probe_mfma_rate(int form, const uint32_t* operands, int iters, float* out, uint64_t* clocks, int blocks,
                        void* stream) {
    const char* fn = "vla_probe_mfma_rate";
    REQUIRE_PTR(operands);
    REQUIRE_PTR(out);
    if (clocks && (reinterpret_cast<uintptr_t>(clocks) & 7u)) return fail(VLA_EALIGN, fn, "clocks is not 8-byte aligned");
    if (form < VLA_MFMA_BF16_32X32X16 || form > VLA_MFMA_FP8_16X16X128)
        return fail(VLA_EINVAL, fn, "form=%d is not a VLA_MFMA_* value", form);
    if (iters <= 0 || iters > (1 << 24)) return fail(VLA_EINVAL, fn, "iters=%d outside 1..2^24", iters);
    if (blocks <= 0 || blocks > 65536) return fail(VLA_EINVAL, fn, "blocks=%d outside 1..65536", blocks);
    hipError_t e = vla::launch_mfma_rate(form, operands, iters, out, clocks, blocks, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? VLA_OK : hip_fail(fn, "kernel launch", e);
}

size_t vla_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int wfmt) {
    if (M <= 0 || N <= 0 || K <= 0) return 0;
    if (wfmt == VLA_WFMT_MXFP4)
        return vla::gemm_ws_bytes(vla::plan_gemm(M, N, K, vla::AType::BF16, vla::WType::FP4, vla::Epi::PLAIN), M, N);
    const vla::WType wt = (wfmt == VLA_WFMT_BF16) ? vla::WType::BF16 : vla::WType::FP8;
    size_t best = 0;
    const vla::AType ats[2] = {vla::AType::BF16, vla::AType::FP8};
    const vla::Epi eps[2] = {vla::Epi::PLAIN, vla::Epi::GELU_MUL};
    for (auto at : ats)
        for (auto ep : eps) {
            const size_t b = vla::gemm_ws_bytes(vla::plan_gemm(M, N, K, at, wt, ep), M, N);
            if (b > best) best = b;
        }
    return best;
}

int vla_gemm_supported(int64_t M, int64_t N, int64_t K, int wfmt, int fp8_act, int gelu_mul) {
    return vla_gemm_plan(M, N, K, wfmt, fp8_act, gelu_mul, nullptr, 0);
}

int vla_gemm_plan(int64_t M, int64_t N, int64_t K, int wfmt, int fp8_act, int gelu_mul, int64_t* info,
                  int n_info) {
    const char* fn = "vla_gemm_plan";
    if (n_info < 0 || (n_info > 0 && !info)) return fail(VLA_EINVAL, fn, "info is NULL or n_info < 0");
    if (int rc = check_mnk(fn, M, N, K)) return rc;
    if (wfmt != VLA_WFMT_BF16 && wfmt != VLA_WFMT_E4M3_OCP && wfmt != VLA_WFMT_MXFP4)
        return fail(VLA_EINVAL, fn, "wfmt=%d", wfmt);
    const vla::AType at = fp8_act ? vla::AType::FP8 : vla::AType::BF16;
    const vla::WType wt = (wfmt == VLA_WFMT_BF16) ? vla::WType::BF16
                          : (wfmt == VLA_WFMT_MXFP4 ? vla::WType::FP4 : vla::WType::FP8);
    const vla::Epi epi = gelu_mul ? vla::Epi::GELU_MUL : vla::Epi::PLAIN;
    if ((gelu_mul || fp8_act) && wt != vla::WType::FP8) return fail(VLA_EINVAL, fn, "fp8_act and gelu_mul need FP8 weights");
    if (gelu_mul && fp8_act) return fail(VLA_EINVAL, fn, "gelu_mul takes bf16 activations");
    if (gelu_mul && (N % 32) != 0) return fail(VLA_ESHAPE, fn, "gelu_mul needs N = 2I with I a multiple of 16");
    const vla::GemmPlan p = vla::plan_gemm(M, N, K, at, wt, epi);
    const size_t ws = vla::gemm_ws_bytes(p, M, N);
    const int64_t v[10] = {p.kernel,
                           p.nt,
                           p.groups,
                           p.kernel == 0 ? p.ksplit : p.mblocks,
                           p.kernel == 0 ? p.mblocks : p.ksplit,
                           p.ksplit,
                           static_cast<int64_t>(ws),
                           static_cast<int64_t>(ws - vla::kCounterBytes),
                           static_cast<int64_t>(p.waves) * 64,
                           p.kernel == 0 ? static_cast<int64_t>(p.groups) * p.mblocks
                                         : static_cast<int64_t>(p.groups) * p.mblocks * vla::kWideCounters};
    for (int i = 0; i < n_info && i < 10; ++i) info[i] = v[i];
    if (!vla::plan_dispatchable(p, at, wt, epi))
        return fail(VLA_ESHAPE, fn, "M=%lld N=%lld K=%lld exceeds the kernels' limits", (long long)M, (long long)N,
                    (long long)K);
    return VLA_OK;
}

int vla_gemm_fp8w(const void* A, const float* s_a, const uint8_t* Wq, const float* s_w,
                  const uint16_t* bias, const uint16_t* residual, uint16_t* Y, void* ws,
                  size_t ws_bytes, int64_t M, int64_t N, int64_t K, void* stream) {
    const char* fn = "vla_gemm_fp8w";
    if (int rc = check_mnk(fn, M, N, K)) return rc;
    REQUIRE_PTR(A);
    OPTIONAL_PTR(s_a);
    REQUIRE_PTR(Wq);
    REQUIRE_PTR(s_w);
    OPTIONAL_PTR(bias);
    OPTIONAL_PTR(residual);
    REQUIRE_PTR(Y);
    REQUIRE_PTR(ws);
    vla::GemmProblem p{};
    p.A = A; p.s_a = s_a; p.W = Wq; p.s_w = s_w; p.bias = bias; p.resid = residual; p.Y = Y; p.ws = ws;
    p.M = M; p.N = N; p.K = K;
    p.atype = s_a ? vla::AType::FP8 : vla::AType::BF16;
    p.wtype = vla::WType::FP8;
    p.epi = vla::Epi::PLAIN;
    return run_gemm(fn, p, ws_bytes, static_cast<hipStream_t>(stream));
}

int vla_gemm_fp8w_noalloc(const void* A, const float* s_a, const uint8_t* Wq, const float* s_w,
                          const uint16_t* bias, const uint16_t* residual, uint16_t* Y, int64_t M, int64_t N,
                          int64_t K, void* stream) {
    const char* fn = "vla_gemm_fp8w_noalloc";
    if (int rc = check_mnk(fn, M, N, K)) return rc;
    REQUIRE_PTR(A);
    OPTIONAL_PTR(s_a);
    REQUIRE_PTR(Wq);
    REQUIRE_PTR(s_w);
    OPTIONAL_PTR(bias);
    OPTIONAL_PTR(residual);
    REQUIRE_PTR(Y);
    vla::GemmProblem p{};
    p.A = A; p.s_a = s_a; p.W = Wq; p.s_w = s_w; p.bias = bias; p.resid = residual; p.Y = Y;
    p.M = M; p.N = N; p.K = K;
    p.atype = s_a ? vla::AType::FP8 : vla::AType::BF16;
    p.wtype = vla::WType::FP8;
    p.epi = vla::Epi::PLAIN;
    // refuse what the library's workspace cannot hold before any device work
    const vla::GemmPlan plan = vla::plan_gemm(M, N, K, p.atype, p.wtype, p.epi);
    if (!vla::plan_dispatchable(plan, p.atype, p.wtype, p.epi))
        return fail(VLA_ESHAPE, fn, "M=%lld N=%lld K=%lld exceeds the kernels' limits", (long long)M, (long long)N,
                    (long long)K);
    const size_t need = vla::gemm_ws_bytes(plan, M, N);
    if (need > vla::kNoAllocWorkspaceBytes)
        return fail(VLA_EWORKSPACE, fn, "M=%lld N=%lld K=%lld needs a %zu-byte workspace; the library's holds %zu",
                    (long long)M, (long long)N, (long long)K, need, vla::kNoAllocWorkspaceBytes);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = vla::noalloc_workspace(s, &p.ws);
    if (e != hipSuccess) return hip_fail(fn, "workspace set-up", e);
    return run_gemm(fn, p, vla::kNoAllocWorkspaceBytes, s);
}

int vla_gemm_bf16(const uint16_t* A, const uint16_t* Wq, const uint16_t* bias,
                  const uint16_t* residual, uint16_t* Y, void* ws, size_t ws_bytes, int64_t M,
                  int64_t N, int64_t K, void* stream) {
    const char* fn = "vla_gemm_bf16";
    if (int rc = check_mnk(fn, M, N, K)) return rc;
    REQUIRE_PTR(A);
    REQUIRE_PTR(Wq);
    OPTIONAL_PTR(bias);
    OPTIONAL_PTR(residual);
    REQUIRE_PTR(Y);
    REQUIRE_PTR(ws);
    vla::GemmProblem p{};
    p.A = A; p.W = Wq; p.bias = bias; p.resid = residual; p.Y = Y; p.ws = ws;
    p.M = M; p.N = N; p.K = K;
    p.atype = vla::AType::BF16;
    p.wtype = vla::WType::BF16;
    p.epi = vla::Epi::PLAIN;
    return run_gemm(fn, p, ws_bytes, static_cast<hipStream_t>(stream));
}

int vla_gemm_mxfp4w(const uint16_t* A, const uint8_t* Wq, const uint16_t* bias, const uint16_t* residual,
                    uint16_t* Y, void* ws, size_t ws_bytes, int64_t M, int64_t N, int64_t K, void* stream) {
    const char* fn = "vla_gemm_mxfp4w";
    if (int rc = check_mnk(fn, M, N, K)) return rc;
    REQUIRE_PTR(A);
    REQUIRE_PTR(Wq);
    OPTIONAL_PTR(bias);
    OPTIONAL_PTR(residual);
    REQUIRE_PTR(Y);
    REQUIRE_PTR(ws);
    vla::GemmProblem p{};
    p.A = A; p.W = Wq; p.bias = bias; p.resid = residual; p.Y = Y; p.ws = ws;
    p.M = M; p.N = N; p.K = K;
    p.atype = vla::AType::BF16;
    p.wtype = vla::WType::FP4;
    p.epi = vla::Epi::PLAIN;
    return run_gemm(fn, p, ws_bytes, static_cast<hipStream_t>(stream));
}

int vla_gemm_fp8w_gelu_mul(const uint16_t* A, const uint8_t* Wgu, const float* s_gu, const uint16_t* bias,
                           uint16_t* act, uint16_t* gu, void* ws, size_t ws_bytes, int64_t M,
                           int64_t I, int64_t K, void* stream) {
    const char* fn = "vla_gemm_fp8w_gelu_mul";
    if (int rc = check_mnk(fn, M, 2 * I, K)) return rc;
    if (I % 16 != 0) return fail(VLA_ESHAPE, fn, "I=%lld is not a multiple of 16", (long long)I);
    REQUIRE_PTR(A);
    REQUIRE_PTR(Wgu);
    REQUIRE_PTR(s_gu);
    OPTIONAL_PTR(bias);
    REQUIRE_PTR(act);
    OPTIONAL_PTR(gu);
    REQUIRE_PTR(ws);
    vla::GemmProblem p{};
    p.A = A; p.W = Wgu; p.s_w = s_gu; p.bias = bias; p.Y = act; p.gu = gu; p.ws = ws;
    p.M = M; p.N = 2 * I; p.K = K;
    p.atype = vla::AType::BF16;
    p.wtype = vla::WType::FP8;
    p.epi = vla::Epi::GELU_MUL;
    return run_gemm(fn, p, ws_bytes, static_cast<hipStream_t>(stream));
}

size_t vla_mlp_chain_scratch_bytes(int64_t M, int64_t H, int64_t I) {
    if (M <= 0 || H <= 0 || I <= 0) return 0;
    return chain_layout(M, H, I).total;
}

int vla_mlp_chain_enqueue(const uint8_t* const* wgu, const float* const* sgu,
                          const uint8_t* const* wd, const float* const* sd, const uint16_t* x_in,
                          uint16_t* x_out, void* scratch, size_t scratch_bytes, int L, int64_t M,
                          int64_t H, int64_t I, void* stream) {
    const char* fn = "vla_mlp_chain_enqueue";
    if (int rc = check_chain(fn, wgu, sgu, wd, sd, x_in, x_out, scratch, scratch_bytes, L, M, H, I)) return rc;
    return enqueue_chain(fn, wgu, sgu, wd, sd, x_in, x_out, scratch, L, M, H, I, ChainStages{},
                         static_cast<hipStream_t>(stream));
}

int vla_mlp_chain_enqueue_staged(const uint8_t* const* wgu, const float* const* sgu,
                                 const uint8_t* const* wd, const float* const* sd, const uint16_t* x_in,
                                 uint16_t* x_out, uint16_t* gu_out, uint16_t* act_out, uint16_t* down_out,
                                 uint16_t* x_layers, void* scratch, size_t scratch_bytes, int L, int64_t M,
                                 int64_t H, int64_t I, void* stream) {
    const char* fn = "vla_mlp_chain_enqueue_staged";
    if (int rc = check_chain(fn, wgu, sgu, wd, sd, x_in, x_out, scratch, scratch_bytes, L, M, H, I)) return rc;
    OPTIONAL_PTR(gu_out);
    OPTIONAL_PTR(act_out);
    OPTIONAL_PTR(down_out);
    OPTIONAL_PTR(x_layers);
    const size_t mh = static_cast<size_t>(M) * H * 2 * L, mi = static_cast<size_t>(M) * I * 2 * L;
    struct Range { const void* p; size_t n; };
    const Range outs[4] = {{gu_out, 2 * mi}, {act_out, mi}, {down_out, mh}, {x_layers, mh}};
    const Range others[3] = {{x_in, static_cast<size_t>(M) * H * 2}, {x_out, static_cast<size_t>(M) * H * 2},
                             {scratch, chain_layout(M, H, I).total}};
    auto overlap = [](const Range& x, const Range& y) {
        const uint8_t *a = static_cast<const uint8_t*>(x.p), *b = static_cast<const uint8_t*>(y.p);
        return a && b && a < b + y.n && b < a + x.n;
    };
    for (int i = 0; i < 4; ++i) {
        for (int j = i + 1; j < 4; ++j)
            if (overlap(outs[i], outs[j])) return fail(VLA_EINVAL, fn, "stage outputs %d and %d overlap", i, j);
        for (int j = 0; j < 3; ++j)
            if (overlap(outs[i], others[j])) return fail(VLA_EINVAL, fn, "stage output %d overlaps x_in, x_out or scratch", i);
    }
    ChainStages st;
    st.gu = gu_out; st.act = act_out; st.down = down_out; st.x = x_layers;
    return enqueue_chain(fn, wgu, sgu, wd, sd, x_in, x_out, scratch, L, M, H, I, st, static_cast<hipStream_t>(stream));
}

int vla_mlp_chain_create(const uint8_t* const* wgu, const float* const* sgu,
                         const uint8_t* const* wd, const float* const* sd, const uint16_t* x_in,
                         uint16_t* x_out, void* scratch, size_t scratch_bytes, int L, int64_t M,
                         int64_t H, int64_t I, void* capture_stream, vla_mlp_chain** out) {
    const char* fn = "vla_mlp_chain_create";
    if (!out) return fail(VLA_EINVAL, fn, "out is NULL");
    *out = nullptr;
    if (!capture_stream) return fail(VLA_EINVAL, fn, "capture_stream must not be the null stream");
    if (int rc = check_chain(fn, wgu, sgu, wd, sd, x_in, x_out, scratch, scratch_bytes, L, M, H, I)) return rc;
    return capture_chain(fn, capture_stream, L, out, [&](hipStream_t s) {
        return enqueue_chain(fn, wgu, sgu, wd, sd, x_in, x_out, scratch, L, M, H, I, ChainStages{}, s);
    });
}

int vla_mlp_chain_fused_supported(int64_t M, int64_t H, int64_t I, int L) {
    int npa = 0;
    return (vla::chain_fused_plan(M, H, I, L, &npa) && vla::chain_fused_resident(H, I, npa)) ? 1 : 0;
}

int vla_decoder_chain_fused_supported(int64_t M, int64_t H, int64_t I, int L, int style_per_row) {
    return decoder_fused(M, H, I, L, style_per_row) ? 1 : 0;
}

size_t vla_decoder_chain_scratch_bytes(int64_t M, int64_t H, int64_t I) {
    if (M <= 0 || H <= 0 || I <= 0) return 0;
    return decoder_layout(M, H, I).total;
}

int vla_decoder_chain_enqueue(const uint8_t* const* wgu, const float* const* sgu, const uint8_t* const* wd,
                              const float* const* sd, const uint16_t* const* style, int style_per_row, float eps,
                              const uint16_t* x_in, const uint16_t* h_in, const uint16_t* gate_in, uint16_t* x_out,
                              uint16_t* h_out, uint16_t* gate_out, void* scratch, size_t scratch_bytes, int L,
                              int64_t M, int64_t H, int64_t I, void* stream) {
    const char* fn = "vla_decoder_chain_enqueue";
    if (int rc = check_decoder(fn, wgu, sgu, wd, sd, style, style_per_row, eps, x_in, h_in, gate_in, x_out, h_out,
                               gate_out, scratch, scratch_bytes, L, M, H, I))
        return rc;
    return enqueue_decoder(fn, wgu, sgu, wd, sd, style, style_per_row, eps, x_in, h_in, gate_in, x_out, h_out,
                           gate_out, scratch, L, M, H, I, DecoderStages{}, static_cast<hipStream_t>(stream));
}

int vla_decoder_chain_enqueue_staged(const uint8_t* const* wgu, const float* const* sgu, const uint8_t* const* wd,
                                     const float* const* sd, const uint16_t* const* style, int style_per_row,
                                     float eps, const uint16_t* x_in, const uint16_t* h_in, const uint16_t* gate_in,
                                     uint16_t* x_out, uint16_t* h_out, uint16_t* gate_out, uint16_t* gu_out,
                                     uint16_t* act_out, uint16_t* down_out, uint16_t* x_layers, uint16_t* h_layers,
                                     void* scratch, size_t scratch_bytes, int L, int64_t M, int64_t H, int64_t I,
                                     void* stream) {
    const char* fn = "vla_decoder_chain_enqueue_staged";
    if (int rc = check_decoder(fn, wgu, sgu, wd, sd, style, style_per_row, eps, x_in, h_in, gate_in, x_out, h_out,
                               gate_out, scratch, scratch_bytes, L, M, H, I))
        return rc;
    OPTIONAL_PTR(gu_out);
    OPTIONAL_PTR(act_out);
    OPTIONAL_PTR(down_out);
    OPTIONAL_PTR(x_layers);
    OPTIONAL_PTR(h_layers);
    const size_t mh = static_cast<size_t>(M) * H * 2, mhl = mh * L, mil = static_cast<size_t>(M) * I * 2 * L;
    struct Range { const void* p; size_t n; };
    const Range outs[5] = {{gu_out, 2 * mil}, {act_out, mil}, {down_out, mhl}, {x_layers, mhl}, {h_layers, mhl}};
    const Range others[7] = {{x_in, mh}, {h_in, mh}, {gate_in, mh}, {x_out, mh}, {h_out, mh}, {gate_out, mh},
                             {scratch, decoder_layout(M, H, I).total}};
    auto overlap = [](const Range& x, const Range& y) {
        const uint8_t *a = static_cast<const uint8_t*>(x.p), *b = static_cast<const uint8_t*>(y.p);
        return a && b && a < b + y.n && b < a + x.n;
    };
    const size_t sty = static_cast<size_t>(style_per_row ? M : 1) * 3 * H * 2;
    for (int i = 0; i < 5; ++i) {
        for (int j = i + 1; j < 5; ++j)
            if (overlap(outs[i], outs[j])) return fail(VLA_EINVAL, fn, "stage outputs %d and %d overlap", i, j);
        for (int j = 0; j < 7; ++j)
            if (overlap(outs[i], others[j])) return fail(VLA_EINVAL, fn, "stage output %d overlaps an input, output or the scratch", i);
        for (int l = 0; l < L; ++l)
            if (overlap(outs[i], Range{style[l], sty})) return fail(VLA_EINVAL, fn, "stage output %d overlaps style %d", i, l);
    }
    DecoderStages st;
    st.mlp.gu = gu_out; st.mlp.act = act_out; st.mlp.down = down_out; st.mlp.x = x_layers; st.h = h_layers;
    return enqueue_decoder(fn, wgu, sgu, wd, sd, style, style_per_row, eps, x_in, h_in, gate_in, x_out, h_out,
                           gate_out, scratch, L, M, H, I, st, static_cast<hipStream_t>(stream));
}

int vla_decoder_chain_create(const uint8_t* const* wgu, const float* const* sgu, const uint8_t* const* wd,
                             const float* const* sd, const uint16_t* const* style, int style_per_row, float eps,
                             const uint16_t* x_in, const uint16_t* h_in, const uint16_t* gate_in, uint16_t* x_out,
                             uint16_t* h_out, uint16_t* gate_out, void* scratch, size_t scratch_bytes, int L,
                             int64_t M, int64_t H, int64_t I, void* capture_stream, vla_mlp_chain** out) {
    const char* fn = "vla_decoder_chain_create";
    if (!out) return fail(VLA_EINVAL, fn, "out is NULL");
    *out = nullptr;
    if (!capture_stream) return fail(VLA_EINVAL, fn, "capture_stream must not be the null stream");
    if (int rc = check_decoder(fn, wgu, sgu, wd, sd, style, style_per_row, eps, x_in, h_in, gate_in, x_out, h_out,
                               gate_out, scratch, scratch_bytes, L, M, H, I))
        return rc;
    return capture_chain(fn, capture_stream, L, out, [&](hipStream_t s) {
        return enqueue_decoder(fn, wgu, sgu, wd, sd, style, style_per_row, eps, x_in, h_in, gate_in, x_out, h_out,
                               gate_out, scratch, L, M, H, I, DecoderStages{}, s);
    });
}

int vla_mlp_chain_replay(vla_mlp_chain* chain, void* stream) {
    const char* fn = "vla_mlp_chain_replay";
    {
        std::lock_guard<std::mutex> lk(g_chain_mu);
        if (!chain || g_chains.find(chain) == g_chains.end())
            return fail(VLA_ESTATE, fn, "no graph captured (handle is NULL or destroyed)");
    }
    hipError_t e = hipGraphLaunch(chain->exec, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? VLA_OK : hip_fail(fn, "hipGraphLaunch", e);
}

int vla_mlp_chain_destroy(vla_mlp_chain* chain) {
    const char* fn = "vla_mlp_chain_destroy";
    if (!chain) return VLA_OK;
    {
        std::lock_guard<std::mutex> lk(g_chain_mu);
        auto it = g_chains.find(chain);
        if (it == g_chains.end()) return fail(VLA_ESTATE, fn, "handle already destroyed");
        g_chains.erase(it);
    }
    hipError_t e1 = hipGraphExecDestroy(chain->exec);
    hipError_t e2 = hipGraphDestroy(chain->graph);
    delete chain;
    if (e1 != hipSuccess) return hip_fail(fn, "hipGraphExecDestroy", e1);
    if (e2 != hipSuccess) return hip_fail(fn, "hipGraphDestroy", e2);
    return VLA_OK;
}

}  // extern "C"
