"""GPU parity of the gated-MLP chain, stage by stage on the GPU's own
inputs: every layer's merged gate/up GEMM and down GEMM against the oracle
GEMM (|y - y_ref| <= 4e-3 * sum |a w|), GELU*mul within one bf16 ulp of the
oracle, and the residual add bit for bit; eager vs graph replay (bitwise)
and graph purity under input mutation.  The end-to-end cosine against the
oracle's fp64 chain is reported, not asserted."""
import numpy as np
import pytest
import torch

import bf16_gemm_vla_amd as vla
import oracle
import synthetic
from oracle import OCP
from tests.gpu_util import Guarded, assert_gemm_close, bf16_f64, dev, host, zeros_ws

pytestmark = pytest.mark.gpu


class ChainWeights:
    def __init__(self, L, H, I, seed=0, with_down=True):
        gate, up, down = synthetic.chain_weights(L, H, I, seed)
        self.L, self.H, self.I = L, H, I
        self.wgu, self.sgu, self.wd, self.sd = [], [], [], []
        self.o_gu, self.o_sgu, self.o_d, self.o_sd = [], [], [], []
        for l in range(L):
            W = np.concatenate([gate[l], up[l]])
            q = torch.empty(2 * I * H, dtype=torch.uint8, device="cuda")
            s = torch.empty(2 * I, dtype=torch.float32, device="cuda")
            vla.vla_quantize_pack(dev(W), q, s, 2 * I, H, vla.VLA_WFMT_E4M3_OCP, vla.VLA_LAYOUT_MFMA)
            self.wgu.append(q); self.sgu.append(s)
            a, b = oracle.quantize_rows(W, OCP)
            self.o_gu.append(a); self.o_sgu.append(b)
            if not with_down:
                continue
            qd = torch.empty(H * I, dtype=torch.uint8, device="cuda")
            sd = torch.empty(H, dtype=torch.float32, device="cuda")
            vla.vla_quantize_pack(dev(down[l]), qd, sd, H, I, vla.VLA_WFMT_E4M3_OCP, vla.VLA_LAYOUT_MFMA)
            self.wd.append(qd); self.sd.append(sd)
            c, d = oracle.quantize_rows(down[l], OCP)
            self.o_d.append(c); self.o_sd.append(d)


@pytest.mark.parametrize("M,I,K", [(50, 4096, 1024), (4, 64, 128), (17, 48, 96), (300, 256, 512),
                                   (33, 4112, 1024), (40, 4128, 1024)])
def test_gelu_mul_stage(M, I, K):
    print(f"gelu_mul M={M} I={I} K={K}", flush=True)
    cw = ChainWeights(1, K, I, seed=M, with_down=False)
    A = synthetic.activations(M, K, 7000 + M)
    act, gu = Guarded(M * I * 2), Guarded(M * 2 * I * 2)
    ws = zeros_ws(vla.vla_gemm_workspace_bytes(M, 2 * I, K, 1))
    vla.vla_gemm_fp8w_gelu_mul(dev(A), cw.wgu[0], cw.sgu[0], None, act.t, gu.t, ws, ws.numel(), M, I, K)
    act.check(); gu.check()
    gu_bits = gu.numpy(np.uint16).reshape(M, 2 * I)
    # stage 1: the merged GEMM against the oracle GEMM
    ref, yabs = oracle.gemm(bf16_f64(A), oracle.dequant_rows(cw.o_gu[0], cw.o_sgu[0]))
    assert_gemm_close(gu_bits, ref, yabs)
    # stage 2: GELU*mul on the GPU's own g and u, within 1 bf16 ulp of the oracle
    want = oracle.gelu_mul(gu_bits[:, :I], gu_bits[:, I:])
    got = act.numpy(np.uint16).reshape(M, I)
    diff = np.abs(got.astype(np.int32) - want.astype(np.int32))
    same_sign = (got >> 15) == (want >> 15)
    assert np.all((diff <= 1) & same_sign | (got == want))
    # without the debug output the activation is identical
    act2 = torch.empty(M * I, dtype=torch.int16, device="cuda")
    vla.vla_gemm_fp8w_gelu_mul(dev(A), cw.wgu[0], cw.sgu[0], None, act2, None, ws, ws.numel(), M, I, K)
    assert np.array_equal(host(act2).view(np.uint16).reshape(M, I), got)


@pytest.mark.parametrize("M,I,K", [(50, 4096, 1024), (17, 48, 96), (300, 256, 512)])
def test_gelu_mul_stage_bias(M, I, K):
    """The merged gate/up GEMM adds [b_gate, b_up] in its epilogue: g and u
    against the oracle GEMM with the bias, act from the GPU's own g and u."""
    print(f"gelu_mul bias M={M} I={I} K={K}", flush=True)
    cw = ChainWeights(1, K, I, seed=M + 1, with_down=False)
    A = synthetic.activations(M, K, 7100 + M)
    b_bits = synthetic.activations(1, 2 * I, 7200 + M)[0]
    act, gu = Guarded(M * I * 2), Guarded(M * 2 * I * 2)
    ws = zeros_ws(vla.vla_gemm_workspace_bytes(M, 2 * I, K, 1))
    vla.vla_gemm_fp8w_gelu_mul(dev(A), cw.wgu[0], cw.sgu[0], dev(b_bits), act.t, gu.t, ws, ws.numel(), M, I, K)
    act.check(); gu.check()
    gu_bits = gu.numpy(np.uint16).reshape(M, 2 * I)
    ref, yabs = oracle.gemm(bf16_f64(A), oracle.dequant_rows(cw.o_gu[0], cw.o_sgu[0]), bf16_f64(b_bits))
    assert_gemm_close(gu_bits, ref, yabs)
    want = oracle.gelu_mul(gu_bits[:, :I], gu_bits[:, I:])
    got = act.numpy(np.uint16).reshape(M, I)
    diff = np.abs(got.astype(np.int32) - want.astype(np.int32))
    same_sign = (got >> 15) == (want >> 15)
    assert np.all((diff <= 1) & same_sign | (got == want))
    # every split-K counter is back at zero after the call
    assert int(host(ws[:61440]).view(np.uint32).sum()) == 0


@pytest.mark.parametrize("M", [50, 200])
def test_gelu_mul_tail_values(M):
    """One-hot gate/up weights (scale 1) pass activation columns through as g
    and u exactly, so GELU*mul sees constructed values: g across the negative
    tail where gelu(g) is tiny (down to where it underflows) and across the
    ordinary range, u from 1e-3 to 1e37 of both signs.  Every act within one
    bf16 ulp of the oracle, for the skinny (M <= 64) and the wide epilogue."""
    I, K = 64, 128
    g_vals = np.concatenate([np.linspace(-12.5, -7.0, 45), np.linspace(-6.0, 6.0, 19)]).astype(np.float32)
    rng = synthetic.rng(7300 + M)
    u_mag = (10.0 ** rng.uniform(-3, 37, (M, I))).astype(np.float32) * rng.choice([-1.0, 1.0], (M, I)).astype(np.float32)
    A = np.zeros((M, K), np.float32)
    A[:, :I] = rng.permuted(np.tile(g_vals, (M, 1)), axis=1)
    A[:, I:] = u_mag
    A_bits = synthetic.fp32_to_bf16_bits(A)
    q = np.zeros((2 * I, K), np.uint8)
    q[np.arange(2 * I), np.arange(2 * I)] = 0x38                  # gate row j <- column j, up row j <- column I + j
    ws = zeros_ws(vla.vla_gemm_workspace_bytes(M, 2 * I, K, 1))
    act, gu = Guarded(M * I * 2), Guarded(M * 2 * I * 2)
    vla.vla_gemm_fp8w_gelu_mul(dev(A_bits), dev(oracle.pack(q, 8)), dev(np.ones(2 * I, np.float32)), None,
                               act.t, gu.t, ws, ws.numel(), M, I, K)
    act.check(); gu.check()
    gu_bits = gu.numpy(np.uint16).reshape(M, 2 * I)
    assert np.array_equal(gu_bits, A_bits)                          # g and u are the columns, exactly
    want = oracle.gelu_mul(A_bits[:, :I], A_bits[:, I:])
    got = act.numpy(np.uint16).reshape(M, I)
    diff = np.abs(got.astype(np.int32) - want.astype(np.int32))
    ok = ((diff <= 1) & ((got >> 15) == (want >> 15))) | (got == want)
    assert ok.all(), f"{(~ok).sum()} differ; g={bf16_f64(A_bits[:, :I][~ok])[:4]} u={bf16_f64(A_bits[:, I:][~ok])[:4]}"
    wv = bf16_f64(want)
    assert (wv != 0).mean() > 0.8 and ((wv != 0) & (np.abs(wv) < 1e-30)).mean() > 0.05   # tiny, not underflow


def make_chain(L, M, H, I, seed=0):
    cw = ChainWeights(L, H, I, seed)
    x = synthetic.activations(M, H, synthetic.IDS["chain.x"] + seed)
    xin = dev(x)
    xout = torch.empty(M * H, dtype=torch.int16, device="cuda")
    nbytes = vla.vla_mlp_chain_scratch_bytes(M, H, I)
    scratch = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    return cw, x, xin, xout, scratch


def eager(cw, xin, xout, scratch, M):
    vla.vla_mlp_chain_enqueue(cw.wgu, cw.sgu, cw.wd, cw.sd, xin, xout, scratch, scratch.numel(),
                              cw.L, M, cw.H, cw.I)
    return host(xout).view(np.uint16).reshape(M, cw.H).copy()


def stage_outputs(cw, xin, M, scratch):
    """Run the staged chain; returns x_out and the per-layer stage arrays."""
    L, H, I = cw.L, cw.H, cw.I
    xout = torch.empty(M * H, dtype=torch.int16, device="cuda")
    bufs = {k: Guarded(L * M * n * 2) for k, n in (("gu", 2 * I), ("act", I), ("down", H), ("x", H))}
    vla.vla_mlp_chain_enqueue_staged(cw.wgu, cw.sgu, cw.wd, cw.sd, xin, xout, bufs["gu"].t, bufs["act"].t,
                                     bufs["down"].t, bufs["x"].t, scratch, scratch.numel(), L, M, H, I)
    for b in bufs.values():
        b.check()
    out = {k: b.numpy(np.uint16).reshape(L, M, -1) for k, b in bufs.items()}
    return host(xout).view(np.uint16).reshape(M, H).copy(), out


def check_stages(cw, x_in, st, M, tag):
    """Every stage of every layer whose inputs and outputs are finite, each on
    the GPU's own stage inputs.  Returns the number of layers checked."""
    L, H, I = cw.L, cw.H, cw.I
    finite = lambda b: bool(np.isfinite(bf16_f64(b)).all())
    x = x_in
    for l in range(L):
        gu, act, down, xn = st["gu"][l], st["act"][l], st["down"][l], st["x"][l]
        if not all(finite(b) for b in (x, gu, act, down, xn)):
            print(f"{tag}: layer {l} holds non-finite values (bf16 overflow); stop", flush=True)
            return l
        # 1. merged gate/up GEMM
        ref, yabs = oracle.gemm(bf16_f64(x), oracle.dequant_rows(cw.o_gu[l], cw.o_sgu[l]))
        assert_gemm_close(gu, ref, yabs)
        # 2. GELU-tanh(g) * u within one bf16 ulp (same sign)
        want = oracle.gelu_mul(gu[:, :I], gu[:, I:])
        diff = np.abs(act.astype(np.int32) - want.astype(np.int32))
        assert np.all(((diff <= 1) & ((act >> 15) == (want >> 15))) | (act == want)), f"{tag} layer {l} gelu_mul"
        # 3. down GEMM before the residual
        ref, yabs = oracle.gemm(bf16_f64(act), oracle.dequant_rows(cw.o_d[l], cw.o_sd[l]))
        assert_gemm_close(down, ref, yabs)
        # 4. residual add, bit for bit
        assert np.array_equal(xn, oracle.bf16_round(bf16_f64(x) + bf16_f64(down))), f"{tag} layer {l} residual"
        x = xn
    return L


def test_chain_small_stagewise():
    L, M, H, I = 3, 50, 256, 512
    assert vla.vla_mlp_chain_fused_supported(M, H, I, L)
    cw, x, xin, xout, scratch = make_chain(L, M, H, I, seed=1)
    got = eager(cw, xin, xout, scratch, M)
    staged_out, st = stage_outputs(cw, xin, M, scratch)
    assert np.array_equal(staged_out, got) and np.array_equal(st["x"][-1], got)
    assert check_stages(cw, x, st, M, "small") == L


@pytest.mark.parametrize("L", [32, 33])
def test_chain_layer_count_limit(L):
    """32 layers is the most the single launch takes (its kernel arguments
    carry every layer's pointers); 33 runs as the graph of GEMM launches.
    Both checked stage by stage (H = 256, I = 512, 20 rows)."""
    M, H, I = 20, 256, 512
    assert vla.vla_mlp_chain_fused_supported(M, H, I, L) == (L <= 32)
    cw, x, xin, xout, scratch = make_chain(L, M, H, I, seed=40 + L)
    got = eager(cw, xin, xout, scratch, M)
    staged_out, st = stage_outputs(cw, xin, M, scratch)
    assert np.array_equal(staged_out, got)
    checked = check_stages(cw, x, st, M, f"L={L}")
    print(f"L={L}: {checked} layers checked stage by stage", flush=True)
    assert checked >= 12
    vla.vla_workspace_status(scratch)


@pytest.mark.parametrize("M", [1, 10, 16, 17, 33, 50, 64])
def test_fused_chain_rows_stagewise(M):
    """The single-launch chain at the decoder's H = 1024, I = 4096 for every
    row-count class (1-16 rows: one gate/up pair per workgroup; 17-32: two;
    33-64: four; ragged last row tile), two layers, every stage on its own
    inputs."""
    L, H, I = 2, 1024, 4096
    assert vla.vla_mlp_chain_fused_supported(M, H, I, L)
    cw, x, xin, xout, scratch = make_chain(L, M, H, I, seed=10 + M)
    got = eager(cw, xin, xout, scratch, M)
    staged_out, st = stage_outputs(cw, xin, M, scratch)
    assert np.array_equal(staged_out, got)
    assert check_stages(cw, x, st, M, f"fused M={M}") == L
    vla.vla_workspace_status(scratch)


def test_fused_chain_barrier_wait_is_bounded():
    """With the wait bound forced down to one poll, grid barriers give up:
    the launch still completes, x_out reads NaN, the status query reports
    it, and the barrier counters are cleared, so the same scratch then gives
    the correct chain again."""
    L, M, H, I = 3, 50, 1024, 4096
    assert vla.vla_mlp_chain_fused_supported(M, H, I, L)
    cw, x, xin, xout, scratch = make_chain(L, M, H, I, seed=7)
    vla.vla_set_wait_limit(1)
    try:
        for _ in range(3):
            vla.vla_mlp_chain_enqueue(cw.wgu, cw.sgu, cw.wd, cw.sd, xin, xout, scratch, scratch.numel(), L, M, H, I)
        torch.cuda.synchronize()
    finally:
        vla.vla_set_wait_limit(0)
    assert np.isnan(bf16_f64(host(xout).view(np.uint16))).any()
    with pytest.raises(RuntimeError, match="fused chain phase barrier"):
        vla.vla_workspace_status(scratch)
    assert int(host(scratch[61440 + 256:61440 + 1024]).view(np.uint32).sum()) == 0
    staged_out, st = stage_outputs(cw, xin, M, scratch)
    assert check_stages(cw, x, st, M, "after give-up") == L
    vla.vla_workspace_status(scratch)


def test_chain_unaligned_scratch_takes_the_graph_path():
    """A scratch buffer that is not 256-byte aligned runs the chain as two
    GEMM launches per layer; every stage still matches."""
    L, M, H, I = 2, 50, 1024, 4096
    cw, x, xin, xout, _ = make_chain(L, M, H, I, seed=8)
    nbytes = vla.vla_mlp_chain_scratch_bytes(M, H, I)
    raw = torch.zeros(nbytes + 256, dtype=torch.uint8, device="cuda")
    scratch = raw[16:16 + nbytes]
    staged_out, st = stage_outputs(cw, xin, M, scratch)
    assert check_stages(cw, x, st, M, "graph path") == L
    vla.vla_workspace_status(scratch)


@pytest.mark.parametrize("M,H,I", [(17, 96, 160), (130, 256, 512)])
def test_chain_ragged_and_wide_stagewise(M, H, I):
    """Ragged rows and tiles, and M > 64 (the wide kernel's fused epilogues):
    shapes the single launch does not cover."""
    L = 2
    assert not vla.vla_mlp_chain_fused_supported(M, H, I, L)
    cw, x, xin, xout, scratch = make_chain(L, M, H, I, seed=3)
    got = eager(cw, xin, xout, scratch, M)
    staged_out, st = stage_outputs(cw, xin, M, scratch)
    assert np.array_equal(staged_out, got)
    assert check_stages(cw, x, st, M, f"M={M}") == L


def test_chain_config_replay_eager_purity():
    """18 layers, M=50, H=1024, I=4096: graph replay == eager bitwise; replay
    after mutating x_in equals a fresh eager run (the recorded region is a
    pure function of its device inputs); replay after destroy raises."""
    L, M, H, I = 18, 50, 1024, 4096
    print("chain config: building weights", flush=True)
    assert vla.vla_mlp_chain_fused_supported(M, H, I, L)
    cw, x, xin, xout, scratch = make_chain(L, M, H, I)
    ref_eager = eager(cw, xin, xout, scratch, M)
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    print("chain config: capture", flush=True)
    h = vla.vla_mlp_chain_create(cw.wgu, cw.sgu, cw.wd, cw.sd, xin, xout, scratch, scratch.numel(),
                                 L, M, H, I, stream)
    try:
        for _ in range(3):
            xout.zero_()
            torch.cuda.synchronize()
            vla.vla_mlp_chain_replay(h, stream)
            stream.synchronize()
            assert np.array_equal(host(xout).view(np.uint16).reshape(M, H), ref_eager)
        # purity: new input in place, replay, compare with eager on the new input
        x2 = synthetic.activations(M, H, 4711)
        xin.copy_(dev(x2))
        torch.cuda.synchronize()
        vla.vla_mlp_chain_replay(h, stream)
        stream.synchronize()
        replayed = host(xout).view(np.uint16).reshape(M, H).copy()
        assert not np.array_equal(replayed, ref_eager)
        assert np.array_equal(replayed, eager(cw, xin, xout, scratch, M))
        xin.copy_(dev(x))
        torch.cuda.synchronize()
    finally:
        vla.vla_mlp_chain_destroy(h)
    with pytest.raises(RuntimeError, match="vla_mlp_chain_replay"):
        vla.vla_mlp_chain_replay(h, stream)
    vla.vla_workspace_status(scratch)


def test_chain_config_stagewise():
    """18 layers, M=50, H=1024, I=4096, every stage of every layer on the
    GPU's own stage inputs.  With the configured N(0, 0.02) weights and no
    normalisation between layers the residual stream grows quadratically
    and overflows bf16 in the last layers (the oracle's fp64 chain does the
    same); every layer before the first non-finite value is checked.  The
    staged run's output equals the plain chain's bit for bit."""
    L, M, H, I = 18, 50, 1024, 4096
    print("chain stages: building weights", flush=True)
    cw, x, xin, xout, scratch = make_chain(L, M, H, I)
    ref_eager = eager(cw, xin, xout, scratch, M)
    staged_out, st = stage_outputs(cw, xin, M, scratch)
    assert np.array_equal(staged_out, ref_eager)
    checked = check_stages(cw, x, st, M, "config")
    print(f"chain stages: {checked} of {L} layers checked stage by stage", flush=True)
    assert checked >= 12
    # reported only: end-to-end agreement with the oracle's fp64 chain over the checked layers
    o_x = oracle.mlp_chain(x, cw.o_gu[:checked], cw.o_sgu[:checked], cw.o_d[:checked], cw.o_sd[:checked])
    a, b = bf16_f64(st["x"][checked - 1]).ravel(), bf16_f64(o_x).ravel()
    print(f"chain end to end after {checked} layers: cosine {float(a @ b / np.linalg.norm(a) / np.linalg.norm(b)):.7f}",
          flush=True)
    vla.vla_workspace_status(scratch)
