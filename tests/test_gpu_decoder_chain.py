"""GPU parity of the decoder-block chain (merged gate/up GEMM with GELU*mul,
down GEMM, decoder boundary per layer).

Single launch (the shapes the fused gated-MLP chain takes): every stage of
every layer, kept by vla_decoder_chain_enqueue_staged, is checked against
the oracle on the GPU's own stage inputs - the GEMMs within 4e-3 * sum
|a w|, GELU*mul within one bf16 ulp, the gated residual and the next gate
bit for bit, h within one bf16 ulp - and the outputs equal the last stage.

Graph of launches (forced by an unaligned scratch): the chain equals, bit
for bit, the same layers run one entry point at a time, every one of those
stages checked against the oracle the same way; eager vs graph replay
(bitwise) and graph purity under input mutation.  End-to-end cosines
against the oracle's fp64 chain are reported, not asserted."""
import numpy as np
import pytest
import torch

import bf16_gemm_vla_amd as vla
import oracle
import synthetic
from tests.gpu_util import assert_gemm_close, bf16_f64, dev, host, zeros_ws
from tests.test_gpu_boundary import assert_close_bf16
from tests.test_gpu_chain import ChainWeights

pytestmark = pytest.mark.gpu


class Decoder:
    def __init__(self, L, M, H, I, per_row=True, seed=0, eps=1e-6, graph_path=False):
        self.cw = ChainWeights(L, H, I, seed)
        self.L, self.M, self.H, self.I, self.per_row, self.eps = L, M, H, I, per_row, eps
        x, h, g, st = synthetic.decoder_chain_inputs(L, M, H, M if per_row else 1, seed)
        self.inputs = (x, h, g)
        self.styles = st
        self.d_in = [dev(a) for a in self.inputs]
        self.d_style = [dev(s) for s in st]
        self.d_out = [torch.empty(M * H, dtype=torch.int16, device="cuda") for _ in range(3)]
        n = vla.vla_decoder_chain_scratch_bytes(M, H, I)
        # a scratch 16 bytes off a 256-byte boundary takes the graph of launches
        self._scratch = torch.zeros(n + 256, dtype=torch.uint8, device="cuda")
        self.scratch = self._scratch[16:16 + n] if graph_path else self._scratch[:n]

    def args(self, layers=None):
        L = self.L if layers is None else layers
        cw = self.cw
        return (cw.wgu[:L], cw.sgu[:L], cw.wd[:L], cw.sd[:L], self.d_style[:L], self.per_row, self.eps,
                *self.d_in, *self.d_out, self.scratch, self.scratch.numel(), L, self.M, self.H, self.I)

    def fused(self):
        return vla.vla_decoder_chain_fused_supported(self.M, self.H, self.I, self.L, self.per_row)

    def staged(self):
        """Run the staged chain; returns the outputs and the per-layer stages."""
        L, M, H, I, cw = self.L, self.M, self.H, self.I, self.cw
        bufs = {k: torch.empty(L * M * n, dtype=torch.int16, device="cuda")
                for k, n in (("gu", 2 * I), ("act", I), ("down", H), ("x", H), ("h", H))}
        vla.vla_decoder_chain_enqueue_staged(cw.wgu, cw.sgu, cw.wd, cw.sd, self.d_style, self.per_row, self.eps,
                                             *self.d_in, *self.d_out, bufs["gu"], bufs["act"], bufs["down"], bufs["x"],
                                             bufs["h"], self.scratch, self.scratch.numel(), L, M, H, I)
        outs = tuple(host(o).view(np.uint16).reshape(M, H).copy() for o in self.d_out)
        st = {k: host(b).view(np.uint16).reshape(L, M, -1).copy() for k, b in bufs.items()}
        return outs, st

    def eager(self, layers=None):
        vla.vla_decoder_chain_enqueue(*self.args(layers))
        return tuple(host(o).view(np.uint16).reshape(self.M, self.H).copy() for o in self.d_out)



def close(a_bits, b_bits):
    a, b = bf16_f64(a_bits).ravel(), bf16_f64(b_bits).ravel()
    return float(a @ b / np.linalg.norm(a) / np.linalg.norm(b))


def check_layers(dec, tag):
    """Run the layers one entry point at a time (the kernels the chain is
    recorded from) and check every stage on its own inputs; returns the final
    (x, h, g), which must equal the chain's output bit for bit."""
    M, H, I, cw = dec.M, dec.H, dec.I, dec.cw
    ws = zeros_ws(max(vla.vla_gemm_workspace_bytes(M, 2 * I, H, 1), vla.vla_gemm_workspace_bytes(M, H, I, 1)))
    act = torch.empty(M * I, dtype=torch.int16, device="cuda")
    gu = torch.empty(M * 2 * I, dtype=torch.int16, device="cuda")
    d = torch.empty(M * H, dtype=torch.int16, device="cuda")
    outs = [torch.empty(M * H, dtype=torch.int16, device="cuda") for _ in range(3)]
    x, h, g = dec.inputs
    for l in range(dec.L):
        vla.vla_gemm_fp8w_gelu_mul(dev(h), cw.wgu[l], cw.sgu[l], None, act, gu, ws, ws.numel(), M, I, H)
        gub = host(gu).view(np.uint16).reshape(M, 2 * I).copy()
        actb = host(act).view(np.uint16).reshape(M, I).copy()
        ref, yabs = oracle.gemm(bf16_f64(h), oracle.dequant_rows(cw.o_gu[l], cw.o_sgu[l]))
        assert_gemm_close(gub, ref, yabs)
        want = oracle.gelu_mul(gub[:, :I], gub[:, I:])
        diff = np.abs(actb.astype(np.int32) - want.astype(np.int32))
        assert np.all(((diff <= 1) & ((actb >> 15) == (want >> 15))) | (actb == want)), f"{tag} layer {l} gelu_mul"
        vla.vla_gemm_fp8w(act, None, cw.wd[l], cw.sd[l], None, None, d, ws, ws.numel(), M, H, I)
        db = host(d).view(np.uint16).reshape(M, H).copy()
        ref, yabs = oracle.gemm(bf16_f64(actb), oracle.dequant_rows(cw.o_d[l], cw.o_sd[l]))
        assert_gemm_close(db, ref, yabs)
        vla.vla_gate_residual_ada_norm(dev(x), d, dev(g), dec.d_style[l], dec.per_row, dec.eps, *outs, M, H)
        xn, hn, gn = (host(o).view(np.uint16).reshape(M, H).copy() for o in outs)
        rx, rh, rg = oracle.gate_residual_ada_norm(x, db, g, dec.styles[l], dec.eps, style_per_row=dec.per_row)
        assert np.array_equal(xn, rx), f"{tag} layer {l} gated residual"
        assert np.array_equal(gn, rg), f"{tag} layer {l} next gate"
        assert_close_bf16(hn, rh)
        x, h, g = xn, hn, gn
    vla.vla_workspace_status(ws)
    return x, h, g


def check_staged(dec, outs, st, tag, min_layers=None):
    """Every stage of every layer of a staged run against the oracle on the
    GPU's own stage inputs; returns the number of layers checked (stops at
    the first non-finite value)."""
    M, H, I, cw = dec.M, dec.H, dec.I, dec.cw
    x, h, g = dec.inputs
    finite = lambda b: bool(np.isfinite(bf16_f64(b)).all())
    differing = []
    for l in range(dec.L):
        gu, act, d, xn, hn = st["gu"][l], st["act"][l], st["down"][l], st["x"][l], st["h"][l]
        if not all(finite(b) for b in (h, gu, act, d, xn, hn)):
            print(f"{tag}: layer {l} holds non-finite values; stop", flush=True)
            return l
        ref, yabs = oracle.gemm(bf16_f64(h), oracle.dequant_rows(cw.o_gu[l], cw.o_sgu[l]))
        assert_gemm_close(gu, ref, yabs)
        want = oracle.gelu_mul(gu[:, :I], gu[:, I:])
        diff = np.abs(act.astype(np.int32) - want.astype(np.int32))
        assert np.all(((diff <= 1) & ((act >> 15) == (want >> 15))) | (act == want)), f"{tag} layer {l} gelu_mul"
        ref, yabs = oracle.gemm(bf16_f64(act), oracle.dequant_rows(cw.o_d[l], cw.o_sd[l]))
        assert_gemm_close(d, ref, yabs)
        rx, rh, rg = oracle.gate_residual_ada_norm(x, d, g, dec.styles[l], dec.eps, style_per_row=dec.per_row)
        assert np.array_equal(xn, rx), f"{tag} layer {l} gated residual"
        differing.append(assert_close_bf16(hn, rh))
        x, h, g = xn, hn, rg
    assert np.array_equal(outs[0], x) and np.array_equal(outs[1], h) and np.array_equal(outs[2], g), f"{tag} outputs"
    print(f"{tag}: {dec.L} layers; h values differing from the fp64 boundary by one ulp: "
          f"{max(differing) if differing else 0:.2e} (largest layer fraction)", flush=True)
    assert max(differing) < 1e-3
    return dec.L


@pytest.mark.parametrize("M,per_row", [(50, False), (1, True), (10, True), (16, True), (17, False), (33, False),
                                       (64, False), (17, True), (50, True)])
def test_decoder_chain_stagewise(M, per_row):
    """The decoder-block chain at H = 256, I = 512, three layers, every
    row-count class and both style forms: one launch, except with a style
    row per activation row beyond one 16-row tile (the graph of launches)."""
    dec = Decoder(3, M, 256, 512, per_row=per_row, seed=2 + M)
    assert dec.fused() == (not per_row or M <= 16)
    outs, st = dec.staged()
    path = "fused" if dec.fused() else "graph"
    assert check_staged(dec, outs, st, f"{path} M={M} per_row={per_row}") == dec.L
    assert all(np.array_equal(a, b) for a, b in zip(outs, dec.eager()))
    vla.vla_workspace_status(dec.scratch)


@pytest.mark.parametrize("M,per_row", [(10, True), (24, False), (64, False)])
def test_decoder_chain_full_width_fused_stagewise(M, per_row):
    """The single launch at the decoder's own widths (H = 1024, I = 4096),
    three layers, one configuration per row-tile count class (one, two and
    four gate/up pairs per workgroup): every stage against the oracle, and
    the plain launch equal to the staged one bit for bit."""
    dec = Decoder(3, M, 1024, 4096, per_row=per_row, seed=40 + M)
    assert dec.fused()
    outs, st = dec.staged()
    assert check_staged(dec, outs, st, f"fused full width M={M} per_row={per_row}") == dec.L
    assert all(np.array_equal(a, b) for a, b in zip(outs, dec.eager()))
    vla.vla_workspace_status(dec.scratch)


@pytest.mark.parametrize("per_row", [True, False])
def test_decoder_chain_small_layerwise(per_row):
    """The graph of launches (unaligned scratch) equals the layers run one
    entry point at a time, bit for bit; its staged run checks out too."""
    dec = Decoder(3, 50, 256, 512, per_row=per_row, seed=2, graph_path=True)
    final = check_layers(dec, "small")
    assert all(np.array_equal(a, b) for a, b in zip(final, dec.eager()))
    outs, st = dec.staged()
    assert check_staged(dec, outs, st, f"graph per_row={per_row}") == dec.L
    assert all(np.array_equal(a, b) for a, b in zip(outs, final))


@pytest.mark.parametrize("graph_path", [False, True])
def test_decoder_chain_config_replay_purity_and_layers(graph_path):
    """18 layers, M=50, H=1024, I=4096, as one launch (one style row for
    every row) and as the graph of launches (a style row per row, unaligned
    scratch): graph replay == eager bitwise, replay after mutating the inputs
    equals a fresh eager run, and every stage of every layer matches the
    oracle on the GPU's own stage inputs."""
    L, M, H, I = 18, 50, 1024, 4096
    print(f"decoder chain (graph path {graph_path}): building weights", flush=True)
    # one style row for all rows takes the single launch at this shape
    dec = Decoder(L, M, H, I, per_row=graph_path, graph_path=graph_path)
    assert dec.fused() == (not graph_path)
    ref = dec.eager()
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    print("decoder chain: capture", flush=True)
    handle = vla.vla_decoder_chain_create(*dec.args(), stream)
    try:
        for _ in range(3):
            for o in dec.d_out:
                o.zero_()
            torch.cuda.synchronize()
            vla.vla_mlp_chain_replay(handle, stream)
            stream.synchronize()
            got = tuple(host(o).view(np.uint16).reshape(M, H) for o in dec.d_out)
            assert all(np.array_equal(a, b) for a, b in zip(got, ref))
        x2 = synthetic.activations(M, H, 4712)
        dec.d_in[0].copy_(dev(x2))
        torch.cuda.synchronize()
        vla.vla_mlp_chain_replay(handle, stream)
        stream.synchronize()
        replayed = tuple(host(o).view(np.uint16).reshape(M, H).copy() for o in dec.d_out)
        assert not np.array_equal(replayed[0], ref[0])
        fresh = dec.eager()
        assert all(np.array_equal(a, b) for a, b in zip(replayed, fresh))
        dec.d_in[0].copy_(dev(dec.inputs[0]))
        torch.cuda.synchronize()
    finally:
        vla.vla_mlp_chain_destroy(handle)
    print("decoder chain: per-stage oracle", flush=True)
    if graph_path:
        final = check_layers(dec, "config")
        assert all(np.array_equal(a, b) for a, b in zip(final, ref))
    outs, st = dec.staged()
    assert all(np.array_equal(a, b) for a, b in zip(outs, ref))
    assert check_staged(dec, outs, st, f"config graph path {graph_path}") == L
    cw = dec.cw
    e2e = oracle.decoder_chain(*dec.inputs, cw.o_gu, cw.o_sgu, cw.o_d, cw.o_sd, dec.styles, dec.eps,
                               style_per_row=dec.per_row)
    for name, a, b in (("x", ref[0], e2e[0]), ("h", ref[1], e2e[1])):
        print(f"end to end {name}: cosine={close(a, b):.7f} (reported)", flush=True)
    vla.vla_workspace_status(dec.scratch)


@pytest.mark.parametrize("L", [1, 32, 33])
def test_decoder_chain_layer_count_limit(L):
    """One layer (the single launch's last-layer path only), 32 (the most
    the single launch takes) and 33 (the graph of launches), 10 rows with a
    style row per row, H = 256, I = 512: every stage against the oracle."""
    dec = Decoder(L, 10, 256, 512, per_row=True, seed=60 + L)
    assert dec.fused() == (L <= 32)
    outs, st = dec.staged()
    checked = check_staged(dec, outs, st, f"L={L}")
    assert checked == L
    assert all(np.array_equal(a, b) for a, b in zip(outs, dec.eager()))
    vla.vla_workspace_status(dec.scratch)


def test_fused_decoder_chain_barrier_wait_is_bounded():
    """With the wait bound forced down to one poll the single launch's
    barriers give up: the launch completes, x_out, h_out and gate_out read
    NaN, the status query names the cause, and the same scratch then gives the
    correct chain again."""
    dec = Decoder(3, 50, 1024, 4096, per_row=False, seed=9)
    assert dec.fused()
    vla.vla_set_wait_limit(1)
    try:
        for _ in range(3):
            vla.vla_decoder_chain_enqueue(*dec.args())
        torch.cuda.synchronize()
    finally:
        vla.vla_set_wait_limit(0)
    x_out, h_out, g_out = (host(o).view(np.uint16) for o in dec.d_out)
    assert all(np.isnan(bf16_f64(o)).any() for o in (x_out, h_out, g_out))
    with pytest.raises(RuntimeError, match="fused chain phase barrier"):
        vla.vla_workspace_status(dec.scratch)
    outs, st = dec.staged()
    assert check_staged(dec, outs, st, "after give-up") == dec.L
    assert all(np.array_equal(a, b) for a, b in zip(outs, dec.eager()))
    vla.vla_workspace_status(dec.scratch)
