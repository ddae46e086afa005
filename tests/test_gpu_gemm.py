"""GPU parity of the GEMMs against the oracle's fp64 GEMM on the same
dequantized operands: |y - y_ref| <= 4e-3 * sum_k |a w| elementwise, for every
output of every configuration (the full encoder sizes included); lane-map
probes (one-hot weights must reproduce A's columns bit for bit) on both wide
tile widths; canaries, repeatability, bias, the residual add bit for bit,
ragged shapes, and the bounded split-K wait."""
import numpy as np
import pytest
import torch

import bf16_gemm_vla_amd as vla
import oracle
import synthetic
from oracle import OCP
from tests.gpu_util import Guarded, assert_gemm_close, bf16_f64, dev, host, zeros_ws

pytestmark = pytest.mark.gpu


class Weights:
    """An fp32 weight quantized+packed on the GPU, and its oracle codes."""

    def __init__(self, W: np.ndarray, wfmt: int):
        self.N, self.K = W.shape
        self.wfmt = wfmt
        nbytes = vla.vla_packed_bytes(self.N, self.K, wfmt)
        self.q = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        self.s = torch.empty(self.N, dtype=torch.float32, device="cuda") if wfmt != vla.VLA_WFMT_BF16 else None
        vla.vla_quantize_pack(dev(W), self.q, self.s, self.N, self.K, wfmt, vla.VLA_LAYOUT_MFMA)
        if wfmt == vla.VLA_WFMT_BF16:
            self.w = oracle.bf16_value(oracle.bf16_round(W.astype(np.float64)))
        else:
            qo, so = oracle.quantize_rows(W, OCP)
            self.w = oracle.dequant_rows(qo, so, OCP)


def run_gemm(A_dev, w: Weights, M, s_a=None, bias=None, resid=None, Y=None):
    N, K = w.N, w.K
    ws = zeros_ws(vla.vla_gemm_workspace_bytes(M, N, K, w.wfmt))
    out = Y if Y is not None else Guarded(M * N * 2)
    ydev = out.t if isinstance(out, Guarded) else out
    if w.wfmt == vla.VLA_WFMT_BF16:
        vla.vla_gemm_bf16(A_dev, w.q, bias, resid, ydev, ws, ws.numel(), M, N, K)
    else:
        vla.vla_gemm_fp8w(A_dev, s_a, w.q, w.s, bias, resid, ydev, ws, ws.numel(), M, N, K)
    if isinstance(out, Guarded):
        out.check()
        return out.numpy(np.uint16).reshape(M, N), ws
    return host(out, np.uint16).reshape(M, N), ws


def check(M, N, K, wfmt, seed, bias=False):
    print(f"gemm M={M} N={N} K={K} wfmt={wfmt} bias={bias}", flush=True)
    A = synthetic.activations(M, K, seed)
    w = Weights(synthetic.weights(N, K, seed + 1), wfmt)
    b_bits = synthetic.activations(1, N, seed + 2)[0] if bias else None
    y, ws = run_gemm(dev(A), w, M, bias=None if b_bits is None else dev(b_bits))
    ref, yabs = oracle.gemm(bf16_f64(A), w.w, None if b_bits is None else bf16_f64(b_bits))
    assert_gemm_close(y, ref, yabs)
    # every split-K counter is back at zero after the call, no wait gave up
    assert int(host(ws[:61440]).view(np.uint32).sum()) == 0
    vla.vla_workspace_status(ws)
    return y


# ---------------------------------------------------------------- probes

@pytest.mark.parametrize("M", [50, 200])
def test_lane_map_probe_one_hot(M):
    """Each weight row a single 1.0 code: Y must equal permuted columns of A exactly."""
    g = synthetic.rng(5000 + M)
    N, K = 128, 256
    perm = g.integers(0, K, N)
    q = np.zeros((N, K), np.uint8)
    q[np.arange(N), perm] = 0x38
    qp = dev(oracle.pack(q, 8))
    s = dev(np.ones(N, np.float32))
    A = synthetic.activations(M, K, 5001)
    ws = zeros_ws(vla.vla_gemm_workspace_bytes(M, N, K, 1))
    Y = Guarded(M * N * 2)
    vla.vla_gemm_fp8w(dev(A), None, qp, s, None, None, Y.t, ws, ws.numel(), M, N, K)
    Y.check()
    assert np.array_equal(Y.numpy(np.uint16).reshape(M, N), A[:, perm])


@pytest.mark.parametrize("M", [50, 200])
def test_decode_every_code_through_gemm(M):
    """A one-hot activation row picks one weight code per output: with s = 1,
    Y[m, n] = dec(q[n, m]) exactly, for every non-NaN OCP code, through the
    weight path of the skinny (M <= 64) and the wide kernel."""
    g = synthetic.rng(5200 + M)
    N, K = 256, 256
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F and c != 0x80], np.uint8)
    q = codes[g.integers(0, codes.size, (N, K))]
    q[:, :M] = np.resize(codes, (N, M)) if M * N >= codes.size else q[:, :M]
    A = np.zeros((M, K), np.uint16)
    A[np.arange(M), np.arange(M)] = 0x3F80                      # bf16 1.0
    ws = zeros_ws(vla.vla_gemm_workspace_bytes(M, N, K, 1))
    Y = Guarded(M * N * 2)
    vla.vla_gemm_fp8w(dev(A), None, dev(oracle.pack(q, 8)), dev(np.ones(N, np.float32)), None, None,
                      Y.t, ws, ws.numel(), M, N, K)
    got = bf16_f64(Y.numpy(np.uint16).reshape(M, N))
    want = oracle.decode(q[:, :M].T, OCP)
    assert set(q[:, :M].ravel().tolist()) == set(codes.tolist())
    assert np.array_equal(got, want)


def test_lane_map_probe_one_hot_fp8_x_fp8():
    """FP8 x FP8: one-hot weights select A's codes; s_a = 1 gives dec(A) exactly."""
    g = synthetic.rng(5100)
    M, N, K = 192, 128, 256
    perm = g.integers(0, K, N)
    q = np.zeros((N, K), np.uint8)
    q[np.arange(N), perm] = 0x38
    qa = g.integers(0, 256, (M, K)).astype(np.uint8)
    qa[(qa & 0x7F) == 0x7F] = 0x38           # no NaN codes
    qa[qa == 0x80] = 0x00                    # a one-hot sum of -0 and +0 products is +0
    ws = zeros_ws(vla.vla_gemm_workspace_bytes(M, N, K, 1))
    Y = Guarded(M * N * 2)
    vla.vla_gemm_fp8w(dev(qa), dev(np.ones(1, np.float32)), dev(oracle.pack(q, 8)), dev(np.ones(N, np.float32)),
                      None, None, Y.t, ws, ws.numel(), M, N, K)
    want = oracle.bf16_round(oracle.decode(qa, OCP)[:, perm])
    got = Y.numpy(np.uint16).reshape(M, N)
    bad = got != want
    if bad.any():
        codes = sorted(set(qa[:, perm][bad].tolist()))
        raise AssertionError(f"{bad.sum()} mismatches; A codes involved: {[hex(c) for c in codes[:32]]}; "
                             f"got {[hex(v) for v in got[bad][:8]]} want {[hex(v) for v in want[bad][:8]]}")


def plan(M, N, K, wfmt=vla.VLA_WFMT_E4M3_OCP, fp8_act=False):
    rc, info = vla.vla_gemm_plan(M, N, K, wfmt, fp8_act)
    assert rc == 0
    return info


@pytest.mark.parametrize("K", [64, 96, 160, 256, 320, 352, 448])
@pytest.mark.parametrize("kind", ["w8a16", "fp8xfp8", "mxfp4"])
def test_lane_map_probe_256_tiles(kind, K):
    """One-hot weights at M = 768, N = 16384 (the encoder up-projection's
    row and column counts), which the wide kernel runs on 256-column tiles:
    Y must be A's permuted columns bit for bit (FP8 x FP8: the decoded codes;
    MXFP4: each weight a single 4.0 code in a block of scale 2^-2).  The K
    values give 1 to 7 pipeline stages of 64, two with a ragged last stage,
    so every remainder of the stage ring (and of its pairs) runs."""
    M, N = 768, 16384
    wfmt = vla.VLA_WFMT_MXFP4 if kind == "mxfp4" else vla.VLA_WFMT_E4M3_OCP
    info = plan(M, N, K, wfmt, kind == "fp8xfp8")
    assert info[0] == 1 and info[1] == 256, info          # the wide kernel, 256-column tiles
    print(f"probe256 {kind} K={K} plan={info}", flush=True)
    g = synthetic.rng(5300 + K + len(kind))
    perm = g.integers(0, K, N)
    ws = zeros_ws(vla.vla_gemm_workspace_bytes(M, N, K, wfmt))
    Y = Guarded(M * N * 2)
    if kind == "mxfp4":
        W = np.zeros((N, K), np.float32)
        W[np.arange(N), perm] = 1.0
        q = torch.empty(vla.vla_packed_bytes(N, K, wfmt), dtype=torch.uint8, device="cuda")
        vla.vla_quantize_pack(dev(W), q, None, N, K, wfmt, vla.VLA_LAYOUT_MFMA)
        A = synthetic.activations(M, K, 5301)
        vla.vla_gemm_mxfp4w(dev(A), q, None, None, Y.t, ws, ws.numel(), M, N, K)
        want = A[:, perm]
    else:
        q = np.zeros((N, K), np.uint8)
        q[np.arange(N), perm] = 0x38
        s = dev(np.ones(N, np.float32))
        if kind == "w8a16":
            A = synthetic.activations(M, K, 5302)
            vla.vla_gemm_fp8w(dev(A), None, dev(oracle.pack(q, 8)), s, None, None, Y.t, ws, ws.numel(), M, N, K)
            want = A[:, perm]
        else:
            qa = g.integers(0, 256, (M, K)).astype(np.uint8)
            qa[(qa & 0x7F) == 0x7F] = 0x38       # no NaN codes
            qa[qa == 0x80] = 0x00                # a one-hot sum of -0 and +0 products is +0
            vla.vla_gemm_fp8w(dev(qa), dev(np.ones(1, np.float32)), dev(oracle.pack(q, 8)), s, None, None,
                              Y.t, ws, ws.numel(), M, N, K)
            want = oracle.bf16_round(oracle.decode(qa, OCP)[:, perm])
    Y.check()
    got = Y.numpy(np.uint16).reshape(M, N)
    bad = got != want
    assert not bad.any(), f"{bad.sum()} of {bad.size} differ, first at {tuple(np.argwhere(bad)[0])}"


# ------------------------------------------------------- configs + edges

def test_tiny_config():
    """A 4 x 128 bf16, W 64 x 128 -> OCP per-channel (absmax/448)."""
    check(4, 64, 128, vla.VLA_WFMT_E4M3_OCP, synthetic.IDS["tiny.A"])


@pytest.mark.parametrize("wfmt", [vla.VLA_WFMT_E4M3_OCP, vla.VLA_WFMT_BF16])
@pytest.mark.parametrize("N,K", [(4096, 1024), (1024, 4096)])
def test_skinny_configs(wfmt, N, K):
    """Action-decoder shapes, M = 50, up- and down-projection."""
    check(50, N, K, wfmt, synthetic.IDS["skinny.up.A"] if N == 4096 else synthetic.IDS["skinny.down.A"])


@pytest.mark.parametrize("wfmt", [vla.VLA_WFMT_E4M3_OCP, vla.VLA_WFMT_BF16])
@pytest.mark.parametrize("M,N", [(33, 4112), (64, 4096), (40, 8224)])
def test_two_tiles_row_halves(wfmt, M, N):
    """More than 32 rows and >= 256 column tiles: workgroups of two column
    tiles x half the rows, with a ragged last group and a one-row half."""
    check(M, N, 1024, wfmt, 6400 + M + N)


@pytest.mark.parametrize("M", [1, 10, 16, 17, 33, 64, 65, 100, 129, 571])
def test_ragged_rows(M):
    check(M, 96, 160, vla.VLA_WFMT_E4M3_OCP, 6000 + M)


@pytest.mark.parametrize("N,K", [(16, 32), (48, 96), (80, 32), (16, 4096), (2048, 64), (272, 1056)])
@pytest.mark.parametrize("M", [50, 300])
def test_ragged_tiles(M, N, K):
    check(M, N, K, vla.VLA_WFMT_E4M3_OCP, 6100 + N + K)


@pytest.mark.parametrize("M", [50, 256])
def test_bias_epilogue(M):
    check(M, 256, 512, vla.VLA_WFMT_E4M3_OCP, 6200 + M, bias=True)
    check(M, 256, 512, vla.VLA_WFMT_BF16, 6300 + M, bias=True)


@pytest.mark.parametrize("M,N,K", [(50, 1024, 4096), (200, 256, 1024)])
def test_residual_in_place(M, N, K):
    A = synthetic.activations(M, K, 6400)
    w = Weights(synthetic.weights(N, K, 6401), vla.VLA_WFMT_E4M3_OCP)
    x = synthetic.activations(M, N, 6402)
    xd = dev(x)
    ws = zeros_ws(vla.vla_gemm_workspace_bytes(M, N, K, 1))
    vla.vla_gemm_fp8w(dev(A), None, w.q, w.s, None, xd, xd, ws, ws.numel(), M, N, K)   # x += A W^T
    got = bf16_f64(host(xd, np.uint16).reshape(M, N))
    ref, yabs = oracle.gemm(bf16_f64(A), w.w)
    xf = bf16_f64(x)
    bound = 4e-3 * yabs + 2.0 ** -8 * (np.abs(xf) + np.abs(ref))
    assert np.all(np.abs(got - (xf + ref)) <= bound)


@pytest.mark.parametrize("wfmt", [vla.VLA_WFMT_E4M3_OCP, vla.VLA_WFMT_BF16, vla.VLA_WFMT_MXFP4])
@pytest.mark.parametrize("M,N,K", [(50, 1024, 4096), (10, 256, 8192), (200, 256, 1024), (768, 2048, 16384)])
def test_residual_bit_exact(wfmt, M, N, K):
    """The fused residual add is bf16(x + y) bit for bit, where y is the same
    GEMM run without a residual (its reduction order is fixed per shape):
    skinny without and with a K split across workgroups, wide without and
    with one; into a separate output and in place."""
    plan_info = plan(M, N, K, wfmt)
    print(f"residual M={M} N={N} K={K} wfmt={wfmt} plan={plan_info}", flush=True)
    A = dev(synthetic.activations(M, K, 6700 + M))
    x = synthetic.activations(M, N, 6701 + M)
    ws = zeros_ws(vla.vla_gemm_workspace_bytes(M, N, K, wfmt))
    if wfmt == vla.VLA_WFMT_MXFP4:
        Wf = synthetic.weights(N, K, 6702 + M)
        q = torch.empty(vla.vla_packed_bytes(N, K, wfmt), dtype=torch.uint8, device="cuda")
        vla.vla_quantize_pack(dev(Wf), q, None, N, K, wfmt, vla.VLA_LAYOUT_MFMA)

        def call(resid, Y):
            vla.vla_gemm_mxfp4w(A, q, None, resid, Y, ws, ws.numel(), M, N, K)
    else:
        w = Weights(synthetic.weights(N, K, 6702 + M), wfmt)

        def call(resid, Y):
            if wfmt == vla.VLA_WFMT_BF16:
                vla.vla_gemm_bf16(A, w.q, None, resid, Y, ws, ws.numel(), M, N, K)
            else:
                vla.vla_gemm_fp8w(A, None, w.q, w.s, None, resid, Y, ws, ws.numel(), M, N, K)
    y = torch.empty(M * N, dtype=torch.int16, device="cuda")
    call(None, y)
    z = Guarded(M * N * 2)
    xd = dev(x)
    call(xd, z.t)
    z.check()
    call(xd, xd)                                   # in place
    want = oracle.bf16_round(bf16_f64(x) + bf16_f64(host(y, np.uint16).reshape(M, N)))
    assert np.array_equal(z.numpy(np.uint16).reshape(M, N), want)
    assert np.array_equal(host(xd, np.uint16).reshape(M, N), want)
    vla.vla_workspace_status(ws)


def test_wide_splitk_wait_is_bounded():
    """The wide kernel's split-K owners wait for the other splits' partials
    with a bounded poll.  With the bound forced down to one poll from the
    host, owners that would wait give up: every workgroup still exits, the
    call completes, the workspace's counters are cleared, the slices left
    unfinished read NaN, and the status query reports them.  With the bound
    restored the same
    workspace gives the full, correct result."""
    M, N, K = 768, 2048, 16384
    info = plan(M, N, K)
    assert info[0] == 1 and info[5] > 1, info              # wide, K split across workgroups
    A = synthetic.activations(M, K, 6800)
    w = Weights(synthetic.weights(N, K, 6801), vla.VLA_WFMT_E4M3_OCP)
    Ad = dev(A)
    ws = zeros_ws(vla.vla_gemm_workspace_bytes(M, N, K, w.wfmt))
    Y = torch.empty(M * N, dtype=torch.int16, device="cuda")
    vla.vla_set_wait_limit(1)
    try:
        for _ in range(4):
            vla.vla_gemm_fp8w(Ad, None, w.q, w.s, None, None, Y, ws, ws.numel(), M, N, K)
    finally:
        vla.vla_set_wait_limit(0)
    torch.cuda.synchronize()
    assert int(host(ws[:61440]).view(np.uint32).sum()) == 0
    assert np.isnan(bf16_f64(host(Y, np.uint16))).any()      # the unfinished slices read NaN
    with pytest.raises(RuntimeError, match="wait gave up"):
        vla.vla_workspace_status(ws)
    vla.vla_workspace_status(ws)                             # the query cleared the word
    y, _ = run_gemm(Ad, w, M)
    ref, yabs = oracle.gemm(bf16_f64(A), w.w)
    assert_gemm_close(y, ref, yabs)


@pytest.mark.parametrize("M,N,K", [(50, 4096, 1024), (50, 1024, 4096), (768, 512, 4096)])
def test_repeat_runs_bitwise_equal(M, N, K):
    A = dev(synthetic.activations(M, K, 6500))
    w = Weights(synthetic.weights(N, K, 6501), vla.VLA_WFMT_E4M3_OCP)
    ws = zeros_ws(vla.vla_gemm_workspace_bytes(M, N, K, 1))
    outs = []
    for _ in range(5):
        Y = torch.empty(M * N, dtype=torch.int16, device="cuda")
        vla.vla_gemm_fp8w(A, None, w.q, w.s, None, None, Y, ws, ws.numel(), M, N, K)
        outs.append(host(Y))
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


# ----------------------------------------------------- encoder-size runs

@pytest.mark.parametrize("N,K", [(16384, 2048), (2048, 16384)])
@pytest.mark.parametrize("fp8_act", [False, True])
def test_wide_config_full(N, K, fp8_act):
    """M = 768 encoder shapes at full size, in the launch configuration the
    bench times (2048 -> 16384 on 256-column tiles, 16384 -> 2048 split over
    K): every output against the oracle."""
    M = 768
    print(f"wide config N={N} K={K} fp8_act={fp8_act}", flush=True)
    tid = synthetic.IDS["wide.up.A"] if N == 16384 else synthetic.IDS["wide.down.A"]
    A = synthetic.activations(M, K, tid)
    w = Weights(synthetic.weights(N, K, tid + 1), vla.VLA_WFMT_E4M3_OCP)
    Ad = dev(A)
    if fp8_act:
        qa = torch.empty(M * K, dtype=torch.uint8, device="cuda")
        sa = torch.empty(1, dtype=torch.float32, device="cuda")
        wq = torch.zeros(vla.vla_quantize_act_workspace_bytes(M, K), dtype=torch.uint8, device="cuda")
        vla.vla_quantize_act(Ad, qa, sa, wq, wq.numel(), M, K)
        y, _ = run_gemm(qa, w, M, s_a=sa)
        ref_qa, ref_sa = oracle.quantize_act(A)
        assert np.array_equal(host(qa).reshape(M, K), ref_qa)
        a_val = oracle.decode(ref_qa, OCP) * np.float64(ref_sa)
    else:
        y, _ = run_gemm(Ad, w, M)
        a_val = bf16_f64(A)
    ref, yabs = oracle.gemm(a_val, w.w)
    assert_gemm_close(y, ref, yabs)


# ------------------------------------------------- the pages' own row counts

@pytest.mark.parametrize("wfmt", [vla.VLA_WFMT_E4M3_OCP, vla.VLA_WFMT_BF16])
@pytest.mark.parametrize("N,K,bias", [(4096, 1024, False), (1024, 4096, False), (8192, 1024, True)])
def test_page_decoder_rows(wfmt, N, K, bias):
    """The 10-row action decoder the pages time: up, down, and the merged
    gate/up GEMM (10, 8192, 1024) with its bias epilogue."""
    check(10, N, K, wfmt, 7000 + N // 16 + K // 32, bias=bias)


@pytest.mark.parametrize("N,K", [(16384, 2048), (2048, 16384)])
@pytest.mark.parametrize("fp8_act", [False, True])
def test_page_encoder_rows(N, K, fp8_act):
    """The 571-row encoder GEMMs the pages time (two full 192-row blocks and a
    ragged 187-row one): every output against the oracle."""
    M = 571
    print(f"encoder rows M={M} N={N} K={K} fp8_act={fp8_act}", flush=True)
    A = synthetic.activations(M, K, 7100 + N // 1024)
    w = Weights(synthetic.weights(N, K, 7101 + N // 1024), vla.VLA_WFMT_E4M3_OCP)
    Ad = dev(A)
    if fp8_act:
        qa = torch.empty(M * K, dtype=torch.uint8, device="cuda")
        sa = torch.empty(1, dtype=torch.float32, device="cuda")
        wq = torch.zeros(vla.vla_quantize_act_workspace_bytes(M, K), dtype=torch.uint8, device="cuda")
        vla.vla_quantize_act(Ad, qa, sa, wq, wq.numel(), M, K)
        y, _ = run_gemm(qa, w, M, s_a=sa)
        ref_qa, ref_sa = oracle.quantize_act(A)
        a_val = oracle.decode(ref_qa, OCP) * np.float64(ref_sa)
    else:
        y, _ = run_gemm(Ad, w, M)
        a_val = bf16_f64(A)
    ref, yabs = oracle.gemm(a_val, w.w)
    assert_gemm_close(y, ref, yabs)


def test_concurrent_streams_with_separate_workspaces():
    """Split-K GEMMs of different shapes on two streams at once, each with its
    own workspace, give the same bits as the same calls run one after the
    other (the arrival counters live in each call's workspace)."""
    shapes = [(10, 1024, 4096), (768, 2048, 16384)]
    data = []
    for i, (M, N, K) in enumerate(shapes):
        A = dev(synthetic.activations(M, K, 9900 + i))
        w = Weights(synthetic.weights(N, K, 9910 + i), vla.VLA_WFMT_E4M3_OCP)
        ws = zeros_ws(vla.vla_gemm_workspace_bytes(M, N, K, w.wfmt))
        data.append((A, w, ws, M, N, K))

    def call(d, Y, stream=None):
        A, w, ws, M, N, K = d
        vla.vla_gemm_fp8w(A, None, w.q, w.s, None, None, Y, ws, ws.numel(), M, N, K, stream=stream)
    seq = []
    for d in data:
        Y = torch.empty(d[3] * d[4], dtype=torch.int16, device="cuda")
        call(d, Y)
        seq.append(Y)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [[torch.empty(d[3] * d[4], dtype=torch.int16, device="cuda") for _ in range(4)] for d in data]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    for r in range(4):
        for i, d in enumerate(data):
            call(d, outs[i][r], stream=streams[i])
    torch.cuda.synchronize()
    for i in range(len(data)):
        for r in range(4):
            assert torch.equal(outs[i][r], seq[i])
        assert int(host(data[i][2][:61440]).view(np.uint32).sum()) == 0


def test_graph_replays_equal_eager():
    """Split-K skinny and wide GEMMs (FP8 and MXFP4 weights), the fused gate/up
    GEMM with a bias and both activation quantizers captured in one HIP
    graph: every replay, with other eager work and synchronizations between
    replays, equals the eager results bit for bit."""
    calls = []
    for i, (M, N, K) in enumerate([(10, 1024, 4096), (50, 1024, 4096), (768, 2048, 16384), (300, 256, 4096)]):
        A = dev(synthetic.activations(M, K, 9950 + i))
        w = Weights(synthetic.weights(N, K, 9960 + i), vla.VLA_WFMT_E4M3_OCP)
        ws = zeros_ws(vla.vla_gemm_workspace_bytes(M, N, K, w.wfmt))
        Y = torch.empty(M * N, dtype=torch.int16, device="cuda")
        calls.append(lambda A=A, w=w, ws=ws, Y=Y, M=M, N=N, K=K: vla.vla_gemm_fp8w(
            A, None, w.q, w.s, None, None, Y, ws, ws.numel(), M, N, K))
        calls[-1].Y = Y
    M, I, K = 50, 4096, 1024
    Ag = dev(synthetic.activations(M, K, 9970))
    wg = Weights(synthetic.weights(2 * I, K, 9971), vla.VLA_WFMT_E4M3_OCP)
    wsg = zeros_ws(vla.vla_gemm_workspace_bytes(M, 2 * I, K, 1))
    act = torch.empty(M * I, dtype=torch.int16, device="cuda")
    bg = dev(synthetic.activations(1, 2 * I, 9972)[0])
    calls.append(lambda: vla.vla_gemm_fp8w_gelu_mul(Ag, wg.q, wg.s, bg, act, None, wsg, wsg.numel(), M, I, K))
    calls[-1].Y = act
    # wide MXFP4 (128-column tiles, K split over workgroups)
    M4, N4, K4 = 768, 2048, 16384
    A4 = dev(synthetic.activations(M4, K4, 9973))
    q4 = torch.empty(vla.vla_packed_bytes(N4, K4, vla.VLA_WFMT_MXFP4), dtype=torch.uint8, device="cuda")
    vla.vla_quantize_pack(dev(synthetic.weights(N4, K4, 9974)), q4, None, N4, K4, vla.VLA_WFMT_MXFP4, vla.VLA_LAYOUT_MFMA)
    ws4 = zeros_ws(vla.vla_gemm_workspace_bytes(M4, N4, K4, vla.VLA_WFMT_MXFP4))
    Y4 = torch.empty(M4 * N4, dtype=torch.int16, device="cuda")
    calls.append(lambda: vla.vla_gemm_mxfp4w(A4, q4, None, None, Y4, ws4, ws4.numel(), M4, N4, K4))
    calls[-1].Y = Y4
    # activation quantization, dynamic (two kernels through the workspace) and frozen scale
    Mq, Kq = 768, 2048
    Aq = dev(synthetic.activations(Mq, Kq, 9975))
    qa, sa = torch.empty(Mq * Kq, dtype=torch.uint8, device="cuda"), torch.empty(1, dtype=torch.float32, device="cuda")
    wsq = zeros_ws(vla.vla_quantize_act_workspace_bytes(Mq, Kq))
    calls.append(lambda: vla.vla_quantize_act(Aq, qa, sa, wsq, wsq.numel(), Mq, Kq))
    calls[-1].Y = qa
    sfix = dev(np.float32([0.0125]))
    qs = torch.empty(Mq * Kq, dtype=torch.uint8, device="cuda")
    calls.append(lambda: vla.vla_quantize_act_static(Aq, sfix, qs, Mq, Kq))
    calls[-1].Y = qs

    for c in calls:
        c()
    torch.cuda.synchronize()
    eager = [c.Y.clone() for c in calls]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        for c in calls:
            c()
    for r in range(3):
        for c in calls:
            c.Y.zero_()
        junk = torch.randn(1 << 20, device="cuda").sum()     # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for c, e in zip(calls, eager):
            assert torch.equal(c.Y, e), f"replay {r} differs"
        del junk
