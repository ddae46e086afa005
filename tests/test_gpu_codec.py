"""GPU parity of the codecs: quantize+pack, FP8 pack, FNUZ->OCP re-encode and
activation quantization must equal the oracle byte for byte."""
import numpy as np
import pytest
import torch

import bf16_gemm_vla_amd as vla
import oracle
import synthetic
from oracle import FNUZ, OCP
from tests.gpu_util import Guarded, dev, host, zeros_ws

pytestmark = pytest.mark.gpu

WFMT = {OCP: vla.VLA_WFMT_E4M3_OCP, FNUZ: vla.VLA_WFMT_E4M3_FNUZ}


def gpu_quantize(W: np.ndarray, wfmt: int, layout: int):
    N, K = W.shape
    nbytes = vla.vla_packed_bytes(N, K, wfmt)
    q = Guarded(nbytes)
    s = Guarded(N * 4) if wfmt != vla.VLA_WFMT_BF16 else None
    vla.vla_quantize_pack(dev(W), q.t, None if s is None else s.t, N, K, wfmt, layout)
    q.check()
    if s is not None:
        s.check()
    return q, s


def oracle_codes(W, dialect, layout):
    q, s = oracle.quantize_rows(W, dialect)
    return (oracle.pack(q, 8) if layout == vla.VLA_LAYOUT_MFMA else q.reshape(-1)), s


# K a multiple of 512 up to 4096 takes the 1024-thread register-resident kernels, other multiples
# of 128 up to 2048 the 256-thread one, the others the two-pass kernel
SHAPES = [(64, 128, "tiny.W"), (16, 32, "edge.min"), (48, 96, "edge.ragged"), (1024, 4096, "skinny.down.W"),
          (4096, 1024, "skinny.up.W"), (32, 384, "edge.spt3"), (48, 2048, "wide.up.A"), (32, 2560, "edge.k2560")]


@pytest.mark.parametrize("dialect", [OCP, FNUZ])
@pytest.mark.parametrize("layout", [vla.VLA_LAYOUT_MFMA, vla.VLA_LAYOUT_ROWMAJOR])
@pytest.mark.parametrize("N,K,name", SHAPES)
def test_quantize_pack_bit_exact(dialect, layout, N, K, name):
    print(f"quantize_pack dialect={dialect} layout={layout} N={N} K={K}", flush=True)
    W = synthetic.weights(N, K, synthetic.IDS.get(name, 555))
    W[N // 2] = 0.0                                   # all-zero row -> s = 1, codes 0
    W[1, 0] = -0.0
    q, s = gpu_quantize(W, WFMT[dialect], layout)
    ref_q, ref_s = oracle_codes(W, dialect, layout)
    assert np.array_equal(s.numpy(np.float32), ref_s)
    got = q.numpy(np.uint8)
    assert np.array_equal(got, ref_q), f"{(got != ref_q).sum()} bytes differ"


def _e4m3_grid(fnuz):
    """Non-negative finite E4M3 values in increasing order (OCP: max 448; FNUZ:
    every OCP byte's value halved, 0x7F = 240 included)."""
    vals = [m / 8 * 2.0 ** -6 for m in range(8)]
    vals += [2.0 ** (e - 7) * (1 + m / 8) for e in range(1, 16) for m in range(8)]
    vals = vals[:-1]                                      # OCP 0x7F is NaN
    return [v / 2 for v in vals] + [240.0] if fnuz else vals


@pytest.mark.parametrize("dialect", [OCP, FNUZ])
@pytest.mark.parametrize("layout", [vla.VLA_LAYOUT_MFMA, vla.VLA_LAYOUT_ROWMAJOR])
@pytest.mark.parametrize("K", [512, 96])
def test_quantize_pack_rounding_midpoints(dialect, layout, K):
    """Quotients placed within a few fp32 ulps of every E4M3 rounding midpoint
    (and of every grid value, the range top and the subnormal range), where
    a reciprocal-based encoder must fall back to exact division."""
    print(f"quantize_pack midpoints dialect={dialect} layout={layout} K={K}", flush=True)
    grid = _e4m3_grid(dialect == FNUZ)
    fmax = grid[-1]
    amax = np.float32(3.7)
    s = np.float32(np.float64(amax) / fmax)
    targets = [(a + b) / 2 for a, b in zip(grid[:-1], grid[1:])] + grid[1:] + [grid[1] / 2, grid[1] / 4]
    cand = []
    for t in targets:
        w = np.float32(t * np.float64(s))
        for k in range(-4, 5):
            x = w
            for _ in range(abs(k)):
                x = np.nextafter(x, np.float32(np.inf if k > 0 else -np.inf))
            if abs(x) <= amax:
                cand += [x, -x]
    per_row = K - 1
    N = -(-len(cand) // per_row)
    N = -(-N // 16) * 16
    rng = np.random.default_rng(77)
    W = rng.uniform(-3.5, 3.5, size=(N, K)).astype(np.float32)
    flat = W[:, 1:].reshape(-1)
    flat[:len(cand)] = np.float32(cand)
    W[:, 1:] = flat.reshape(N, per_row)
    W[:, 0] = np.where(np.arange(N) % 2 == 0, amax, -amax)
    q, sg = gpu_quantize(W, WFMT[dialect], layout)
    ref_q, ref_s = oracle_codes(W, dialect, layout)
    assert np.array_equal(sg.numpy(np.float32), ref_s)
    got = q.numpy(np.uint8)
    assert np.array_equal(got, ref_q), f"{(got != ref_q).sum()} bytes differ"


def test_quantize_pack_bf16_bit_exact():
    N, K = 256, 512
    W = synthetic.weights(N, K, 556)
    W[3, :8] = np.float32([1.0, -2.5, 3.0039062, 1e-40, -1e-38, 65504.0, 3.3895314e38, 0.0])
    q, _ = gpu_quantize(W, vla.VLA_WFMT_BF16, vla.VLA_LAYOUT_MFMA)
    ref = oracle.pack(oracle.bf16_round(W.astype(np.float64)), 8)
    assert np.array_equal(q.numpy(np.uint16), ref)


def test_dialect_config_fnuz_reencode_pack():
    """16384 x 2048 N(0, 0.02) -> FNUZ (absmax/240) -> OCP -> MFMA pack, byte for byte."""
    N, K = 16384, 2048
    print("dialect config: quantize FNUZ row-major, re-encode, pack", flush=True)
    W = synthetic.weights(N, K, synthetic.IDS["dialect.W"])
    q, s = gpu_quantize(W, vla.VLA_WFMT_E4M3_FNUZ, vla.VLA_LAYOUT_ROWMAJOR)
    q2, s2 = Guarded(N * K), Guarded(N * 4)
    vla.vla_reencode_fnuz_to_ocp(q.t, s.t, q2.t, s2.t, N, K, vla.VLA_LAYOUT_ROWMAJOR)
    qp = Guarded(N * K)
    vla.vla_pack_fp8(q2.t, qp.t, N, K)
    for b in (q2, s2, qp):
        b.check()
    ref_q, ref_s = oracle.quantize_rows(W, FNUZ)
    assert np.array_equal(q.numpy(np.uint8).reshape(N, K), ref_q)
    ref_q2, ref_s2 = oracle.reencode_fnuz_to_ocp(ref_q, ref_s)
    assert np.array_equal(s2.numpy(np.float32), ref_s2)
    assert np.array_equal(q2.numpy(np.uint8).reshape(N, K), ref_q2)
    assert np.array_equal(qp.numpy(np.uint8), oracle.pack(ref_q2, 8))


@pytest.mark.parametrize("K", [256, 160, 2048])
@pytest.mark.parametrize("layout", [vla.VLA_LAYOUT_MFMA, vla.VLA_LAYOUT_ROWMAJOR])
def test_reencode_j1_rows_and_in_place(layout, K):
    """Rows without +-240 keep their bytes at half scale; in-place use allowed."""
    g = synthetic.rng(4242)
    N = 64
    allowed = np.array([b for b in range(256) if b not in (0x7F, 0xFF, 0x80)], np.uint8)
    q = allowed[g.integers(0, len(allowed), (N, K))]
    q[::3, 5] = 0x7F            # every third row holds +240 -> j = 0
    q[1, 7] = 0x80              # FNUZ NaN
    s = g.uniform(1e-4, 1e-2, N).astype(np.float32)
    ref_q, ref_s = oracle.reencode_fnuz_to_ocp(q, s)
    stored = oracle.pack(q, 8) if layout == vla.VLA_LAYOUT_MFMA else q.reshape(-1)
    dq, ds = dev(stored), dev(s)
    vla.vla_reencode_fnuz_to_ocp(dq, ds, dq, ds, N, K, layout)       # in place
    want = oracle.pack(ref_q, 8) if layout == vla.VLA_LAYOUT_MFMA else ref_q.reshape(-1)
    assert np.array_equal(host(dq), want)
    assert np.array_equal(host(ds), ref_s)


@pytest.mark.parametrize("N,K", [(80, 160), (32, 8192), (16, 8224), (48, 32)])
def test_pack_fp8_matches_oracle(N, K):
    """K up to 8192 packs a tile through LDS, longer rows slot by slot."""
    g = synthetic.rng(4243 + K)
    q = g.integers(0, 256, (N, K)).astype(np.uint8)
    out = Guarded(N * K)
    vla.vla_pack_fp8(dev(q), out.t, N, K)
    out.check()
    assert np.array_equal(out.numpy(np.uint8), oracle.pack(q, 8))


@pytest.mark.parametrize("M,K", [(4, 128), (50, 1024), (768, 2048), (3, 32)])
def test_quantize_act_bit_exact(M, K):
    A = synthetic.activations(M, K, 4300 + M)
    qa, sa = Guarded(M * K), Guarded(16)
    ws = zeros_ws(vla.vla_quantize_act_workspace_bytes(M, K))
    vla.vla_quantize_act(dev(A), qa.t, sa.t, ws, ws.numel(), M, K)
    qa.check()
    ref_q, ref_s = oracle.quantize_act(A)
    assert sa.numpy(np.float32)[0] == ref_s
    assert np.array_equal(qa.numpy(np.uint8).reshape(M, K), ref_q)


@pytest.mark.parametrize("top", [0x4100, 0x3F00, 0x7F80])
def test_quantize_act_every_bf16_value(top):
    """Every finite bf16 value below `top` (both signs) in one tensor: the
    codes must equal the oracle's IEEE-division codes bit for bit (the fast
    reciprocal path decides every code away from E4M3 rounding midpoints)."""
    pos = np.arange(0, top, dtype=np.uint16)
    vals = np.concatenate([pos, pos | np.uint16(0x8000)])
    K = 256
    M = (vals.size + K - 1) // K
    A = np.zeros(M * K, np.uint16)
    A[:vals.size] = vals
    A = A.reshape(M, K)
    qa, sa = Guarded(M * K), Guarded(16)
    ws = zeros_ws(vla.vla_quantize_act_workspace_bytes(M, K))
    vla.vla_quantize_act(dev(A), qa.t, sa.t, ws, ws.numel(), M, K)
    qa.check()
    ref_q, ref_s = oracle.quantize_act(A)
    assert sa.numpy(np.float32)[0] == ref_s
    got = qa.numpy(np.uint8).reshape(M, K)
    bad = got != ref_q
    assert not bad.any(), f"{bad.sum()} codes differ, first input {hex(int(A[bad][0]))}"


def gpu_act_static(A, s):
    M, K = A.shape
    qa, sa = Guarded(M * K), Guarded(16)
    sa.t[:4].copy_(torch.from_numpy(np.array([s], np.float32).view(np.uint8)))
    vla.vla_quantize_act_static(dev(A), sa.t, qa.t, M, K)
    qa.check()
    return qa.numpy(np.uint8).reshape(M, K)


@pytest.mark.parametrize("M,K", [(4, 128), (50, 1024), (768, 2048), (3, 32)])
@pytest.mark.parametrize("scale_mul", [1.0, 0.25, 3.0])
def test_quantize_act_static_bit_exact(M, K, scale_mul):
    A = synthetic.activations(M, K, 4400 + M)
    _, s_dyn = oracle.quantize_act(A)
    s = np.float32(s_dyn * np.float32(scale_mul))
    assert np.array_equal(gpu_act_static(A, s), oracle.quantize_act_static(A, s))


@pytest.mark.parametrize("s", [1.0, 2.0 ** -7, 3.0e-3, 0.0, float("inf")])
def test_quantize_act_static_every_bf16_value(s):
    """Every bf16 bit pattern (both signs, infinities and NaNs included) under
    a frozen scale, including the degenerate scales 0 and inf."""
    A = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16).reshape(256, 256)
    got = gpu_act_static(A, np.float32(s))
    ref = oracle.quantize_act_static(A, np.float32(s))
    # where the quotient is NaN (NaN in, 0/0, inf/inf) IEEE 754 leaves the
    # sign of the result open, so any NaN code (0x7F, 0xFF) is accepted
    nan = (ref & 0x7F) == 0x7F
    assert ((got[nan] & 0x7F) == 0x7F).all()
    bad = (got != ref) & ~nan
    assert not bad.any(), f"{bad.sum()} codes differ, first input {hex(int(A[bad][0]))}"


def test_quantize_act_static_reuses_calibrated_scale():
    """Calibrate on one batch with vla_quantize_act, freeze its device scale,
    encode another batch with it."""
    M, K = 50, 1024
    A0 = synthetic.activations(M, K, 4501)
    A1 = synthetic.activations(M, K, 4502)
    qa0, sa = Guarded(M * K), Guarded(16)
    ws = zeros_ws(vla.vla_quantize_act_workspace_bytes(M, K))
    vla.vla_quantize_act(dev(A0), qa0.t, sa.t, ws, ws.numel(), M, K)
    qa1 = Guarded(M * K)
    vla.vla_quantize_act_static(dev(A1), sa.t, qa1.t, M, K)
    qa1.check()
    s0 = oracle.quantize_act(A0)[1]
    assert np.array_equal(qa1.numpy(np.uint8).reshape(M, K), oracle.quantize_act_static(A1, s0))


@pytest.mark.parametrize("blocks", [1, 256, 1024])
def test_probe_stream_read_runs(blocks):
    """The probe reads every byte and writes nothing for all-zero data."""
    src = torch.zeros(1 << 22, dtype=torch.uint8, device="cuda")
    sink = Guarded(16, fill=0xA5)
    vla.vla_probe_stream_read(src, src.numel(), sink.t, blocks)
    sink.check()
    assert (sink.numpy(np.uint8) == 0xA5).all()


def test_quantize_act_all_zero():
    M, K = 8, 64
    A = np.zeros((M, K), np.uint16)
    qa, sa = Guarded(M * K), Guarded(16)
    ws = zeros_ws(vla.vla_quantize_act_workspace_bytes(M, K))
    vla.vla_quantize_act(dev(A), qa.t, sa.t, ws, ws.numel(), M, K)
    assert sa.numpy(np.float32)[0] == 1.0
    assert np.all(qa.numpy(np.uint8) == 0)
