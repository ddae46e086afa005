"""GPU parity of the fused decoder boundary (gated residual + adaptive RMS
norm) against the oracle: the residual and next gate bit for bit, the
normalized output within one bf16 ulp (both sides compute in fp64 and round
once; only the order of the sum of squares differs)."""
import numpy as np
import pytest
import torch

import bf16_gemm_vla_amd as vla
import oracle
import synthetic
from tests.gpu_util import Guarded, dev

pytestmark = pytest.mark.gpu


def run_gpu(x, y, g, st, eps, per_row=True, in_place=False, with_ng=True):
    M, D = x.shape
    xd, yd, gd, sd = dev(x), dev(y), dev(g), dev(st)
    r = None if in_place else Guarded(M * D * 2)
    h = Guarded(M * D * 2)
    ng = Guarded(M * D * 2) if with_ng else None
    vla.vla_gate_residual_ada_norm(xd, yd, gd, sd, per_row, eps, xd if in_place else r.t, h.t,
                                   None if ng is None else ng.t, M, D)
    h.check()
    rb = xd.cpu().numpy().view(np.uint16).reshape(M, D) if in_place else (r.check() or r.numpy(np.uint16).reshape(M, D))
    return rb, h.numpy(np.uint16).reshape(M, D), (None if ng is None else (ng.check() or ng.numpy(np.uint16).reshape(M, D)))


def values(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def assert_close_bf16(got, ref):
    """Within one bf16 ulp of the oracle's bf16 result, value-wise."""
    gv, rv = values(got), values(ref)
    e = np.floor(np.log2(np.maximum(np.abs(rv), 2.0 ** -126)))
    bad = np.abs(gv - rv) > 2.0 ** (e - 7)
    assert not bad.any(), f"{bad.sum()} values off by more than 1 ulp"
    return float((got != ref).mean())


@pytest.mark.parametrize("M,D", [(50, 1024), (1, 4), (3, 1028), (7, 2048), (64, 4096), (2, 8192), (5, 260)])
def test_boundary_matches_oracle(M, D):
    x, y, g, st = synthetic.boundary_inputs(M, D, M)
    r, h, ng = run_gpu(x, y, g, st, 1e-6)
    rr, rh, rng_ = oracle.gate_residual_ada_norm(x, y, g, st, 1e-6)
    assert np.array_equal(r, rr)
    assert np.array_equal(ng, rng_)
    mismatch = assert_close_bf16(h, rh)
    assert mismatch < 1e-3


@pytest.mark.parametrize("eps", [0.0, 0.5])
def test_boundary_shared_style_and_eps(eps):
    M, D = 50, 1024
    x, y, g, st = synthetic.boundary_inputs(M, D, 1)
    r, h, ng = run_gpu(x, y, g, st, eps, per_row=False)
    rr, rh, rng_ = oracle.gate_residual_ada_norm(x, y, g, st, eps, style_per_row=False)
    assert np.array_equal(r, rr) and np.array_equal(ng, rng_)
    assert_close_bf16(h, rh)


def test_boundary_in_place_residual_and_no_next_gate():
    M, D = 50, 1024
    x, y, g, st = synthetic.boundary_inputs(M, D, M)
    r, h, ng = run_gpu(x, y, g, st, 1e-6, in_place=True, with_ng=False)
    rr, rh, _ = oracle.gate_residual_ada_norm(x, y, g, st, 1e-6)
    assert ng is None
    assert np.array_equal(r, rr)
    assert_close_bf16(h, rh)


def test_boundary_residual_ties_and_extremes():
    """Exact bf16 ties in the residual sum go to the even pattern; large and
    tiny magnitudes, a zero row (normalized = shift) and signed zeros."""
    M, D = 4, 64
    x = np.full((M, D), 0x3F80, np.uint16)
    y = np.full((M, D), 0x3B80, np.uint16)
    g = np.full((M, D), 0x3F80, np.uint16)
    x[0, 1::2] = 0x3F81
    x[1] = 0x7F00                      # 2^127
    y[1] = 0x0080                      # 2^-126
    x[2] = 0x0000
    y[2] = 0x0000                      # zero row: r = 0, h = shift
    x[3, :32] = 0x8000                 # -0 + 0 * g
    y[3, :32] = 0x0000
    _, _, _, st = synthetic.boundary_inputs(M, D, M)
    r, h, ng = run_gpu(x, y, g, st, 1e-6)
    rr, rh, rng_ = oracle.gate_residual_ada_norm(x, y, g, st, 1e-6)
    assert np.array_equal(r, rr) and np.array_equal(ng, rng_)
    assert np.array_equal(h[2], rh[2])
    assert_close_bf16(h, rh)


def test_boundary_repeatable_and_capturable():
    """Two eager calls give identical bits; a captured graph replays them."""
    M, D = 50, 1024
    x, y, g, st = synthetic.boundary_inputs(M, D, M)
    xd, yd, gd, sd = dev(x), dev(y), dev(g), dev(st)
    outs = [torch.empty(M * D, dtype=torch.int16, device="cuda") for _ in range(3)]

    def call(s=None):
        vla.vla_gate_residual_ada_norm(xd, yd, gd, sd, True, 1e-6, outs[0], outs[1], outs[2], M, D, stream=s)
    call()
    torch.cuda.synchronize()
    first = [o.clone() for o in outs]
    gr = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(gr, stream=s):
        call(s)
    for _ in range(3):
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        for o, f in zip(outs, first):
            assert torch.equal(o, f)
