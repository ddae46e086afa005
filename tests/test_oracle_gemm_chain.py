"""Pins of the oracle's GEMM, GELU-tanh*mul and gated-MLP chain (CPU only)."""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from oracle import OCP
from synthetic import rng


def bf16_bits_to_f64(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()


def f64_to_bf16_bits(x):
    """Library rounding for pins: torch rounds fp64 -> fp32 -> bf16, exact here because
    every input passed in has at most 24 significant bits."""
    t = torch.from_numpy(np.ascontiguousarray(x, np.float64))
    assert torch.equal(t.to(torch.float32).to(torch.float64), t)
    return t.to(torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


# ------------------------------------------------------------------- GEMM

def test_gemm_matches_numpy_matmul():
    A = bf16_bits_to_f64(synthetic.activations(4, 128, synthetic.IDS["tiny.A"]))
    q, s = oracle.quantize_rows(synthetic.weights(64, 128, synthetic.IDS["tiny.W"]), OCP)
    w = oracle.dequant_rows(q, s)
    bias = rng(800).standard_normal(64)
    y, yabs = oracle.gemm(A, w, bias)
    assert np.allclose(y, A @ w.T + bias, rtol=1e-13, atol=1e-13)
    assert np.allclose(yabs, np.abs(A) @ np.abs(w).T + np.abs(bias), rtol=1e-13, atol=0)


def test_gemm_tiny_is_exact_in_fp64():
    """K=128 bf16 x fp8*s products fit in 53 bits and their sum is exact: integer check."""
    g = rng(801)
    a = g.integers(-128, 128, (4, 128)).astype(np.float64)
    w = g.integers(-16, 16, (64, 128)).astype(np.float64)
    y, _ = oracle.gemm(a, w)
    ref = a.astype(np.int64) @ w.astype(np.int64).T
    assert np.array_equal(y, ref.astype(np.float64))


def test_gemm_one_hot_permutation():
    """Rows of W that are single 1.0 codes (0x38) with s=1 select columns of A exactly."""
    g = rng(802)
    M, K, N = 5, 96, 48
    A = bf16_bits_to_f64(synthetic.activations(M, K, 803))
    perm = g.integers(0, K, N)
    q = np.zeros((N, K), np.uint8)
    q[np.arange(N), perm] = 0x38
    w = oracle.dequant_rows(q, np.ones(N, np.float32))
    y, _ = oracle.gemm(A, w)
    assert np.array_equal(y, A[:, perm])


def test_gemm_linearity_and_merge():
    A = bf16_bits_to_f64(synthetic.activations(6, 64, 804))
    wg = oracle.dequant_rows(*oracle.quantize_rows(synthetic.weights(32, 64, 805), OCP))
    wu = oracle.dequant_rows(*oracle.quantize_rows(synthetic.weights(32, 64, 806), OCP))
    y_g, _ = oracle.gemm(A, wg)
    y_u, _ = oracle.gemm(A, wu)
    y_m, _ = oracle.gemm(A, np.concatenate([wg, wu]))
    assert np.array_equal(y_m, np.concatenate([y_g, y_u], axis=1))
    y_2a, _ = oracle.gemm(2 * A, wg)
    assert np.array_equal(y_2a, 2 * y_g)


# ------------------------------------------------------------------- GELU

def test_gelu_tanh_matches_torch():
    x = np.concatenate([np.linspace(-12, 12, 4001), [0.0, 1e-8, -1e-8, 30.0, -30.0]])
    ref = torch.nn.functional.gelu(torch.from_numpy(x), approximate="tanh").numpy()
    got = np.array([oracle.gelu_tanh(v) for v in x])
    # cancellation in 1 + tanh(.) for large negative x: bound relative to |x|
    assert np.all(np.abs(got - ref) <= 4e-16 * np.maximum(np.abs(x), 1.0))
    assert oracle.gelu_tanh(0.0) == 0.0 and oracle.gelu_tanh(30.0) == 30.0 and oracle.gelu_tanh(-30.0) == 0.0


def _gelu_definition(g, digits=120):
    """The GELU tanh form evaluated literally, 0.5 g (1 + tanh z) with
    tanh z = (e^{2z} - 1) / (e^{2z} + 1), in decimal arithmetic with 120
    significant digits: the cancellation in 1 + tanh z costs at most ~90 of
    them for |z| <= 100, leaving far more than fp64 needs."""
    import decimal

    with decimal.localcontext() as ctx:
        ctx.prec = digits
        G = decimal.Decimal(float(g))
        c = (decimal.Decimal(2) / decimal.Decimal(ctx.create_decimal("3.14159265358979323846264338327950288419716939937510582097494459230781640628620899862803482534211706798214808651328230664709384460955058223172535940812848111745028410270193852110555964462294895493038196"))).sqrt()
        z = c * (G + decimal.Decimal("0.044715") * G * G * G)
        e = (2 * z).exp()
        return 0.5 * g if z == 0 else float(decimal.Decimal("0.5") * G * (1 + (e - 1) / (e + 1)))


def test_gelu_tanh_matches_high_precision_definition():
    """Including the negative tail where the true value is tiny but not zero
    (g = -8: about -1e-21; g = -10: about -1e-38), which a literal fp64
    evaluation of 1 + tanh z turns into 0."""
    gs = np.concatenate([np.linspace(-14, 6, 401), [-7.5, -8.0, -9.0, -10.0, -10.25, -11.0, -12.0, 1e-6, -1e-6]])
    for g in gs:
        want = _gelu_definition(g)
        got = oracle.gelu_tanh(float(g))
        c = np.sqrt(2 / np.pi)
        z = abs(c * (g + 0.044715 * g ** 3))
        assert abs(got - want) <= 4e-16 * (4 + 2 * z) * abs(want) + 1e-300, (g, got, want)
    assert oracle.gelu_tanh(-8.0) < -1e-22 and oracle.gelu_tanh(-10.0) < -1e-40


def test_gelu_mul_tail_large_up():
    """act = bf16(gelu(g) u) where gelu(g) is tiny and u large (the values
    deep in a chain whose residual stream grows): within half a bf16 ulp of
    the high-precision definition times u."""
    gs = np.array([-8.0, -9.0, -9.5, -10.0, -10.125, -10.25, -10.5], np.float32)
    us = np.array([1.0, 1e3, 1e20, -3e30, 2.5e38], np.float32)
    g_bits = synthetic.fp32_to_bf16_bits(np.repeat(gs, us.size))
    u_bits = synthetic.fp32_to_bf16_bits(np.tile(us, gs.size))
    got = bf16_bits_to_f64(oracle.gelu_mul(g_bits, u_bits))
    for gb, ub, v in zip(bf16_bits_to_f64(g_bits), bf16_bits_to_f64(u_bits), got):
        exact = _gelu_definition(gb) * ub
        if abs(exact) < 2.0 ** -133:                          # below half the smallest bf16 subnormal
            assert v == 0.0
            continue
        e = np.floor(np.log2(abs(exact)))
        ulp = 2.0 ** (max(e, -126) - 7)
        assert abs(v - exact) <= 0.5 * ulp * (1 + 1e-12), (gb, ub, v, exact)


def test_gelu_mul_matches_torch():
    g = synthetic.activations(16, 512, 807)
    u = synthetic.activations(16, 512, 808)
    gf, uf = torch.from_numpy(bf16_bits_to_f64(g)), torch.from_numpy(bf16_bits_to_f64(u))
    ref = (torch.nn.functional.gelu(gf, approximate="tanh") * uf).numpy()
    got = oracle.gelu_mul(g, u)
    # compare against torch's fp64 result rounded by the oracle-independent route:
    # exact bf16 neighbours of the fp64 value
    lo = torch.from_numpy(ref).to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    gv = bf16_bits_to_f64(got)
    ulp = np.abs(np.spacing(lo.astype(np.float32)).astype(np.float64)) * 2 ** 16
    assert np.all(np.abs(gv - ref) <= 0.5 * ulp + 1e-300)
    assert np.mean(gv == lo) > 0.999


# ------------------------------------------------------------------ chain

def _ocp_layer(gate, up, down):
    qgu, sgu = oracle.quantize_rows(np.concatenate([gate, up]), OCP)
    qd, sd = oracle.quantize_rows(down, OCP)
    return qgu, sgu, qd, sd


def test_chain_zero_down_is_identity():
    M, H, I = 3, 64, 96
    x = synthetic.activations(M, H, 900)
    gate, up, _ = synthetic.chain_weights(2, H, I)
    qd = [np.zeros((H, I), np.uint8)] * 2
    sd = [np.ones(H, np.float32)] * 2
    lay = [_ocp_layer(gate[l], up[l], np.zeros((H, I), np.float32)) for l in range(2)]
    out = oracle.mlp_chain(x, [l[0] for l in lay], [l[1] for l in lay], qd, sd)
    assert np.array_equal(out, x)


def test_chain_one_hot_layer_against_torch():
    """One-hot weights make each GEMM a column selection: the layer reduces to torch ops."""
    g = rng(901)
    M, H, I = 4, 64, 32
    x = synthetic.activations(M, H, 902)
    pg, pu, pd = g.integers(0, H, I), g.integers(0, H, I), g.integers(0, I, H)
    qgu = np.zeros((2 * I, H), np.uint8)
    qgu[np.arange(I), pg] = 0x38
    qgu[I + np.arange(I), pu] = 0x38
    qd = np.zeros((H, I), np.uint8)
    qd[np.arange(H), pd] = 0x38
    one = lambda n: np.ones(n, np.float32)
    out, gu, act, _ = oracle.mlp_chain(x, [qgu], [one(2 * I)], [qd], [one(H)], stages=True)
    xf = torch.from_numpy(bf16_bits_to_f64(x))
    gt, ut = xf[:, pg], xf[:, pu]
    act_ref = (torch.nn.functional.gelu(gt, approximate="tanh") * ut)
    act_ref_b = torch.from_numpy(np.ascontiguousarray(act_ref.numpy())).to(torch.float32).to(torch.bfloat16)
    # gelu*u in fp64 vs torch fp64: equal to the last bits except at exact rounding
    # boundaries, which these inputs do not hit
    assert np.array_equal(act[0], act_ref_b.view(torch.int16).numpy().view(np.uint16))
    x_ref = (xf + act_ref_b.to(torch.float64)[:, pd]).to(torch.float32).to(torch.bfloat16)
    assert np.array_equal(out, x_ref.view(torch.int16).numpy().view(np.uint16))
    assert np.array_equal(gu[0][:, :I], x[:, pg]) and np.array_equal(gu[0][:, I:], x[:, pu])


def test_chain_composes_layer_by_layer():
    M, H, I, L = 3, 64, 96, 3
    x = synthetic.activations(M, H, 903)
    gate, up, down = synthetic.chain_weights(L, H, I)
    lay = [_ocp_layer(gate[l], up[l], down[l]) for l in range(L)]
    full, _, _, xl = oracle.mlp_chain(x, *[[l[i] for l in lay] for i in range(4)], stages=True)
    step = x
    for l in range(L):
        step = oracle.mlp_chain(step, [lay[l][0]], [lay[l][1]], [lay[l][2]], [lay[l][3]])
        assert np.array_equal(step, xl[l])
    assert np.array_equal(full, step)


def test_chain_stage_gemm_matches_numpy():
    M, H, I = 5, 64, 96
    x = synthetic.activations(M, H, 904)
    gate, up, down = synthetic.chain_weights(1, H, I)
    qgu, sgu, qd, sd = _ocp_layer(gate[0], up[0], down[0])
    out, gu, act, _ = oracle.mlp_chain(x, [qgu], [sgu], [qd], [sd], stages=True)
    xf = bf16_bits_to_f64(x)
    gu_ref = xf @ oracle.dequant_rows(qgu, sgu).T
    assert np.all(np.abs(bf16_bits_to_f64(gu[0]) - gu_ref) <= np.abs(gu_ref) * 2 ** -8 + 1e-30)
    d_ref = bf16_bits_to_f64(act[0]) @ oracle.dequant_rows(qd, sd).T
    res = bf16_bits_to_f64(out) - xf
    assert np.all(np.abs(res - d_ref) <= (np.abs(d_ref) + np.abs(xf)) * 2 ** -7 + 1e-30)
