"""Pins of the oracle's fused decoder boundary (gated residual + adaptive RMS
norm), against definitions that share nothing with its code: a brute-force
nearest-bf16 search (ties to the even pattern) on the exact fp64 residual,
and torch's own fp64 rms_norm for the normalized output (CPU only)."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synthetic


def bf16_values(bits):
    """Exact values of bf16 bit patterns (uint16) as fp64, via fp32 bits."""
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def nearest_bf16(v):
    """Brute force: among the bf16 patterns next to fp32(v), the one nearest
    to the exact v, ties to the even pattern."""
    v = np.asarray(v, np.float64)
    base = (np.float32(0) + v.astype(np.float32)).view(np.uint32) >> 16
    best = None
    best_err = None
    for d in (-1, 0, 1):
        c = (base.astype(np.int64) + d) & 0xFFFF
        c = c.astype(np.uint16)
        err = np.abs(bf16_values(c) - v)
        if best is None:
            best, best_err = c.copy(), err
            continue
        better = (err < best_err) | ((err == best_err) & ((c & 1) == 0) & ((best & 1) == 1))
        best = np.where(better, c, best)
        best_err = np.where(better, err, best_err)
    return best


def ulp_bf16(v):
    e = np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** -126)))
    return 2.0 ** (e - 7)


@pytest.mark.parametrize("M,D", [(4, 64), (50, 1024), (3, 2048)])
def test_residual_is_nearest_bf16_of_exact_sum(M, D):
    x, y, g, st = synthetic.boundary_inputs(M, D, M)
    r, _, _ = oracle.gate_residual_ada_norm(x, y, g, st, 1e-6)
    exact = bf16_values(x) + bf16_values(y) * bf16_values(g)    # exact in fp64
    assert np.array_equal(r, nearest_bf16(exact))


def test_residual_ties_and_zero_gate():
    """A sum exactly halfway between two bf16 values goes to the even
    pattern; a zero gate leaves the residual bits unchanged."""
    D = 64
    x = np.full((1, D), 0x3F80, np.uint16)            # 1.0
    y = np.full((1, D), 0x3B80, np.uint16)            # 2^-8: 1 + 2^-8 is a tie
    g = np.full((1, D), 0x3F80, np.uint16)            # 1.0
    x[0, 1] = 0x3F81                                   # 1 + 2^-7 (odd): + 2^-8 is a tie, goes up
    st = np.zeros((1, 3 * D), np.uint16)
    r, _, _ = oracle.gate_residual_ada_norm(x, y, g, st, 1e-6)
    assert r[0, 0] == 0x3F80 and r[0, 1] == 0x3F82
    x2, y2, _, st2 = synthetic.boundary_inputs(8, 256, 8)
    r2, _, _ = oracle.gate_residual_ada_norm(x2, y2, np.zeros_like(x2), st2, 1e-6)
    assert np.array_equal(r2, x2)


@pytest.mark.parametrize("eps", [1e-6, 0.5])
@pytest.mark.parametrize("per_row", [True, False])
def test_normalized_against_torch_rms_norm(eps, per_row):
    M, D = 50, 1024
    x, y, g, st = synthetic.boundary_inputs(M, D, M if per_row else 1)
    r, h, ng = oracle.gate_residual_ada_norm(x, y, g, st, eps, style_per_row=per_row)
    r64 = torch.from_numpy(bf16_values(r))
    s64 = torch.from_numpy(bf16_values(st)).expand(M, 3 * D)
    scale, shift = s64[:, :D], s64[:, D:2 * D]
    ref = (F.rms_norm(r64, (D,), eps=float(np.float32(eps))) * (1.0 + scale) + shift).numpy()
    err = np.abs(bf16_values(h) - ref)
    assert (err <= 0.5 * ulp_bf16(ref) * (1 + 1e-9) + 1e-300).all(), float((err / ulp_bf16(ref)).max())
    assert np.array_equal(ng, np.broadcast_to(st[:, 2 * D:], (M, D)))


def test_unit_rms_without_modulation():
    M, D = 16, 1024
    x, y, g, _ = synthetic.boundary_inputs(M, D, M)
    st = np.zeros((M, 3 * D), np.uint16)
    _, h, _ = oracle.gate_residual_ada_norm(x, y, g, st, 0.0)
    ms = (bf16_values(h) ** 2).mean(axis=1)
    assert np.allclose(ms, 1.0, atol=2.0 ** -7)


def test_shared_style_equals_repeated_rows():
    M, D = 6, 128
    x, y, g, st = synthetic.boundary_inputs(M, D, 1)
    a = oracle.gate_residual_ada_norm(x, y, g, st, 1e-6, style_per_row=False)
    b = oracle.gate_residual_ada_norm(x, y, g, np.repeat(st, M, axis=0), 1e-6, style_per_row=True)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


def test_rows_are_independent():
    M, D = 10, 256
    x, y, g, st = synthetic.boundary_inputs(M, D, M)
    full = oracle.gate_residual_ada_norm(x, y, g, st, 1e-6)
    part = oracle.gate_residual_ada_norm(x[3:7], y[3:7], g[3:7], st[3:7], 1e-6)
    for u, v in zip(full, part):
        assert np.array_equal(u[3:7], v)


# ------------------------------------------------------ decoder-block chain

def _chain_layer_weights(L, H, I, seed):
    gate, up, down = synthetic.chain_weights(L, H, I, seed)
    wgu, sgu, wd, sd = [], [], [], []
    for l in range(L):
        q, s = oracle.quantize_rows(np.concatenate([gate[l], up[l]]), oracle.OCP)
        wgu.append(q); sgu.append(s)
        q, s = oracle.quantize_rows(down[l], oracle.OCP)
        wd.append(q); sd.append(s)
    return wgu, sgu, wd, sd


def test_decoder_chain_one_layer_is_the_stage_composition():
    """One layer = merged GEMM, bf16, GELU*mul, down GEMM, bf16, boundary —
    each stage an oracle function pinned on its own."""
    L, M, H, I = 1, 6, 64, 128
    wgu, sgu, wd, sd = _chain_layer_weights(L, H, I, 3)
    x, h, g, st = synthetic.decoder_chain_inputs(L, M, H, M)
    got = oracle.decoder_chain(x, h, g, wgu, sgu, wd, sd, st, 1e-6)
    gu, _ = oracle.gemm(oracle.bf16_value(h), oracle.dequant_rows(wgu[0], sgu[0]))
    gub = oracle.bf16_round(gu)
    act = oracle.gelu_mul(gub[:, :I], gub[:, I:])
    d, _ = oracle.gemm(oracle.bf16_value(act), oracle.dequant_rows(wd[0], sd[0]))
    want = oracle.gate_residual_ada_norm(x, oracle.bf16_round(d), g, st[0], 1e-6)
    for u, v in zip(got, want):
        assert np.array_equal(u, v)


def test_decoder_chain_layers_compose():
    L, M, H, I = 3, 5, 64, 96
    wgu, sgu, wd, sd = _chain_layer_weights(L, H, I, 4)
    x, h, g, st = synthetic.decoder_chain_inputs(L, M, H, 1)
    full = oracle.decoder_chain(x, h, g, wgu, sgu, wd, sd, st, 1e-6, style_per_row=False)
    cur = (x, h, g)
    for l in range(L):
        cur = oracle.decoder_chain(*cur, wgu[l:l + 1], sgu[l:l + 1], wd[l:l + 1], sd[l:l + 1], st[l:l + 1], 1e-6,
                                   style_per_row=False)
    for u, v in zip(full, cur):
        assert np.array_equal(u, v)


def test_decoder_chain_zero_down_weights_keep_the_residual():
    """All-zero down weights: d = 0, so the residual passes through bit for bit
    and the next input is the adaptive norm of the unchanged residual."""
    L, M, H, I = 2, 4, 64, 64
    wgu, sgu, _, _ = _chain_layer_weights(L, H, I, 5)
    wd = [np.zeros((H, I), np.uint8) for _ in range(L)]
    sd = [np.ones(H, np.float32) for _ in range(L)]
    x, h, g, st = synthetic.decoder_chain_inputs(L, M, H, M)
    xo, ho, go = oracle.decoder_chain(x, h, g, wgu, sgu, wd, sd, st, 1e-6)
    assert np.array_equal(xo, x)
    _, h_ref, g_ref = oracle.gate_residual_ada_norm(x, np.zeros_like(x), g, st[-1], 1e-6)
    assert np.array_equal(ho, h_ref) and np.array_equal(go, g_ref)
