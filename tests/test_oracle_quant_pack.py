"""Pins of the oracle's quantizers, FNUZ->OCP re-encoder and MFMA packer (CPU only)."""
import os

import numpy as np
import pytest
import torch

import oracle
import synthetic
from oracle import FNUZ, OCP
from synthetic import rng

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def page_facts():
    facts = {}
    for line in open(os.path.join(GOLDEN, "page_facts.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = line.split()
            facts[k] = v
    return facts


# --------------------------------------------------------------- quantizer

@pytest.mark.parametrize("dialect,tdtype,maxv", [(OCP, torch.float8_e4m3fn, 448.0),
                                                 (FNUZ, torch.float8_e4m3fnuz, 240.0)])
def test_quantize_rows_against_torch(dialect, tdtype, maxv):
    W = synthetic.weights(64, 128, synthetic.IDS["tiny.W"])
    W[5] = 0.0                                 # an all-zero row
    W[7, 3] = 0.5                              # an outlier row
    q, s = oracle.quantize_rows(W, dialect)
    # scale: fp32(absmax / max); check via torch's fp32 division
    amax = torch.from_numpy(np.abs(W).max(axis=1))
    ref_s = torch.where(amax == 0, torch.ones_like(amax), amax / maxv).numpy()
    assert np.array_equal(s, ref_s)
    # codes: torch's own fp32 division and float8 conversion
    ref_q = (torch.from_numpy(W) / torch.from_numpy(s)[:, None]).to(tdtype).view(torch.uint8).numpy()
    assert np.array_equal(q, ref_q)
    assert s[5] == 1.0 and np.all(q[5] == 0)


@pytest.mark.parametrize("dialect", [OCP, FNUZ])
def test_quantize_rows_hits_max_and_error_bound(dialect):
    W = synthetic.weights(256, 512, 77)
    q, s = oracle.quantize_rows(W, dialect)
    maxcode = 0x7E if dialect == OCP else 0x7F
    assert np.all(((q & 0x7F) == maxcode).any(axis=1))
    w = oracle.dequant_rows(q, s, dialect)
    step = 2.0 ** (-9 if dialect == OCP else -10)    # subnormal quantum of the format
    bound = 2.0 ** -4 * np.abs(W.astype(np.float64)) + 0.5 * step * s[:, None].astype(np.float64)
    assert np.all(np.abs(w - W) <= bound)


def test_quantize_rows_is_per_row():
    """quantize(concat) == concat(quantize): the merged gate/up weight."""
    a = synthetic.weights(64, 256, 501)
    b = synthetic.weights(32, 256, 502) * 3
    qa, sa = oracle.quantize_rows(a, OCP)
    qb, sb = oracle.quantize_rows(b, OCP)
    qc, sc = oracle.quantize_rows(np.concatenate([a, b]), OCP)
    assert np.array_equal(qc, np.concatenate([qa, qb])) and np.array_equal(sc, np.concatenate([sa, sb]))


def test_quantize_act_against_torch():
    A = synthetic.activations(50, 1024, 503)
    qa, s_a = oracle.quantize_act(A)
    Af = torch.from_numpy(A.view(np.int16)).view(torch.bfloat16).to(torch.float32)
    ref_s = (Af.abs().max() / 448.0).item()
    assert np.float32(ref_s) == s_a
    ref_q = (Af / torch.tensor(s_a, dtype=torch.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(qa, ref_q)
    assert ((qa & 0x7F) == 0x7E).any()


@pytest.mark.parametrize("scale_mul", [1.0, 0.25, 3.0])
def test_quantize_act_static_against_torch(scale_mul):
    """A frozen scale: torch's float8_e4m3fn cast (round to nearest even) of
    the IEEE quotient, clamped to +-448 first because the cast does not
    saturate.  A scale of a quarter of the absmax scale saturates the tails."""
    A = synthetic.activations(50, 1024, 504)
    _, s_dyn = oracle.quantize_act(A)
    s = np.float32(s_dyn * np.float32(scale_mul))
    qa = oracle.quantize_act_static(A, s)
    Af = torch.from_numpy(A.view(np.int16)).view(torch.bfloat16).to(torch.float32)
    ref = torch.clamp(Af / torch.tensor(s, dtype=torch.float32), -448.0, 448.0)
    assert np.array_equal(qa, ref.to(torch.float8_e4m3fn).view(torch.uint8).numpy())
    if scale_mul == 1.0:
        assert np.array_equal(qa, oracle.quantize_act(A)[0])
    if scale_mul < 1.0:
        assert ((qa & 0x7F) == 0x7E).sum() > 100


def test_quantize_act_static_special_values():
    """Infinities saturate, NaN keeps its sign as 0x7F / 0xFF, -0 stays 0x80,
    and a zero scale turns every finite non-zero value into a saturated code."""
    A = np.array([[0x7F80, 0xFF80, 0x7FC0, 0xFFC0, 0x8000, 0x0000, 0x3F80, 0xBF80] * 4], np.uint16)
    q1 = oracle.quantize_act_static(A, np.float32(1.0))[0, :8]
    assert list(q1) == [0x7E, 0xFE, 0x7F, 0xFF, 0x80, 0x00, 0x38, 0xB8]
    q0 = oracle.quantize_act_static(A, np.float32(0.0))[0, :8]
    assert list(q0[[0, 1, 6, 7]]) == [0x7E, 0xFE, 0x7E, 0xFE]
    assert (q0[[2, 3, 4, 5]] & 0x7F).tolist() == [0x7F] * 4     # NaN in, and 0/0


# ------------------------------------------------------------- re-encoder

def _value(q, s, dialect):
    return oracle.decode_table(dialect)[q] * s[:, None].astype(np.float64)


def test_reencode_same_byte_half_scale_when_no_240():
    """Rows without a +-240 code keep every byte and halve the scale (pages' identity)."""
    g = rng(600)
    allowed = np.array([b for b in range(256) if b not in (0x7F, 0xFF, 0x80)], np.uint8)
    q = allowed[g.integers(0, len(allowed), (32, 256))]
    s = g.uniform(1e-4, 1e-2, 32).astype(np.float32)
    q2, s2 = oracle.reencode_fnuz_to_ocp(q, s)
    assert np.array_equal(q2, q)
    assert np.array_equal(s2, s / np.float32(2))
    assert np.array_equal(_value(q2, s2, OCP), _value(q, s, FNUZ))


def test_reencode_rows_with_240_codes():
    t_f, t_o = oracle.decode_table(FNUZ), oracle.decode_table(OCP)
    codes = np.array([b for b in range(256) if b != 0x80], np.uint8)
    q = np.tile(codes, (4, 1))
    s = np.float32([1.0, 0.5, 3e-3, 7.0])
    q2, s2 = oracle.reencode_fnuz_to_ocp(q, s)
    assert np.array_equal(s2, s)                           # j = 0: scale unchanged
    v_in, v_out = t_f[q[0]], t_o[q2[0]]
    exact = v_in == v_out
    ties = ~exact
    odd_small = [b for b in codes if (b & 0x7F) < 0x10 and (b & 1)]
    assert exact.sum() == 239 and set(codes[ties]) == set(odd_small) and len(odd_small) == 16
    # the 16 ties sit exactly halfway between two OCP codes and go to the even one
    for b, b2 in zip(codes[ties].tolist(), q2[0][ties].tolist()):
        v = t_f[b]
        assert b2 & 1 == 0
        nb = b2 + (1 if abs(v) > abs(t_o[b2]) else -1)
        assert abs(abs(v) - abs(t_o[b2])) == abs(abs(t_o[nb]) - abs(v))
    # NaN stays NaN
    q3, _ = oracle.reencode_fnuz_to_ocp(np.uint8([[0x80, 0x7F]]), np.float32([1.0]))
    assert q3[0, 0] == 0x7F and q3[0, 1] == 0x77   # 0x77 = OCP 240


def test_reencode_dialect_workload_values():
    """Config-like rows (absmax/240): every row holds +-240, so j = 0, error <= half subnormal step."""
    W = synthetic.weights(128, 2048, 31)
    q, s = oracle.quantize_rows(W, FNUZ)
    q2, s2 = oracle.reencode_fnuz_to_ocp(q, s)
    assert np.array_equal(s2, s)
    err = np.abs(_value(q2, s2, OCP) - _value(q, s, FNUZ))
    assert np.all(err <= 2.0 ** -10 * s[:, None])


# ------------------------------------------------------------------ packer

def _cdna3_operand_layout(W_kn: np.ndarray) -> np.ndarray:
    """Packed order for CDNA3's 16x16x16 MFMA, built element by element from
    the instruction's operand lane map ("Real-time VLA inference on AMD
    hardware", section "Packing around the instruction": weights are stored
    in the order the instruction's lanes consume them).

    W is K x N (the page multiplies A x W).  In one 16x16x16 step, lane l
    supplies output column l % 16 and the four consecutive K values
    4 * (l // 16) .. +3 of that step; steps run over K within an output tile
    of 16 columns, tiles over N.  Element (k, n) therefore lands at
    ((tile * steps_per_tile + step) * 64 + lane) * 4 + (k % 4).
    """
    K, N = W_kn.shape
    out = np.empty(K * N, dtype=W_kn.dtype)
    steps = K // 16
    for k in range(K):
        for n in range(N):
            tile, step = n // 16, k // 16
            lane = 16 * ((k % 16) // 4) + n % 16
            out[((tile * steps + step) * 64 + lane) * 4 + k % 4] = W_kn[k, n]
    return out


def test_pack_kl4_matches_cdna3_operand_layout():
    g = rng(700)
    K, N = 64, 48
    W_kn = g.integers(0, 65535, (K, N)).astype(np.uint16)
    ours = oracle.pack(np.ascontiguousarray(W_kn.T), KL=4)
    assert np.array_equal(ours, _cdna3_operand_layout(W_kn))


def test_pack_kl8_lane_slices():
    """KL=8: each of the 64 lanes holds 8 contiguous K values of one output row."""
    facts = page_facts()
    assert int(facts["bf16_values_per_lane_cdna4"]) == 8 and int(facts["lanes_per_wavefront"]) == 64
    N, K = 32, 96
    W = np.arange(N * K, dtype=np.int32).reshape(N, K)
    P = oracle.pack(W, KL=8).reshape(N // 16, K // 32, 64, 8)
    for n0 in range(N // 16):
        for k0 in range(K // 32):
            for lane in range(64):
                row, kg = 16 * n0 + lane % 16, lane // 16
                assert np.array_equal(P[n0, k0, lane], W[row, 32 * k0 + 8 * kg: 32 * k0 + 8 * kg + 8])


@pytest.mark.parametrize("KL,dtype", [(8, np.uint8), (8, np.uint16), (4, np.uint16), (16, np.uint8)])
def test_pack_bijection(KL, dtype):
    g = rng(701)
    N, K = 48, 4 * KL * 3
    W = g.integers(0, 255, (N, K)).astype(dtype)
    P = oracle.pack(W, KL)
    assert sorted(P.tolist()) == sorted(W.reshape(-1).tolist())
    assert np.array_equal(oracle.unpack(P, N, K, KL), W)


def test_down_proj_tile_count_from_page():
    """1024 output columns in 16-column tiles are the 64 workgroups the page reports."""
    facts = page_facts()
    N = int(facts["down_proj_columns"])
    W = np.zeros((N, 32), np.uint8)
    tiles = oracle.pack(W, KL=8).size // (16 * 32)
    assert tiles == int(facts["down_proj_workgroups"])
