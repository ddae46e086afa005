"""Pins of the oracle's MXFP4 codec (E2M1 elements with an E8M0 scale per
32 values): the OCP MX specification's value table (golden fixture), a
brute-force nearest search for the element encoder, and invariants of the
block quantizer (block maximum code, error bound, power-of-two scale
invariance, block independence)."""
import os

import numpy as np
import pytest

import oracle
import synthetic

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mxfp4_e2m1.txt")


def golden():
    fp4, e8 = {}, {}
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        kind, a, b = line.split()
        (fp4 if kind == "fp4" else e8)[int(a)] = float(b)
    return fp4, e8


def test_decode_table_matches_the_specification():
    fp4, e8 = golden()
    table = oracle.fp4_decode_table()
    for c, v in fp4.items():
        assert table[c] == v
        assert table[c | 8] == -v
    assert np.signbit(table[8])
    # E8M0 scales as the dequantizer applies them: code 2 (1.0) x 2^(e - 127)
    for e, lg in e8.items():
        got = oracle.mxfp4_dequant_rows(np.full((1, 32), 2, np.uint8), np.array([[e]], np.uint8))[0, 0]
        assert got == 2.0 ** lg


def nearest_code(x):
    """Brute force over the 8 magnitudes; ties go to the even code."""
    mags = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    a = np.abs(x)[:, None]
    err = np.abs(a - mags[None, :])
    best = np.argmin(err + (np.arange(8)[None, :] & 1) * 1e-12 * (err == err.min(axis=1, keepdims=True)), axis=1)
    return best.astype(np.uint8) | np.where(np.signbit(x), 8, 0).astype(np.uint8)


def test_encode_is_nearest_with_ties_to_even():
    mags = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    mids = (mags[1:] + mags[:-1]) / 2
    r = synthetic.rng(9100)
    xs = np.concatenate([r.uniform(-7.5, 7.5, 20000), mids, -mids, mids + 1e-9, mids - 1e-9, mags, -mags,
                         [6.5, 100.0, -1e30, 0.0, -0.0]])
    got = oracle.fp4_encode(xs)
    want = nearest_code(np.clip(xs, -6.0, 6.0))
    assert np.array_equal(got, want)
    # exact ties: 0.25 -> 0, 0.75 -> 1.0, 1.25 -> 1.0, 1.75 -> 2, 2.5 -> 2, 3.5 -> 4, 5 -> 4
    assert list(oracle.fp4_encode(mids)) == [0, 2, 2, 4, 4, 6, 6]


@pytest.mark.parametrize("N,K", [(16, 64), (64, 1024)])
def test_block_quantizer_invariants(N, K):
    W = synthetic.weights(N, K, 9200 + K)
    W[3, 32:64] = 0.0                                             # one all-zero block
    codes, scales = oracle.mxfp4_quantize_rows(W)
    se = scales.astype(np.int64) - 127
    dq = oracle.mxfp4_dequant_rows(codes, scales)
    blocks = np.abs(W.astype(np.float64)).reshape(N, K // 32, 32)
    # an all-zero block: scale 1, codes 0
    assert scales[3, 1] == 127 and not codes[3, 32:64].any()
    nz = blocks.max(axis=2) > 0
    # the largest code magnitude of every non-zero block is 4 or 6
    vals = np.abs(oracle.fp4_decode_table()[codes]).reshape(N, K // 32, 32).max(axis=2)
    assert set(np.unique(vals[nz])) <= {4.0, 6.0}
    # error bound: half the top spacing, or the clamp from [6, 8) to 6
    bound = np.repeat(2.0 ** (se + 1), 32, axis=1)
    assert (np.abs(dq - W.astype(np.float64)) <= bound).all()
    # the block maximum lies in [2^(e+2), 2^(e+3))
    mx = blocks.max(axis=2)
    assert ((mx[nz] >= 2.0 ** (se[nz] + 2)) & (mx[nz] < 2.0 ** (se[nz] + 3))).all()


def test_power_of_two_scale_invariance_and_block_independence():
    N, K = 16, 256
    W = synthetic.weights(N, K, 9300)
    c0, s0 = oracle.mxfp4_quantize_rows(W)
    for j in (-5, 3):
        c1, s1 = oracle.mxfp4_quantize_rows((W * np.float32(2.0 ** j)).astype(np.float32))
        assert np.array_equal(c0, c1) and np.array_equal(s1.astype(int), s0.astype(int) + j)
    W2 = W.copy()
    W2[:, 64:96] *= 100.0
    c2, s2 = oracle.mxfp4_quantize_rows(W2)
    keep = np.ones(K, bool)
    keep[64:96] = False
    assert np.array_equal(c0[:, keep], c2[:, keep])
    assert np.array_equal(np.delete(s0, 2, axis=1), np.delete(s2, 2, axis=1))
