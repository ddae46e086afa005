"""Pins of the oracle's FP8 codec and bf16 rounding (CPU only).

Each test checks the oracle against something other than its own formula:
published code values (tests/golden/fp8_codes.txt), torch's float8 and
bfloat16 conversions (library routines), a brute-force nearest search over
the 256 decoded codes, and the invariants the pages state (FNUZ decodes the
same byte to half the OCP value; FNUZ has no -0 and no inf).
"""
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import FNUZ, OCP
from synthetic import rng

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _torch_decode(dtype):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(dtype).to(torch.float64).numpy()


def _read_golden_codes():
    rows = []
    for line in open(os.path.join(GOLDEN, "fp8_codes.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        d, c, v = line.split()
        rows.append((OCP if d == "ocp" else FNUZ, int(c, 16), float(v)))
    return rows


# ------------------------------------------------------------------ decode

def test_decode_golden_values():
    for dialect, code, val in _read_golden_codes():
        got = oracle.decode_table(dialect)[code]
        if np.isnan(val):
            assert np.isnan(got), (dialect, hex(code))
        else:
            assert got == val and np.signbit(got) == np.signbit(val), (dialect, hex(code), got)


@pytest.mark.parametrize("dialect,tdtype", [(OCP, torch.float8_e4m3fn), (FNUZ, torch.float8_e4m3fnuz)])
def test_decode_table_matches_torch(dialect, tdtype):
    ours = oracle.decode_table(dialect)
    ref = _torch_decode(tdtype)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.array_equal(np.signbit(ours[ok]), np.signbit(ref[ok]))


def test_nan_and_zero_counts():
    ocp, fnuz = oracle.decode_table(OCP), oracle.decode_table(FNUZ)
    assert np.isnan(ocp).sum() == 2 and set(np.flatnonzero(np.isnan(ocp))) == {0x7F, 0xFF}
    assert np.isnan(fnuz).sum() == 1 and np.flatnonzero(np.isnan(fnuz))[0] == 0x80
    assert (ocp == 0).sum() == 2          # +0 and -0
    assert (fnuz == 0).sum() == 1         # unsigned zero only
    assert not np.isinf(ocp).any() and not np.isinf(fnuz).any()
    assert np.nanmax(ocp) == 448.0 and np.nanmin(ocp) == -448.0
    assert np.nanmax(fnuz) == 240.0 and np.nanmin(fnuz) == -240.0


def test_halving_identity_exact_code_set():
    """Same byte, FNUZ value is exactly half the OCP value (pages' identity)."""
    ocp, fnuz = oracle.decode_table(OCP), oracle.decode_table(FNUZ)
    holds = [b for b in range(256)
             if np.isfinite(ocp[b]) and np.isfinite(fnuz[b]) and ocp[b] != 0
             and fnuz[b] == ocp[b] / 2]
    assert len(holds) == 252
    assert set(range(256)) - set(holds) == {0x00, 0x80, 0x7F, 0xFF}


@pytest.mark.parametrize("dialect,top", [(OCP, 0x7E), (FNUZ, 0x7F)])
def test_monotone_and_symmetric(dialect, top):
    t = oracle.decode_table(dialect)
    pos = t[: top + 1]
    assert np.all(np.diff(pos) > 0)
    for b in range(1, 128):
        if np.isfinite(t[b]):
            assert t[b | 0x80] == -t[b]


@pytest.mark.parametrize("dialect", [OCP, FNUZ])
def test_every_code_exact_in_bf16(dialect):
    t = oracle.decode_table(dialect)
    fin = t[np.isfinite(t)]
    back = torch.from_numpy(fin).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(back, fin)


# ------------------------------------------------------------------ encode

def _nearest_even_bruteforce(x: np.ndarray, dialect: int) -> np.ndarray:
    """Nearest finite code by exhaustive search; ties -> code with even mantissa.

    Saturation and signed zero follow the format rules: |x| >= max gives the
    max code; zero results keep the sign in OCP (0x80) and are 0x00 in FNUZ.
    """
    table = oracle.decode_table(dialect)
    maxv = 448.0 if dialect == OCP else 240.0
    cand = np.array([b for b in range(128) if np.isfinite(table[b])], np.int64)   # non-negative codes
    vals = table[cand]
    a = np.abs(x.astype(np.float64))
    d = np.abs(a[:, None] - vals[None, :])
    dmin = d.min(axis=1, keepdims=True)
    tie = d == dmin
    # among tied candidates prefer even mantissa (code LSB 0)
    score = np.where(tie, (cand[None, :] & 1), 9)
    pick = cand[np.argmin(score, axis=1)]
    pick = np.where(a >= maxv, 0x7E if dialect == OCP else 0x7F, pick)
    neg = np.signbit(x)
    out = np.where(neg & (pick != 0), pick | 0x80, pick)
    if dialect == OCP:
        out = np.where(neg & (pick == 0), 0x80, out)
    return out.astype(np.uint8)


@pytest.mark.parametrize("dialect", [OCP, FNUZ])
def test_encode_round_trip(dialect):
    t = oracle.decode_table(dialect)
    codes = np.array([b for b in range(256) if not np.isnan(t[b])], np.uint8)
    assert len(codes) == (254 if dialect == OCP else 255)
    x = t[codes].astype(np.float32)
    assert np.array_equal(oracle.encode(x, dialect), codes)


@pytest.mark.parametrize("dialect", [OCP, FNUZ])
def test_encode_midpoints_go_to_even(dialect):
    t = oracle.decode_table(dialect)
    top = 0x7E if dialect == OCP else 0x7F
    pos = t[: top + 1]
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (pos[:-1] + pos[1:]) / 2)  # exact in fp32
    got = oracle.encode(mids, dialect)
    lo = np.arange(top, dtype=np.int64)
    even = np.where(lo % 2 == 0, lo, lo + 1).astype(np.uint8)
    assert np.array_equal(got, even)
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(-np.inf))
    assert np.array_equal(oracle.encode(up, dialect), (lo + 1).astype(np.uint8))
    assert np.array_equal(oracle.encode(dn, dialect), lo.astype(np.uint8))
    # negative side mirrors
    assert np.array_equal(oracle.encode(-mids[1:], dialect), even[1:] | 0x80)


@pytest.mark.parametrize("dialect", [OCP, FNUZ])
def test_encode_bruteforce_nearest(dialect):
    g = rng(9001 + dialect)
    n = 200_000
    mag = np.exp2(g.uniform(-13, 10, n)).astype(np.float32)
    x = np.where(g.random(n) < 0.5, -mag, mag).astype(np.float32)
    x = np.concatenate([x, np.float32([0.0, -0.0, 448.0, -448.0, 464.0, 1e30, -1e30, np.inf, -np.inf,
                                       240.0, 247.9, 248.0, 2.0 ** -11, -(2.0 ** -11), 2.0 ** -10,
                                       2.0 ** -12, -(2.0 ** -12)])])
    assert np.array_equal(oracle.encode(x, dialect), _nearest_even_bruteforce(x, dialect))


@pytest.mark.parametrize("dialect,tdtype,maxv", [(OCP, torch.float8_e4m3fn, 448.0),
                                                 (FNUZ, torch.float8_e4m3fnuz, 240.0)])
def test_encode_matches_torch_in_range(dialect, tdtype, maxv):
    g = rng(9100 + dialect)
    x = (g.standard_normal(300_000) * maxv / 3).astype(np.float32)
    x = x[np.abs(x) < maxv]
    ref = torch.from_numpy(x).to(tdtype).view(torch.uint8).numpy()
    assert np.array_equal(oracle.encode(x, dialect), ref)


def test_encode_specials():
    assert oracle.encode(np.float32([np.nan]), OCP)[0] in (0x7F, 0xFF)
    assert oracle.encode(np.float32([np.nan]), FNUZ)[0] == 0x80
    assert list(oracle.encode(np.float32([np.inf, -np.inf, 1e9, -500.0]), OCP)) == [0x7E, 0xFE, 0x7E, 0xFE]
    assert list(oracle.encode(np.float32([np.inf, -np.inf, 241.0, -300.0]), FNUZ)) == [0x7F, 0xFF, 0x7F, 0xFF]
    # zero sign: OCP keeps it, FNUZ has only +0
    assert list(oracle.encode(np.float32([-0.0, -1e-9, 0.0]), OCP)) == [0x80, 0x80, 0x00]
    assert list(oracle.encode(np.float32([-0.0, -1e-9, 0.0]), FNUZ)) == [0x00, 0x00, 0x00]


# -------------------------------------------------------------------- bf16

def test_bf16_round_matches_torch():
    g = rng(9200)
    x = np.concatenate([
        g.standard_normal(200_000).astype(np.float32),
        (np.exp2(g.uniform(-140, 120, 100_000)) * np.sign(g.standard_normal(100_000))).astype(np.float32),
        np.float32([0.0, -0.0, 1.0, 3.4e38, -3.4e38, 1e-45, np.inf, -np.inf]),
    ])
    # exact bf16 midpoints, both parities
    base = g.integers(0x0080, 0x7F00, 50_000).astype(np.uint32)
    mid = ((base << 16) | 0x8000).view(np.float32)
    x = np.concatenate([x, mid, -mid])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.bf16_round(x.astype(np.float64))
    assert np.array_equal(got, ref)
    assert np.array_equal(oracle.bf16_value(got), torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy())
