"""CPU oracle for the FP8/BF16-weight GEMM path (ctypes binding of oracle.c).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  The HIP library never
loads it, and it never loads the HIP library; the two share only the seeded
input generators in ``synthetic``.

Each wrapper takes and returns numpy arrays.  The arithmetic lives in
``oracle.c`` (scalar, fp64 where the pages leave precision open); see that
file's header for the passages each function follows.

Parity status: every function here is pinned by a ``-m "not gpu"`` test that
does not re-type its formula (torch float8 decoders, brute-force nearest
search, numpy matmul, the CDNA3 packing expression printed on the pages,
closed forms and invariants), except the end-to-end chain, whose composed
output beyond the per-stage pins is "parity unpinned" (the pages print no
worked chain value); its per-stage pins are one-hot and zero-weight cases.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

OCP = 1
FNUZ = 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
# ORACLE_SANITIZE=1 loads a build instrumented with AddressSanitizer and
# UndefinedBehaviorSanitizer (the process must preload the ASan runtime).
_SANITIZE = os.environ.get("ORACLE_SANITIZE") == "1"
_LIB = os.path.join(_HERE, "liboracle_san.so" if _SANITIZE else "liboracle.so")
_lock = threading.Lock()
_lib = None

CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
          "-std=c11", "-D_GNU_SOURCE", "-Wall", "-Wextra"]
SANITIZE_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]


def build(force: bool = True, sanitize: bool | None = None) -> str:
    """Compile oracle.c with gcc into liboracle.so next to it (with sanitize,
    or ORACLE_SANITIZE=1: liboracle_san.so, instrumented with ASan + UBSan)."""
    san = _SANITIZE if sanitize is None else sanitize
    lib = os.path.join(_HERE, "liboracle_san.so" if san else "liboracle.so")
    if force or not os.path.exists(lib):
        tmp = lib + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", *CFLAGS, *(SANITIZE_FLAGS if san else []), _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, lib)
    return lib


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB):
                build(force=True)
            lib = ctypes.CDLL(_LIB)
            P = ctypes.c_void_p
            I64 = ctypes.c_int64
            INT = ctypes.c_int
            sig = {
                "orc_fp8_decode": (ctypes.c_double, [ctypes.c_uint8, INT]),
                "orc_fp8_decode_table": (None, [INT, P]),
                "orc_fp8_encode": (ctypes.c_uint8, [ctypes.c_float, INT]),
                "orc_fp8_encode_array": (None, [P, I64, INT, P]),
                "orc_bf16_round_array": (None, [P, I64, P]),
                "orc_bf16_round_f32_array": (None, [P, I64, P]),
                "orc_bf16_to_f64": (None, [P, I64, P]),
                "orc_quantize_rows": (None, [P, I64, I64, INT, P, P]),
                "orc_quantize_act": (None, [P, I64, I64, P, P]),
                "orc_quantize_act_static": (None, [P, I64, I64, ctypes.c_float, P]),
                "orc_reencode_fnuz_to_ocp": (None, [P, P, I64, I64, P, P]),
                "orc_pack": (None, [P, P, I64, I64, INT, INT]),
                "orc_unpack": (None, [P, P, I64, I64, INT, INT]),
                "orc_dequant_rows": (None, [P, P, I64, I64, INT, P]),
                "orc_gemm": (None, [P, P, P, I64, I64, I64, P, P]),
                "orc_gelu_tanh": (ctypes.c_double, [ctypes.c_double]),
                "orc_gelu_mul": (None, [P, P, I64, P]),
                "orc_mlp_chain": (None, [P, P, P, P, P, INT, I64, I64, I64, P, P, P, P]),
                "orc_gate_residual_ada_norm": (None, [P, P, P, P, INT, ctypes.c_float, I64, I64, P, P, P]),
                "orc_fp4_decode": (ctypes.c_double, [ctypes.c_uint8]),
                "orc_fp4_encode": (ctypes.c_uint8, [ctypes.c_double]),
                "orc_mxfp4_quantize_rows": (None, [P, I64, I64, P, P]),
                "orc_mxfp4_dequant_rows": (None, [P, P, I64, I64, P]),
                "orc_decoder_chain": (None, [P, P, P, P, P, P, P, P, I64, INT, ctypes.c_float, INT, I64, I64, I64,
                                             P, P, P]),
            }
            for name, (res, args) in sig.items():
                fn = getattr(lib, name)
                fn.restype = res
                fn.argtypes = args
            _lib = lib
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---------------------------------------------------------------- codec

def decode_table(dialect: int) -> np.ndarray:
    """The 256 decoded values of a dialect, fp64 (NaN where the code is NaN)."""
    out = np.empty(256, np.float64)
    _load().orc_fp8_decode_table(dialect, _p(out))
    return out


def decode(codes, dialect: int) -> np.ndarray:
    return decode_table(dialect)[np.asarray(codes, np.uint8)]


def encode(x, dialect: int) -> np.ndarray:
    """fp32 -> E4M3 codes, nearest-even with saturation."""
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint8)
    _load().orc_fp8_encode_array(_p(x), x.size, dialect, _p(out))
    return out


def bf16_round(x) -> np.ndarray:
    """fp64 values -> bf16 bit patterns (uint16), nearest-even."""
    x = _c(x, np.float64)
    out = np.empty(x.shape, np.uint16)
    _load().orc_bf16_round_array(_p(x), x.size, _p(out))
    return out


def bf16_value(h) -> np.ndarray:
    h = _c(h, np.uint16)
    out = np.empty(h.shape, np.float64)
    _load().orc_bf16_to_f64(_p(h), h.size, _p(out))
    return out


# ------------------------------------------------------------ quantizers

def quantize_rows(W, dialect: int):
    """Per-output-channel quantization of fp32 W (N x K). Returns (q, s)."""
    W = _c(W, np.float32)
    N, K = W.shape
    q = np.empty((N, K), np.uint8)
    s = np.empty(N, np.float32)
    _load().orc_quantize_rows(_p(W), N, K, dialect, _p(q), _p(s))
    return q, s


def quantize_act(A_bits):
    """Per-tensor OCP quantization of bf16 A (uint16 bits, M x K). Returns (qa, s_a)."""
    A = _c(A_bits, np.uint16)
    M, K = A.shape
    qa = np.empty((M, K), np.uint8)
    s = np.empty(1, np.float32)
    _load().orc_quantize_act(_p(A), M, K, _p(qa), _p(s))
    return qa, np.float32(s[0])


def quantize_act_static(A_bits, s_a):
    """OCP codes of bf16 A (uint16 bits, M x K) under a given fp32 scale s_a."""
    A = _c(A_bits, np.uint16)
    M, K = A.shape
    qa = np.empty((M, K), np.uint8)
    _load().orc_quantize_act_static(_p(A), M, K, ctypes.c_float(float(np.float32(s_a))), _p(qa))
    return qa


def reencode_fnuz_to_ocp(q, s):
    """Row-major FNUZ codes + scales -> OCP codes + scales (per-row j rule)."""
    q = _c(q, np.uint8)
    s = _c(s, np.float32)
    N, K = q.shape
    q2 = np.empty_like(q)
    s2 = np.empty_like(s)
    _load().orc_reencode_fnuz_to_ocp(_p(q), _p(s), N, K, _p(q2), _p(s2))
    return q2, s2


# ---------------------------------------------------------------- packer

def pack(W, KL: int = 8) -> np.ndarray:
    """MFMA lane packing of an N x K matrix (any 1/2/4/8-byte dtype) -> flat array."""
    W = np.ascontiguousarray(W)
    N, K = W.shape
    out = np.empty(N * K, W.dtype)
    _load().orc_pack(_p(W), _p(out), N, K, KL, W.itemsize)
    return out


def unpack(flat, N: int, K: int, KL: int = 8) -> np.ndarray:
    flat = np.ascontiguousarray(flat)
    out = np.empty((N, K), flat.dtype)
    _load().orc_unpack(_p(flat), _p(out), N, K, KL, flat.itemsize)
    return out


# ------------------------------------------------------ dequant and GEMM

def dequant_rows(q, s, dialect: int = OCP) -> np.ndarray:
    q = _c(q, np.uint8)
    s = _c(s, np.float32)
    N, K = q.shape
    w = np.empty((N, K), np.float64)
    _load().orc_dequant_rows(_p(q), _p(s), N, K, dialect, _p(w))
    return w


def gemm(a, w, bias=None):
    """fp64 y = a @ w.T (+ bias) and yabs = |a| @ |w|.T (+ |bias|)."""
    a = _c(a, np.float64)
    w = _c(w, np.float64)
    M, K = a.shape
    N, K2 = w.shape
    assert K == K2
    b = None if bias is None else _c(bias, np.float64)
    y = np.empty((M, N), np.float64)
    yabs = np.empty((M, N), np.float64)
    _load().orc_gemm(_p(a), _p(w), _p(b), M, N, K, _p(y), _p(yabs))
    return y, yabs


def gelu_tanh(g: float) -> float:
    return _load().orc_gelu_tanh(float(g))


def gelu_mul(g_bits, u_bits) -> np.ndarray:
    g = _c(g_bits, np.uint16)
    u = _c(u_bits, np.uint16)
    assert g.shape == u.shape
    out = np.empty(g.shape, np.uint16)
    _load().orc_gelu_mul(_p(g), _p(u), g.size, _p(out))
    return out


def mlp_chain(x_in_bits, wgu, sgu, wd, sd, stages: bool = False):
    """Gated-MLP chain on row-major OCP codes.  wgu[l]: 2I x H, wd[l]: H x I.

    Returns x_out bits (M x H), or (x_out, gu, act, x_layers) with stages=True.
    """
    x = _c(x_in_bits, np.uint16)
    M, H = x.shape
    L = len(wgu)
    I = wgu[0].shape[0] // 2
    keep = [_c(w, np.uint8) for w in wgu] + [_c(w, np.uint8) for w in wd]
    keep_s = [_c(v, np.float32) for v in sgu] + [_c(v, np.float32) for v in sd]
    for w in keep[:L]:
        assert w.shape == (2 * I, H)
    for w in keep[L:]:
        assert w.shape == (H, I)
    arr = lambda xs: (ctypes.c_void_p * len(xs))(*[x.ctypes.data for x in xs])
    pgu, pd = arr(keep[:L]), arr(keep[L:])
    psg, psd = arr(keep_s[:L]), arr(keep_s[L:])
    out = np.empty((M, H), np.uint16)
    gu = act = xl = None
    if stages:
        gu = np.empty((L, M, 2 * I), np.uint16)
        act = np.empty((L, M, I), np.uint16)
        xl = np.empty((L, M, H), np.uint16)
    _load().orc_mlp_chain(_p(x), pgu, psg, pd, psd, L, M, H, I, _p(out), _p(gu), _p(act),
                          _p(xl))
    return (out, gu, act, xl) if stages else out


# ------------------------------------------------------- decoder boundary

def gate_residual_ada_norm(residual, out, gate, style, eps: float, style_per_row: bool = True):
    """Fused decoder boundary on bf16 bit patterns (uint16): residual, out,
    gate are M x D; style is M x 3D (per row) or 1 x 3D (shared), blocks
    [scale | shift | next gate].  Returns (r, h, next_gate), each M x D."""
    residual = _c(residual, np.uint16)
    out = _c(out, np.uint16)
    gate = _c(gate, np.uint16)
    style = _c(style, np.uint16)
    M, D = residual.shape
    assert out.shape == (M, D) and gate.shape == (M, D)
    assert style.shape == ((M if style_per_row else 1), 3 * D)
    r = np.empty((M, D), np.uint16)
    h = np.empty((M, D), np.uint16)
    ng = np.empty((M, D), np.uint16)
    _load().orc_gate_residual_ada_norm(_p(residual), _p(out), _p(gate), _p(style), int(bool(style_per_row)),
                                       ctypes.c_float(float(np.float32(eps))), M, D, _p(r), _p(h), _p(ng))
    return r, h, ng


def decoder_chain(x_in, h_in, g_in, wgu, sgu, wd, sd, styles, eps: float, style_per_row: bool = True):
    """Decoder-block chain on row-major OCP codes: per layer the merged
    gate/up GEMM with GELU*mul, the down GEMM, then the fused boundary.
    x_in, h_in, g_in: M x H bf16 bits; styles: L arrays of (M or 1) x 3H.
    Returns (x_out, h_out, g_out)."""
    x = _c(x_in, np.uint16)
    h = _c(h_in, np.uint16)
    g = _c(g_in, np.uint16)
    M, H = x.shape
    L = len(wgu)
    I = wgu[0].shape[0] // 2
    keep = [_c(w, np.uint8) for w in wgu] + [_c(w, np.uint8) for w in wd]
    keep_s = [_c(v, np.float32) for v in sgu] + [_c(v, np.float32) for v in sd]
    rows = M if style_per_row else 1
    st = np.ascontiguousarray(np.stack([_c(s, np.uint16).reshape(rows, 3 * H) for s in styles]))
    assert st.shape == (L, rows, 3 * H)
    arr = lambda xs: (ctypes.c_void_p * len(xs))(*[a.ctypes.data for a in xs])
    xo, ho, go = (np.empty((M, H), np.uint16) for _ in range(3))
    _load().orc_decoder_chain(_p(x), _p(h), _p(g), arr(keep[:L]), arr(keep_s[:L]), arr(keep[L:]),
                              arr(keep_s[L:]), _p(st), rows * 3 * H, int(bool(style_per_row)),
                              ctypes.c_float(float(np.float32(eps))), L, M, H, I, _p(xo), _p(ho), _p(go))
    return xo, ho, go


# ------------------------------------------------------------------ MXFP4

def fp4_decode_table() -> np.ndarray:
    """Values of the 16 E2M1 codes."""
    lib = _load()
    return np.array([lib.orc_fp4_decode(c) for c in range(16)], np.float64)


def fp4_encode(x) -> np.ndarray:
    lib = _load()
    x = np.asarray(x, np.float64)
    return np.array([lib.orc_fp4_encode(float(v)) for v in x.ravel()], np.uint8).reshape(x.shape)


def mxfp4_quantize_rows(W):
    """fp32 W (N x K) -> (codes N x K uint8 in the low nibble, E8M0 scales N x K/32)."""
    W = _c(W, np.float32)
    N, K = W.shape
    codes = np.empty((N, K), np.uint8)
    scales = np.empty((N, K // 32), np.uint8)
    _load().orc_mxfp4_quantize_rows(_p(W), N, K, _p(codes), _p(scales))
    return codes, scales


def mxfp4_dequant_rows(codes, scales) -> np.ndarray:
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    N, K = codes.shape
    out = np.empty((N, K), np.float64)
    _load().orc_mxfp4_dequant_rows(_p(codes), _p(scales), N, K, _p(out))
    return out
