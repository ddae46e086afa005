"""ctypes binding of libvla.so (the C ABI in include/vla.h).

Argument marshalling only: every function here has the name and argument
order of its C entry point, takes torch tensors (or None) where C takes a
device pointer and plain ints where C takes sizes, enqueues on the given
stream (default: torch's current stream) and raises RuntimeError on a
non-zero status.  There is no fallback path: if the HIP library has not
been built, loading fails loudly.
"""
from __future__ import annotations

import ctypes
import os
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libvla.so")

VLA_OK = 0
VLA_EINVAL = 1
VLA_ESHAPE = 2
VLA_EALIGN = 3
VLA_EWORKSPACE = 4
VLA_EHIP = 5
VLA_ESTATE = 6

VLA_WFMT_BF16 = 0
VLA_WFMT_E4M3_OCP = 1
VLA_WFMT_E4M3_FNUZ = 2
VLA_WFMT_MXFP4 = 3
VLA_LAYOUT_ROWMAJOR = 0
VLA_LAYOUT_MFMA = 1

P = ctypes.c_void_p
I64 = ctypes.c_int64
INT = ctypes.c_int
SZ = ctypes.c_size_t

# name -> (restype, argtypes); mirrors include/vla.h
SIGNATURES = {
    "vla_status_string": (ctypes.c_char_p, [INT]),
    "vla_last_error": (ctypes.c_char_p, []),
    "vla_set_wait_limit": (None, [ctypes.c_uint32]),
    "vla_workspace_status": (INT, [P, P]),
    "vla_gemm_plan": (INT, [I64, I64, I64, INT, INT, INT, P, INT]),
    "vla_mlp_chain_enqueue_staged": (INT, [P, P, P, P, P, P, P, P, P, P, P, SZ, INT, I64, I64, I64, P]),
    "vla_packed_bytes": (SZ, [I64, I64, INT]),
    "vla_quantize_pack": (INT, [P, P, P, I64, I64, INT, INT, P]),
    "vla_pack_fp8": (INT, [P, P, I64, I64, P]),
    "vla_reencode_fnuz_to_ocp": (INT, [P, P, P, P, I64, I64, INT, P]),
    "vla_quantize_act_workspace_bytes": (SZ, [I64, I64]),
    "vla_quantize_act": (INT, [P, P, P, P, SZ, I64, I64, P]),
    "vla_quantize_act_static": (INT, [P, P, P, I64, I64, P]),
    "vla_probe_stream_read": (INT, [P, SZ, P, INT, P]),
    "vla_probe_mfma_rate": (INT, [INT, P, INT, P, P, INT, P]),
    "vla_gate_residual_ada_norm": (INT, [P, P, P, P, INT, ctypes.c_float, P, P, P, I64, I64, P]),
    "vla_gemm_workspace_bytes": (SZ, [I64, I64, I64, INT]),
    "vla_gemm_supported": (INT, [I64, I64, I64, INT, INT, INT]),
    "vla_gemm_fp8w": (INT, [P, P, P, P, P, P, P, P, SZ, I64, I64, I64, P]),
    "vla_gemm_fp8w_noalloc": (INT, [P, P, P, P, P, P, P, I64, I64, I64, P]),
    "vla_gemm_bf16": (INT, [P, P, P, P, P, P, SZ, I64, I64, I64, P]),
    "vla_gemm_mxfp4w": (INT, [P, P, P, P, P, P, SZ, I64, I64, I64, P]),
    "vla_gemm_fp8w_gelu_mul": (INT, [P, P, P, P, P, P, P, SZ, I64, I64, I64, P]),
    "vla_mlp_chain_scratch_bytes": (SZ, [I64, I64, I64]),
    "vla_mlp_chain_fused_supported": (INT, [I64, I64, I64, INT]),
    "vla_decoder_chain_fused_supported": (INT, [I64, I64, I64, INT, INT]),
    "vla_mlp_chain_enqueue": (INT, [P, P, P, P, P, P, P, SZ, INT, I64, I64, I64, P]),
    "vla_mlp_chain_create": (INT, [P, P, P, P, P, P, P, SZ, INT, I64, I64, I64, P, P]),
    "vla_mlp_chain_replay": (INT, [P, P]),
    "vla_decoder_chain_scratch_bytes": (SZ, [I64, I64, I64]),
    "vla_decoder_chain_enqueue": (INT, [P, P, P, P, P, INT, ctypes.c_float, P, P, P, P, P, P, P, SZ, INT, I64, I64,
                                        I64, P]),
    "vla_decoder_chain_enqueue_staged": (INT, [P, P, P, P, P, INT, ctypes.c_float, P, P, P, P, P, P, P, P, P, P, P,
                                               P, SZ, INT, I64, I64, I64, P]),
    "vla_decoder_chain_create": (INT, [P, P, P, P, P, INT, ctypes.c_float, P, P, P, P, P, P, P, SZ, INT, I64, I64,
                                       I64, P, P]),
    "vla_mlp_chain_destroy": (INT, [P]),
}

_lock = threading.Lock()
_lib = None


def load() -> ctypes.CDLL:
    """Load libvla.so (built by ``python -m bf16_gemm_vla_amd.build``)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"HIP library not built: {LIB_PATH} is missing "
                    "(run `python -m bf16_gemm_vla_amd.build`)")
            lib = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(lib, name)
                fn.restype = res
                fn.argtypes = args
            _lib = lib
    return _lib


def status_string(code: int) -> str:
    return load().vla_status_string(code).decode()


def last_error() -> str:
    return load().vla_last_error().decode()


def _check(rc: int, name: str) -> None:
    if rc != VLA_OK:
        raise RuntimeError(f"{name}: {status_string(rc)} ({last_error()})")


def _ptr(t):
    """Device pointer of a tensor, an int address, or NULL for None."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ------------------------------------------------------------------ sizes

def vla_packed_bytes(N: int, K: int, wfmt: int) -> int:
    return load().vla_packed_bytes(N, K, wfmt)


def vla_quantize_act_workspace_bytes(M: int, K: int) -> int:
    return load().vla_quantize_act_workspace_bytes(M, K)


def vla_gemm_workspace_bytes(M: int, N: int, K: int, wfmt: int) -> int:
    return load().vla_gemm_workspace_bytes(M, N, K, wfmt)


def vla_gemm_supported(M: int, N: int, K: int, wfmt: int, fp8_act: bool = False, gelu_mul: bool = False) -> int:
    """Status code (0 = supported) for a GEMM shape; host only, no device work."""
    return load().vla_gemm_supported(M, N, K, wfmt, int(bool(fp8_act)), int(bool(gelu_mul)))


def vla_gemm_plan(M: int, N: int, K: int, wfmt: int, fp8_act: bool = False, gelu_mul: bool = False):
    """(status, info) with info the 10 plan values of include/vla.h; host only."""
    info = (ctypes.c_int64 * 10)()
    rc = load().vla_gemm_plan(M, N, K, wfmt, int(bool(fp8_act)), int(bool(gelu_mul)), info, 10)
    return rc, list(info)


def vla_set_wait_limit(polls: int) -> None:
    load().vla_set_wait_limit(polls)


def vla_workspace_status(ws, stream=None) -> None:
    """Raise RuntimeError if an in-kernel wait of a call that used ws gave up (clears the word)."""
    _check(load().vla_workspace_status(_ptr(ws), _stream(stream)), "vla_workspace_status")


def vla_mlp_chain_scratch_bytes(M: int, H: int, I: int) -> int:
    return load().vla_mlp_chain_scratch_bytes(M, H, I)


def vla_mlp_chain_fused_supported(M: int, H: int, I: int, L: int) -> bool:
    """Whether the chain runs as one persistent launch on the current device."""
    return bool(load().vla_mlp_chain_fused_supported(M, H, I, L))


def vla_decoder_chain_fused_supported(M: int, H: int, I: int, L: int, style_per_row: bool) -> bool:
    """Whether the decoder-block chain of this shape takes the single launch."""
    return bool(load().vla_decoder_chain_fused_supported(M, H, I, L, 1 if style_per_row else 0))


# ----------------------------------------------------------------- codecs

def vla_quantize_pack(W, Wq, scales, N, K, wfmt, layout, stream=None):
    _check(load().vla_quantize_pack(_ptr(W), _ptr(Wq), _ptr(scales), N, K, wfmt, layout,
                                    _stream(stream)), "vla_quantize_pack")


def vla_pack_fp8(q_rowmajor, q_packed, N, K, stream=None):
    _check(load().vla_pack_fp8(_ptr(q_rowmajor), _ptr(q_packed), N, K, _stream(stream)),
           "vla_pack_fp8")


def vla_reencode_fnuz_to_ocp(q_fnuz, s_fnuz, q_ocp, s_ocp, N, K, layout, stream=None):
    _check(load().vla_reencode_fnuz_to_ocp(_ptr(q_fnuz), _ptr(s_fnuz), _ptr(q_ocp), _ptr(s_ocp),
                                           N, K, layout, _stream(stream)),
           "vla_reencode_fnuz_to_ocp")


def vla_quantize_act(A, qa, s_a, ws, ws_bytes, M, K, stream=None):
    _check(load().vla_quantize_act(_ptr(A), _ptr(qa), _ptr(s_a), _ptr(ws), ws_bytes, M, K,
                                   _stream(stream)), "vla_quantize_act")


def vla_gate_residual_ada_norm(residual, out, gate, style, style_per_row, eps, residual_out, normalized,
                               next_gate, M, D, stream=None):
    _check(load().vla_gate_residual_ada_norm(_ptr(residual), _ptr(out), _ptr(gate), _ptr(style),
                                             int(bool(style_per_row)), float(eps), _ptr(residual_out),
                                             _ptr(normalized), _ptr(next_gate), M, D, _stream(stream)),
           "vla_gate_residual_ada_norm")


def vla_probe_stream_read(src, nbytes, sink, blocks, stream=None):
    _check(load().vla_probe_stream_read(_ptr(src), nbytes, _ptr(sink), blocks, _stream(stream)),
           "vla_probe_stream_read")


VLA_MFMA_BF16_32X32X16, VLA_MFMA_BF16_16X16X32, VLA_MFMA_FP8_32X32X64, VLA_MFMA_FP8_16X16X128 = 0, 1, 2, 3


def vla_probe_mfma_rate(form, operands, iters, out, blocks, stream=None, clocks=None):
    _check(load().vla_probe_mfma_rate(form, _ptr(operands), iters, _ptr(out), _ptr(clocks), blocks, _stream(stream)),
           "vla_probe_mfma_rate")


def vla_quantize_act_static(A, s_a, qa, M, K, stream=None):
    _check(load().vla_quantize_act_static(_ptr(A), _ptr(s_a), _ptr(qa), M, K, _stream(stream)),
           "vla_quantize_act_static")


# ------------------------------------------------------------------- GEMM

def vla_gemm_fp8w(A, s_a, Wq, s_w, bias, residual, Y, ws, ws_bytes, M, N, K, stream=None):
    _check(load().vla_gemm_fp8w(_ptr(A), _ptr(s_a), _ptr(Wq), _ptr(s_w), _ptr(bias),
                                _ptr(residual), _ptr(Y), _ptr(ws), ws_bytes, M, N, K,
                                _stream(stream)), "vla_gemm_fp8w")


def vla_gemm_fp8w_noalloc(A, s_a, Wq, s_w, bias, residual, Y, M, N, K, stream=None):
    _check(load().vla_gemm_fp8w_noalloc(_ptr(A), _ptr(s_a), _ptr(Wq), _ptr(s_w), _ptr(bias), _ptr(residual),
                                        _ptr(Y), M, N, K, _stream(stream)), "vla_gemm_fp8w_noalloc")


def vla_gemm_bf16(A, Wq, bias, residual, Y, ws, ws_bytes, M, N, K, stream=None):
    _check(load().vla_gemm_bf16(_ptr(A), _ptr(Wq), _ptr(bias), _ptr(residual), _ptr(Y),
                                _ptr(ws), ws_bytes, M, N, K, _stream(stream)), "vla_gemm_bf16")


def vla_gemm_mxfp4w(A, Wq, bias, residual, Y, ws, ws_bytes, M, N, K, stream=None):
    _check(load().vla_gemm_mxfp4w(_ptr(A), _ptr(Wq), _ptr(bias), _ptr(residual), _ptr(Y), _ptr(ws), ws_bytes,
                                  M, N, K, _stream(stream)), "vla_gemm_mxfp4w")


def vla_gemm_fp8w_gelu_mul(A, Wgu, s_gu, bias, act, gu, ws, ws_bytes, M, I, K, stream=None):
    _check(load().vla_gemm_fp8w_gelu_mul(_ptr(A), _ptr(Wgu), _ptr(s_gu), _ptr(bias), _ptr(act), _ptr(gu),
                                         _ptr(ws), ws_bytes, M, I, K, _stream(stream)),
           "vla_gemm_fp8w_gelu_mul")


# ------------------------------------------------------------------ chain

def _ptr_array(tensors):
    arr = (ctypes.c_void_p * len(tensors))(*[_ptr(t) for t in tensors])
    return arr


def vla_mlp_chain_enqueue(wgu, sgu, wd, sd, x_in, x_out, scratch, scratch_bytes, L, M, H, I,
                          stream=None):
    _check(load().vla_mlp_chain_enqueue(_ptr_array(wgu), _ptr_array(sgu), _ptr_array(wd),
                                        _ptr_array(sd), _ptr(x_in), _ptr(x_out), _ptr(scratch),
                                        scratch_bytes, L, M, H, I, _stream(stream)),
           "vla_mlp_chain_enqueue")


def vla_mlp_chain_enqueue_staged(wgu, sgu, wd, sd, x_in, x_out, gu_out, act_out, down_out, x_layers, scratch,
                                 scratch_bytes, L, M, H, I, stream=None):
    _check(load().vla_mlp_chain_enqueue_staged(_ptr_array(wgu), _ptr_array(sgu), _ptr_array(wd), _ptr_array(sd),
                                               _ptr(x_in), _ptr(x_out), _ptr(gu_out), _ptr(act_out), _ptr(down_out),
                                               _ptr(x_layers), _ptr(scratch), scratch_bytes, L, M, H, I,
                                               _stream(stream)), "vla_mlp_chain_enqueue_staged")


def vla_mlp_chain_create(wgu, sgu, wd, sd, x_in, x_out, scratch, scratch_bytes, L, M, H, I,
                         capture_stream):
    """Returns the chain handle (an opaque int)."""
    out = ctypes.c_void_p()
    _check(load().vla_mlp_chain_create(_ptr_array(wgu), _ptr_array(sgu), _ptr_array(wd),
                                       _ptr_array(sd), _ptr(x_in), _ptr(x_out), _ptr(scratch),
                                       scratch_bytes, L, M, H, I, _stream(capture_stream),
                                       ctypes.byref(out)), "vla_mlp_chain_create")
    return out.value


def vla_decoder_chain_scratch_bytes(M: int, H: int, I: int) -> int:
    return load().vla_decoder_chain_scratch_bytes(M, H, I)


def _decoder_args(wgu, sgu, wd, sd, style, style_per_row, eps, x_in, h_in, gate_in, x_out, h_out, gate_out,
                  scratch, scratch_bytes, L, M, H, I):
    return (_ptr_array(wgu), _ptr_array(sgu), _ptr_array(wd), _ptr_array(sd), _ptr_array(style),
            int(bool(style_per_row)), float(eps), _ptr(x_in), _ptr(h_in), _ptr(gate_in), _ptr(x_out),
            _ptr(h_out), _ptr(gate_out), _ptr(scratch), scratch_bytes, L, M, H, I)


def vla_decoder_chain_enqueue(wgu, sgu, wd, sd, style, style_per_row, eps, x_in, h_in, gate_in, x_out, h_out,
                              gate_out, scratch, scratch_bytes, L, M, H, I, stream=None):
    _check(load().vla_decoder_chain_enqueue(*_decoder_args(wgu, sgu, wd, sd, style, style_per_row, eps, x_in, h_in,
                                                           gate_in, x_out, h_out, gate_out, scratch, scratch_bytes,
                                                           L, M, H, I), _stream(stream)),
           "vla_decoder_chain_enqueue")


def vla_decoder_chain_enqueue_staged(wgu, sgu, wd, sd, style, style_per_row, eps, x_in, h_in, gate_in, x_out,
                                     h_out, gate_out, gu_out, act_out, down_out, x_layers, h_layers, scratch,
                                     scratch_bytes, L, M, H, I, stream=None):
    _check(load().vla_decoder_chain_enqueue_staged(
        _ptr_array(wgu), _ptr_array(sgu), _ptr_array(wd), _ptr_array(sd), _ptr_array(style), int(bool(style_per_row)),
        float(eps), _ptr(x_in), _ptr(h_in), _ptr(gate_in), _ptr(x_out), _ptr(h_out), _ptr(gate_out), _ptr(gu_out),
        _ptr(act_out), _ptr(down_out), _ptr(x_layers), _ptr(h_layers), _ptr(scratch), scratch_bytes, L, M, H, I,
        _stream(stream)), "vla_decoder_chain_enqueue_staged")


def vla_decoder_chain_create(wgu, sgu, wd, sd, style, style_per_row, eps, x_in, h_in, gate_in, x_out, h_out,
                             gate_out, scratch, scratch_bytes, L, M, H, I, capture_stream):
    """Returns the chain handle (an opaque int); replay / destroy it with the
    gated-MLP chain calls."""
    out = ctypes.c_void_p()
    _check(load().vla_decoder_chain_create(*_decoder_args(wgu, sgu, wd, sd, style, style_per_row, eps, x_in, h_in,
                                                          gate_in, x_out, h_out, gate_out, scratch, scratch_bytes,
                                                          L, M, H, I), _stream(capture_stream),
                                           ctypes.byref(out)), "vla_decoder_chain_create")
    return out.value


def vla_mlp_chain_replay(chain, stream=None):
    _check(load().vla_mlp_chain_replay(chain, _stream(stream)), "vla_mlp_chain_replay")


def vla_mlp_chain_destroy(chain):
    _check(load().vla_mlp_chain_destroy(chain), "vla_mlp_chain_destroy")
