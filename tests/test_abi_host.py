"""C ABI checks that need no GPU: the library loads, exports every entry point
include/vla.h declares, and rejects bad arguments before touching the device."""
import ctypes
import os
import re

import pytest

import bf16_gemm_vla_amd as vla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vla.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(vla_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(vla.LIB_PATH):
        from bf16_gemm_vla_amd import build
        build.build()
    return vla.load()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 17
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(vla.SIGNATURES), set(names) ^ set(vla.SIGNATURES)


def test_status_strings(lib):
    for code in range(7):
        assert vla.status_string(code) not in ("", "unknown status")
    assert vla.status_string(99) == "unknown status"


def test_size_queries(lib):
    assert vla.vla_packed_bytes(64, 128, vla.VLA_WFMT_E4M3_OCP) == 64 * 128
    assert vla.vla_packed_bytes(64, 128, vla.VLA_WFMT_BF16) == 64 * 128 * 2
    assert vla.vla_packed_bytes(0, 128, 1) == 0
    assert vla.vla_gemm_workspace_bytes(50, 4096, 1024, 1) >= 256
    assert vla.vla_gemm_workspace_bytes(50, 1024, 4096, 1) > vla.vla_gemm_workspace_bytes(50, 1024, 128, 1)
    assert vla.vla_quantize_act_workspace_bytes(768, 2048) > 0
    # per-layer x and act buffers for up to 32 layers (the single-launch chain)
    assert vla.vla_mlp_chain_scratch_bytes(50, 1024, 4096) >= 31 * 50 * 1024 * 2 + 32 * 50 * 4096 * 2


def test_size_queries_never_crash(lib):
    """Host-side planning for every shape class, including ones too narrow
    for the fused gate/up epilogue (N/16 odd or 1)."""
    for M in (1, 4, 50, 64, 65, 768, 100000):
        for N in (16, 32, 48, 80, 1024, 4096, 8192, 16384, 1 << 20):
            for K in (32, 64, 96, 1024, 4096, 16384):
                for wfmt in (0, 1):
                    assert vla.vla_gemm_workspace_bytes(M, N, K, wfmt) >= 65536
    assert vla.vla_gemm_workspace_bytes(0, 16, 32, 1) == 0


A16 = 0x10000        # a 16-byte aligned fake address, never dereferenced on error paths


def rc_of(fn, *args):
    return getattr(vla.load(), fn)(*args)


@pytest.mark.parametrize("N,K,code", [(17, 128, vla.VLA_ESHAPE), (64, 100, vla.VLA_ESHAPE),
                                      (0, 128, vla.VLA_EINVAL), (64, -32, vla.VLA_EINVAL)])
def test_gemm_shape_errors(lib, N, K, code):
    rc = rc_of("vla_gemm_fp8w", A16, None, A16, A16, None, None, A16, A16, 1 << 20, 50, N, K, None)
    assert rc == code
    assert "vla_gemm_fp8w" in vla.last_error()


def test_gemm_pointer_errors(lib):
    assert rc_of("vla_gemm_fp8w", None, None, A16, A16, None, None, A16, A16, 1 << 20, 50, 64, 128, None) == vla.VLA_EINVAL
    assert rc_of("vla_gemm_fp8w", A16 + 2, None, A16, A16, None, None, A16, A16, 1 << 20, 50, 64, 128, None) == vla.VLA_EALIGN
    assert rc_of("vla_gemm_fp8w", A16, None, A16, A16, A16 + 8, None, A16, A16, 1 << 20, 50, 64, 128, None) == vla.VLA_EALIGN
    assert rc_of("vla_gemm_bf16", A16, A16, None, None, None, A16, 1 << 20, 50, 64, 128, None) == vla.VLA_EINVAL
    assert rc_of("vla_gemm_fp8w", A16, None, A16, A16, None, None, A16, A16, 1 << 20, 0, 64, 128, None) == vla.VLA_EINVAL


def test_gemm_workspace_too_small(lib):
    # the counter region alone is 64 KiB
    assert rc_of("vla_gemm_fp8w", A16, None, A16, A16, None, None, A16, A16, 65535, 50, 1024, 4096, None) == vla.VLA_EWORKSPACE
    assert rc_of("vla_gemm_fp8w", A16, None, A16, A16, None, None, A16, A16, 65535, 768, 2048, 16384, None) == vla.VLA_EWORKSPACE


def test_gelu_mul_shape_errors(lib):
    # I = 24 is not a multiple of 16
    assert rc_of("vla_gemm_fp8w_gelu_mul", A16, A16, A16, None, A16, None, A16, 1 << 20, 50, 24, 128, None) == vla.VLA_ESHAPE
    # a misaligned bias is rejected before any launch
    assert rc_of("vla_gemm_fp8w_gelu_mul", A16, A16, A16, A16 + 2, A16, None, A16, 1 << 20, 50, 32, 128, None) == vla.VLA_EALIGN


def test_codec_errors(lib):
    assert rc_of("vla_quantize_pack", A16, A16, A16, 64, 128, 7, 1, None) == vla.VLA_EINVAL
    assert rc_of("vla_quantize_pack", A16, A16, A16, 64, 128, 1, 5, None) == vla.VLA_EINVAL
    assert rc_of("vla_quantize_pack", A16, A16, A16, 64, 128, vla.VLA_WFMT_BF16, 1, None) == vla.VLA_EINVAL
    assert rc_of("vla_quantize_pack", A16, A16, None, 64, 128, vla.VLA_WFMT_E4M3_OCP, 1, None) == vla.VLA_EINVAL
    assert rc_of("vla_quantize_pack", A16, A16, A16, 64, 96 + 8, 1, 1, None) == vla.VLA_ESHAPE
    assert rc_of("vla_pack_fp8", A16, A16 + 64, 64, 128, None) == vla.VLA_EINVAL        # overlap
    assert rc_of("vla_reencode_fnuz_to_ocp", A16, A16, A16 + 16, A16, 64, 128, 1, None) == vla.VLA_EINVAL
    assert rc_of("vla_quantize_act", A16, A16, A16, A16, 0, 50, 1024, None) == vla.VLA_EWORKSPACE
    assert rc_of("vla_quantize_act_static", A16, None, A16, 50, 1024, None) == vla.VLA_EINVAL
    assert rc_of("vla_probe_stream_read", A16, 1 << 22, A16, 0, None) == vla.VLA_EINVAL
    assert rc_of("vla_probe_stream_read", A16, (1 << 22) + 8, A16, 256, None) == vla.VLA_ESHAPE
    assert rc_of("vla_probe_stream_read", A16 + 8, 1 << 22, A16, 256, None) == vla.VLA_EALIGN
    assert rc_of("vla_probe_stream_read", None, 1 << 22, A16, 256, None) == vla.VLA_EINVAL
    for form, iters, blocks in ((4, 1, 1), (-1, 1, 1), (0, 0, 1), (0, 1, 0), (0, (1 << 24) + 1, 1), (3, 1, 65537)):
        assert rc_of("vla_probe_mfma_rate", form, A16, iters, A16, None, blocks, None) == vla.VLA_EINVAL
    assert rc_of("vla_probe_mfma_rate", 0, A16 + 4, 1, A16, None, 1, None) == vla.VLA_EALIGN
    assert rc_of("vla_probe_mfma_rate", 0, A16, 1, A16, A16 + 4, 1, None) == vla.VLA_EALIGN
    assert rc_of("vla_probe_mfma_rate", 0, A16, 1, None, None, 1, None) == vla.VLA_EINVAL
    assert rc_of("vla_quantize_act_static", A16, A16 + 4, A16, 50, 1024, None) == vla.VLA_EALIGN
    assert rc_of("vla_quantize_act_static", A16, A16, A16, 50, 1000, None) == vla.VLA_ESHAPE
    assert rc_of("vla_quantize_act_static", A16, A16, A16, 0, 1024, None) == vla.VLA_EINVAL
    assert rc_of("vla_quantize_act_static", A16, A16, A16, 1 << 24, 1 << 20, None) == vla.VLA_ESHAPE


def test_mxfp4_errors(lib):
    assert vla.vla_packed_bytes(64, 128, vla.VLA_WFMT_MXFP4) == 64 * 128 // 2 + 64 * 8       # 4 scales padded to 8
    assert vla.vla_packed_bytes(64, 1024, vla.VLA_WFMT_MXFP4) == 64 * 1024 // 2 + 64 * 32
    assert rc_of("vla_quantize_pack", A16, A16, A16, 64, 128, vla.VLA_WFMT_MXFP4, 1, None) == vla.VLA_EINVAL   # scales given
    assert rc_of("vla_quantize_pack", A16, A16, None, 64, 128, vla.VLA_WFMT_MXFP4, 0, None) == vla.VLA_EINVAL  # row-major
    assert rc_of("vla_gemm_mxfp4w", A16, A16, None, None, A16, A16, 1 << 20, 65, 1024, 1000, None) == vla.VLA_ESHAPE
    assert rc_of("vla_gemm_mxfp4w", A16, A16, None, None, A16, A16, 0, 50, 1024, 1024, None) == vla.VLA_EWORKSPACE
    assert vla.vla_gemm_supported(50, 4096, 1024, vla.VLA_WFMT_MXFP4) == 0
    # M > 64 runs the wide kernel
    assert vla.vla_gemm_supported(100, 4096, 1024, vla.VLA_WFMT_MXFP4) == 0
    assert vla.vla_gemm_supported(768, 2048, 16384, vla.VLA_WFMT_MXFP4) == 0
    assert vla.vla_gemm_supported(768, 16384, 2048, vla.VLA_WFMT_MXFP4) == 0
    assert vla.vla_gemm_supported(50, 4096, 1024, vla.VLA_WFMT_MXFP4, gelu_mul=True) == vla.VLA_EINVAL
    assert vla.vla_gemm_workspace_bytes(10, 1024, 4096, vla.VLA_WFMT_MXFP4) >= 65536


def test_boundary_errors(lib):
    mat = 50 * 1024 * 2
    X, Y, G, S = A16, A16 + mat, A16 + 2 * mat, A16 + 3 * mat       # disjoint inputs
    R, H, NG = A16 + 8 * mat, A16 + 9 * mat, A16 + 10 * mat          # disjoint outputs

    def rc(*args):
        return rc_of("vla_gate_residual_ada_norm", *args)
    assert rc(X, Y, G, S, 1, 1e-6, R, H, NG, 0, 1024, None) == vla.VLA_EINVAL
    assert rc(X, Y, G, S, 1, 1e-6, R, H, NG, 50, 1022, None) == vla.VLA_ESHAPE
    assert rc(X, Y, G, S, 1, 1e-6, R, H, NG, 50, 8196, None) == vla.VLA_ESHAPE
    assert rc(X, Y, G, S, 1, -1.0, R, H, NG, 50, 1024, None) == vla.VLA_EINVAL
    assert rc(X, Y, G, S, 1, float("nan"), R, H, NG, 50, 1024, None) == vla.VLA_EINVAL
    assert rc(None, Y, G, S, 1, 1e-6, R, H, NG, 50, 1024, None) == vla.VLA_EINVAL
    assert rc(X + 8, Y, G, S, 1, 1e-6, R, H, NG, 50, 1024, None) == vla.VLA_EALIGN
    assert rc(X, Y, G, S, 1, 1e-6, R, H, NG + 8, 50, 1024, None) == vla.VLA_EALIGN
    assert rc(X, Y, G, S, 1, 1e-6, R, Y, NG, 50, 1024, None) == vla.VLA_EINVAL        # normalized over out
    assert rc(X, Y, G, S, 1, 1e-6, R, H, S + 16, 50, 1024, None) == vla.VLA_EINVAL    # next_gate in style
    assert rc(X, Y, G, S, 1, 1e-6, X + 16, H, NG, 50, 1024, None) == vla.VLA_EINVAL   # partial alias
    assert rc(X, Y, G, S, 1, 1e-6, R, R + 16, NG, 50, 1024, None) == vla.VLA_EINVAL   # outputs overlap
    # a shared style row is 3D wide: an output right after it is fine, inside it is not
    assert rc(X, Y, G, S, 0, 1e-6, R, H, S + 16, 50, 1024, None) == vla.VLA_EINVAL


def test_decoder_chain_errors(lib):
    arr = (ctypes.c_void_p * 2)(A16, A16)
    M, H, I = 50, 1024, 4096
    need = vla.vla_decoder_chain_scratch_bytes(M, H, I)
    assert need > 5 * M * H * 2 + M * I * 2
    mat = M * H * 2
    XI, HI, GI = 1 << 33, (1 << 33) + mat, (1 << 33) + 2 * mat          # inputs
    XO, HO, GO = 1 << 34, (1 << 34) + mat, (1 << 34) + 2 * mat          # outputs
    SC = 1 << 35

    def rc(style=arr, per_row=1, eps=1e-6, xo=XO, ho=HO, go=GO, scratch=SC, nbytes=need, L=2, Hh=H):
        return rc_of("vla_decoder_chain_enqueue", arr, arr, arr, arr, style, per_row, eps, XI, HI, GI, xo, ho, go,
                     scratch, nbytes, L, M, Hh, I, None)
    assert rc(style=None) == vla.VLA_EINVAL
    assert rc(L=0) == vla.VLA_EINVAL
    assert rc(eps=-1.0) == vla.VLA_EINVAL
    assert rc(nbytes=need - 1) == vla.VLA_EWORKSPACE
    assert rc(ho=HI + 16) == vla.VLA_EINVAL                     # output over an input
    assert rc(go=XO + 16) == vla.VLA_EINVAL                     # outputs overlap
    assert rc(xo=SC + 64) == vla.VLA_EINVAL                     # output in scratch
    assert rc(style=(ctypes.c_void_p * 2)(A16, A16 + 8)) == vla.VLA_EALIGN
    assert rc(style=(ctypes.c_void_p * 2)(A16, None)) == vla.VLA_EINVAL
    assert rc(style=(ctypes.c_void_p * 2)(A16, XO - 64)) == vla.VLA_EINVAL    # output over a style array
    assert rc(Hh=1040) == vla.VLA_ESHAPE
    out = ctypes.c_void_p()
    assert rc_of("vla_decoder_chain_create", arr, arr, arr, arr, arr, 1, 1e-6, XI, HI, GI, XO, HO, GO, SC, need, 2,
                 M, H, I, None, ctypes.byref(out)) == vla.VLA_EINVAL


def test_decoder_chain_staged_errors(lib):
    """The staged decoder chain's own checks (every case fails before any
    device work): stage outputs that overlap one another, an input, an
    output, the scratch or a style array, and unaligned stage outputs."""
    arr = (ctypes.c_void_p * 2)(A16, A16)
    M, H, I, L = 50, 1024, 4096, 2
    need = vla.vla_decoder_chain_scratch_bytes(M, H, I)
    mat = M * H * 2
    XI, HI, GI = 1 << 33, (1 << 33) + mat, (1 << 33) + 2 * mat
    XO, HO, GO = 1 << 34, (1 << 34) + mat, (1 << 34) + 2 * mat
    SC = 1 << 35
    GU, ACT, DN, XL, HL = (1 << 36), (1 << 36) + (1 << 30), (1 << 36) + (2 << 30), (1 << 36) + (3 << 30), (1 << 36) + (4 << 30)

    def rc(gu=GU, act=ACT, dn=DN, xl=XL, hl=HL, style=arr):
        return rc_of("vla_decoder_chain_enqueue_staged", arr, arr, arr, arr, style, 1, 1e-6, XI, HI, GI, XO, HO, GO,
                     gu, act, dn, xl, hl, SC, need, L, M, H, I, None)
    assert rc(act=GU + 64) == vla.VLA_EINVAL                    # two stage outputs overlap
    assert rc(hl=XL + L * mat - 16) == vla.VLA_EINVAL           # h stages run into the x stages
    assert rc(dn=XI + 16) == vla.VLA_EINVAL                     # over an input
    assert rc(xl=HO) == vla.VLA_EINVAL                          # over an output
    assert rc(gu=SC + 4096) == vla.VLA_EINVAL                   # inside the scratch
    assert rc(style=(ctypes.c_void_p * 2)(A16, HL + 512)) == vla.VLA_EINVAL    # a style array inside the h stages
    assert rc(act=ACT + 8) == vla.VLA_EALIGN
    assert rc(hl=HL + 4) == vla.VLA_EALIGN


def test_chain_errors(lib):
    arr = (ctypes.c_void_p * 2)(A16, A16)
    need = vla.vla_mlp_chain_scratch_bytes(50, 1024, 4096)
    big = 1 << 30
    # scratch too small
    assert rc_of("vla_mlp_chain_enqueue", arr, arr, arr, arr, A16, 1 << 33, A16 * 3, need - 1, 2, 50, 1024, 4096, None) == vla.VLA_EWORKSPACE
    # x_out overlapping scratch
    assert rc_of("vla_mlp_chain_enqueue", arr, arr, arr, arr, A16, big + 16, big, need, 2, 50, 1024, 4096, None) == vla.VLA_EINVAL
    # null layer pointer
    bad = (ctypes.c_void_p * 2)(A16, None)
    assert rc_of("vla_mlp_chain_enqueue", bad, arr, arr, arr, A16, 1 << 33, big, need, 2, 50, 1024, 4096, None) == vla.VLA_EINVAL
    # L <= 0, bad I
    assert rc_of("vla_mlp_chain_enqueue", arr, arr, arr, arr, A16, 1 << 33, big, need, 0, 50, 1024, 4096, None) == vla.VLA_EINVAL
    assert rc_of("vla_mlp_chain_enqueue", arr, arr, arr, arr, A16, 1 << 33, big, need, 2, 50, 1024, 4104, None) == vla.VLA_ESHAPE
    # create on the null stream is refused before any capture
    out = ctypes.c_void_p()
    assert rc_of("vla_mlp_chain_create", arr, arr, arr, arr, A16, 1 << 33, big, need, 2, 50, 1024, 4096, None, ctypes.byref(out)) == vla.VLA_EINVAL
    assert out.value is None


def test_chain_handle_state_machine(lib):
    assert rc_of("vla_mlp_chain_replay", None, None) == vla.VLA_ESTATE
    assert "No graph captured".lower() in vla.last_error().lower() or "no graph captured" in vla.last_error()
    assert rc_of("vla_mlp_chain_destroy", None) == vla.VLA_OK
    # an address that was never a handle is rejected, not dereferenced
    assert rc_of("vla_mlp_chain_replay", A16, None) == vla.VLA_ESTATE
    assert rc_of("vla_mlp_chain_destroy", A16) == vla.VLA_ESTATE


def test_python_wrapper_raises(lib):
    with pytest.raises(RuntimeError, match="vla_gemm_bf16: unsupported shape"):
        vla.vla_gemm_bf16(A16, A16, None, None, A16, A16, 1 << 20, 50, 20, 128, stream=0)


def test_every_planned_shape_has_a_compiled_kernel(lib):
    """The planner only ever names kernel configurations the library holds:
    skinny shapes of every row count, the wide encoder shapes and ragged
    tiles, for every operand class."""
    Ns = (16, 32, 48, 64, 96, 160, 272, 1024, 2048, 4096, 8192, 16384)
    Ks = (32, 64, 96, 160, 1024, 1056, 2048, 4096, 16384)
    Ms = tuple(range(1, 65)) + (65, 100, 129, 191, 192, 193, 571, 768, 1000)
    for M in Ms:
        for N in Ns:
            for K in Ks:
                assert vla.vla_gemm_supported(M, N, K, vla.VLA_WFMT_E4M3_OCP) == 0, (M, N, K, "w8a16")
                assert vla.vla_gemm_supported(M, N, K, vla.VLA_WFMT_BF16) == 0, (M, N, K, "bf16")
                assert vla.vla_gemm_supported(M, N, K, vla.VLA_WFMT_E4M3_OCP, fp8_act=True) == 0, (M, N, K, "fp8")
                if N % 32 == 0:
                    assert vla.vla_gemm_supported(M, N, K, vla.VLA_WFMT_E4M3_OCP, gelu_mul=True) == 0, (M, N, K, "gelu")


def test_gemm_supported_rejects_bad_arguments(lib):
    assert vla.vla_gemm_supported(0, 64, 64, 1) == vla.VLA_EINVAL
    assert vla.vla_gemm_supported(4, 24, 64, 1) == vla.VLA_ESHAPE
    assert vla.vla_gemm_supported(4, 64, 48, 1) == vla.VLA_ESHAPE
    assert vla.vla_gemm_supported(4, 64, 64, 7) == vla.VLA_EINVAL
    assert vla.vla_gemm_supported(4, 64, 64, vla.VLA_WFMT_BF16, fp8_act=True) == vla.VLA_EINVAL
    assert vla.vla_gemm_supported(4, 48, 64, 1, gelu_mul=True) == vla.VLA_ESHAPE
    # the wide kernel addresses operands with 32-bit offsets
    assert vla.vla_gemm_supported(768, 1 << 20, 4096, 1) == vla.VLA_ESHAPE


def test_plan_sweep_limits(lib):
    """Every plan the library accepts keeps its split-K partials below 2^32
    bytes (the kernels address them with 32-bit buffer offsets) and its
    counters within the 15360 counter slots, sizes its workspace as counters
    plus partials, and covers the output with its grid; shapes past those
    limits are refused (ESHAPE) instead of planned."""
    Ms = (1, 10, 16, 17, 50, 64, 65, 192, 571, 768, 4096, 1 << 16, 1 << 20)
    Ns = (16, 1024, 4096, 16384, 65536, 1 << 20)
    Ks = (32, 1024, 4096, 16384, 262144, 1 << 20)
    classes = [(vla.VLA_WFMT_E4M3_OCP, False, False), (vla.VLA_WFMT_BF16, False, False),
               (vla.VLA_WFMT_E4M3_OCP, True, False), (vla.VLA_WFMT_E4M3_OCP, False, True),
               (vla.VLA_WFMT_MXFP4, False, False)]
    accepted = refused = 0
    for M in Ms:
        for N in Ns:
            for K in Ks:
                if N * K > (1 << 40):
                    continue
                for wfmt, fp8, gelu in classes:
                    rc, info = vla.vla_gemm_plan(M, N, K, wfmt, fp8, gelu)
                    kernel, tile, gx, gy, gz, ksplit, ws, part, threads, counters = info
                    if rc != 0:
                        assert rc == vla.VLA_ESHAPE, (M, N, K, wfmt, fp8, gelu, rc)
                        refused += 1
                        continue
                    accepted += 1
                    key = (M, N, K, wfmt, fp8, gelu, info)
                    assert kernel == (0 if M <= 64 else 1), key
                    assert 0 <= part < (1 << 32), key
                    assert ws == 65536 + (part if ksplit > 1 else 0), key
                    assert ws <= vla.vla_gemm_workspace_bytes(M, N, K, wfmt), key
                    assert ksplit == 1 or counters <= 15360, key
                    assert threads in (256, 512, 1024), key
                    cols = N // 2 if gelu else N
                    if kernel == 0:
                        per_group = tile * 16 // (2 if gelu else 1)
                        assert gx * per_group >= cols and gy == ksplit, key
                    else:
                        per_group = tile // (2 if gelu else 1)
                        assert gx * per_group >= cols and gy * 192 >= M and gz == ksplit, key
    assert accepted > 1000 and refused > 0


def test_partial_offsets_fit_32_bits(lib):
    """A skinny split-K shape whose partials would span exactly 2^32 bytes
    (M=50, N=65536, K=262144, FP8 weights: 256 splits x 2 row blocks x 2048
    groups of 2 x 2 fragments) is refused rather than run with offsets that
    wrap around."""
    rc, info = vla.vla_gemm_plan(50, 65536, 262144, vla.VLA_WFMT_E4M3_OCP)
    assert rc == vla.VLA_ESHAPE and info[7] >= (1 << 32)
    assert rc_of("vla_gemm_fp8w", A16, None, A16, A16, None, None, A16, A16, 1 << 40, 50, 65536, 262144,
                 None) == vla.VLA_ESHAPE


def test_wait_limit_and_status_arguments(lib):
    """The status query validates its pointer before any device access; the
    wait bound is a plain setter (0 restores the default)."""
    assert rc_of("vla_workspace_status", None, None) == vla.VLA_EINVAL
    assert rc_of("vla_workspace_status", A16 + 4, None) == vla.VLA_EALIGN
    vla.vla_set_wait_limit(5)
    vla.vla_set_wait_limit(0)


def test_staged_chain_errors(lib):
    arr = (ctypes.c_void_p * 2)(A16, A16)
    M, H, I, L = 50, 1024, 4096, 2
    need = vla.vla_mlp_chain_scratch_bytes(M, H, I)
    XI, XO, SC = 1 << 33, 1 << 34, 1 << 35
    GU, ACT, DN, XL = 1 << 36, 1 << 37, 1 << 38, 1 << 39

    def rc(gu=GU, act=ACT, dn=DN, xl=XL):
        return rc_of("vla_mlp_chain_enqueue_staged", arr, arr, arr, arr, XI, XO, gu, act, dn, xl, SC, need, L, M,
                     H, I, None)
    assert rc(act=GU + 16) == vla.VLA_EINVAL                          # act over gu
    assert rc(xl=SC + 256) == vla.VLA_EINVAL                          # per-layer x in scratch
    assert rc(dn=XO) == vla.VLA_EINVAL                                # over x_out
    assert rc(gu=GU + 8) == vla.VLA_EALIGN
