"""The GEMM entry point that allocates nothing (vla_gemm_fp8w_noalloc, for
callers that cannot allocate device memory): through the C ABI it gives the
same bits as vla_gemm_fp8w with a caller workspace, on two calls in a row
that share the library's workspace (the second smaller), both within the
oracle's bound; a shape the library's workspace cannot hold is refused
before any device work."""
import numpy as np
import pytest
import torch

import bf16_gemm_vla_amd as vla
import oracle
import synthetic
from oracle import OCP
from tests.gpu_util import Guarded, assert_gemm_close, bf16_f64, dev, host, zeros_ws

pytestmark = pytest.mark.gpu


def _case(M, N, K, seed):
    A = synthetic.activations(M, K, seed)
    W = synthetic.weights(N, K, seed + 1)
    q = torch.empty(N * K, dtype=torch.uint8, device="cuda")
    s = torch.empty(N, dtype=torch.float32, device="cuda")
    vla.vla_quantize_pack(dev(W), q, s, N, K, vla.VLA_WFMT_E4M3_OCP, vla.VLA_LAYOUT_MFMA)
    qo, so = oracle.quantize_rows(W, OCP)
    return A, dev(A), q, s, oracle.dequant_rows(qo, so, OCP)


def test_noalloc_matches_workspace_entry_point():
    # first call: the wide kernel with K split across workgroups (24 MiB of
    # partials in the library's workspace); second, smaller: the skinny kernel
    shapes = [(768, 2048, 16384, 8100), (50, 1024, 4096, 8110)]
    for M, N, K, seed in shapes:
        rc, info = vla.vla_gemm_plan(M, N, K, vla.VLA_WFMT_E4M3_OCP)
        assert rc == 0 and info[6] <= 65536 + (32 << 20)
        print(f"noalloc M={M} N={N} K={K} plan={info}", flush=True)
        A, Ad, q, s, w = _case(M, N, K, seed)
        ws = zeros_ws(vla.vla_gemm_workspace_bytes(M, N, K, vla.VLA_WFMT_E4M3_OCP))
        y_ws = torch.empty(M * N, dtype=torch.int16, device="cuda")
        vla.vla_gemm_fp8w(Ad, None, q, s, None, None, y_ws, ws, ws.numel(), M, N, K)
        y = Guarded(M * N * 2)
        vla.vla_gemm_fp8w_noalloc(Ad, None, q, s, None, None, y.t, M, N, K)
        y.check()
        got = y.numpy(np.uint16).reshape(M, N)
        assert np.array_equal(got, host(y_ws, np.uint16).reshape(M, N))
        ref, yabs = oracle.gemm(bf16_f64(A), w)
        assert_gemm_close(got, ref, yabs)


def test_noalloc_refuses_what_does_not_fit():
    # a skinny K split whose partials would take 2 GiB
    rc, info = vla.vla_gemm_plan(50, 65536, 131072, vla.VLA_WFMT_E4M3_OCP)
    assert rc == 0 and info[6] > 65536 + (32 << 20)
    x = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(RuntimeError, match="vla_gemm_fp8w_noalloc: workspace too small"):
        vla.vla_gemm_fp8w_noalloc(x, None, x, x, None, None, x, 50, 65536, 131072)
