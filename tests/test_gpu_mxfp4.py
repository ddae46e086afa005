"""GPU parity of the MXFP4 weight path: quantize + pack (codes and E8M0 block
scales) byte for byte against the oracle, and the skinny (M <= 64) and wide
GEMMs on MXFP4 weights against the oracle's fp64 GEMM on the dequantized
weights (|y - y_ref| <= 4e-3 * sum |a w|), with one-hot lane-map probes that
must reproduce A's columns bit for bit."""
import numpy as np
import pytest
import torch

import bf16_gemm_vla_amd as vla
import oracle
import synthetic
from tests.gpu_util import Guarded, assert_gemm_close, bf16_f64, dev, host, zeros_ws

pytestmark = pytest.mark.gpu


def oracle_packed(W):
    """The packed bytes vla_quantize_pack(MXFP4) must produce, from the
    oracle's codes and scales: codes in the FP8 fragment order two per byte
    (even position low), then the E8M0 bytes row-major, rows padded with 127
    to K/32 rounded up to 8."""
    N, K = W.shape
    codes, scales = oracle.mxfp4_quantize_rows(W)
    order = oracle.pack(codes, 8).astype(np.uint8)          # one code per element, fragment order
    packed = (order[0::2] | (order[1::2] << 4)).astype(np.uint8)
    P = (K // 32 + 7) // 8 * 8
    sc = np.full((N, P), 127, np.uint8)
    sc[:, :K // 32] = scales
    return np.concatenate([packed, sc.reshape(-1)]), codes, scales


def gpu_pack(W):
    N, K = W.shape
    q = Guarded(vla.vla_packed_bytes(N, K, vla.VLA_WFMT_MXFP4))
    vla.vla_quantize_pack(dev(W), q.t, None, N, K, vla.VLA_WFMT_MXFP4, vla.VLA_LAYOUT_MFMA)
    q.check()
    return q


def special_weights(N, K, seed):
    W = synthetic.weights(N, K, seed)
    W[0, :32] = 0.0                                   # all-zero block
    W[1, :32] = -0.0
    W[2, 32:64] *= np.float32(1e-36)                  # tiny block: scale at the bottom of E8M0
    W[3, :32] = np.float32(2.0 ** -140)               # subnormal block maximum: all-zero codes
    if N > 6:                                         # a row whose every block has scale byte 0 (2^-127)
        k = np.arange(K)
        W[6] = (np.float32(2.0 ** -125) * (1 + (k % 7) / 8) * np.where(k % 2, -1, 1)).astype(np.float32)
    W[4, 64:96] *= np.float32(1e30)                   # huge block
    W[5, :32] = np.linspace(-6.0, 6.0, 32, dtype=np.float32)
    return W


@pytest.mark.parametrize("N,K", [(16, 32), (64, 128), (4096, 1024), (1024, 4096), (48, 96)])
def test_mxfp4_quantize_pack_bit_exact(N, K):
    W = special_weights(N, K, 9400 + N)
    want, _, scales = oracle_packed(W)
    assert (scales[6] == 0).all()
    got = gpu_pack(W).numpy(np.uint8)
    bad = got != want
    assert not bad.any(), f"{bad.sum()} bytes differ, first at {np.argmax(bad)} of {got.size}"


class Mx:
    def __init__(self, W):
        self.N, self.K = W.shape
        self.q = gpu_pack(W).t
        _, codes, scales = oracle_packed(W)
        self.w = oracle.mxfp4_dequant_rows(codes, scales)


def run(A, mx, M, bias=None, resid=None):
    ws = zeros_ws(vla.vla_gemm_workspace_bytes(M, mx.N, mx.K, vla.VLA_WFMT_MXFP4))
    Y = Guarded(M * mx.N * 2)
    vla.vla_gemm_mxfp4w(dev(A), mx.q, bias, resid, Y.t, ws, ws.numel(), M, mx.N, mx.K)
    Y.check()
    assert int(host(ws[:61440]).view(np.uint32).sum()) == 0
    vla.vla_workspace_status(ws)
    return Y.numpy(np.uint16).reshape(M, mx.N)


@pytest.mark.parametrize("M", [1, 10, 17, 50, 64])
@pytest.mark.parametrize("N,K", [(4096, 1024), (1024, 4096), (48, 96), (272, 1056)])
def test_mxfp4_gemm_matches_oracle(M, N, K):
    print(f"mxfp4 gemm M={M} N={N} K={K}", flush=True)
    A = synthetic.activations(M, K, 9500 + M)
    mx = Mx(special_weights(N, K, 9600 + N))
    y = run(A, mx, M)
    ref, yabs = oracle.gemm(bf16_f64(A), mx.w)
    assert_gemm_close(y, ref, yabs)


def test_mxfp4_gemm_bias_and_residual():
    M, N, K = 50, 1024, 4096
    A = synthetic.activations(M, K, 9700)
    mx = Mx(synthetic.weights(N, K, 9701))
    b = synthetic.activations(1, N, 9702)[0]
    r = synthetic.activations(M, N, 9703)
    y = run(A, mx, M, bias=dev(b), resid=dev(r))
    ref, yabs = oracle.gemm(bf16_f64(A), mx.w, bf16_f64(b))
    # y = bf16(r + bf16(A W^T + b)): compare the GEMM part within tolerance, then the residual step
    yv, rv = bf16_f64(y), bf16_f64(r)
    assert np.all(np.abs(yv - (rv + ref)) <= 4e-3 * (yabs + np.abs(rv)) + 2.0 ** -8 * np.abs(rv + ref) + 1e-30)


def test_mxfp4_lane_map_one_hot():
    """Every weight row a single 1.0 at a permuted position (each block a
    single code 4.0 with scale 2^-2, or all zero): Y must be A's permuted
    columns, bit for bit."""
    M, N, K = 50, 256, 512
    perm = synthetic.rng(9800).permutation(K)[:N]
    W = np.zeros((N, K), np.float32)
    W[np.arange(N), perm] = 1.0
    A = synthetic.activations(M, K, 9801)
    y = run(A, Mx(W), M)
    assert np.array_equal(y, A[:, perm])


# ------------------------------------------------------------- wide kernel

@pytest.mark.parametrize("M", [65, 200, 571])
@pytest.mark.parametrize("N,K", [(272, 1056), (512, 2048), (4096, 1024)])
def test_mxfp4_wide_gemm_matches_oracle(M, N, K):
    """M > 64 runs the wide kernel: 256-column tiles, E8M0 scales staged per
    K tile; ragged N (272) and a K tile holding one real block (1056 = 16.5
    tiles of 64) included."""
    print(f"mxfp4 wide gemm M={M} N={N} K={K}", flush=True)
    A = synthetic.activations(M, K, 9900 + M)
    mx = Mx(special_weights(N, K, 9910 + N))
    y = run(A, mx, M)
    ref, yabs = oracle.gemm(bf16_f64(A), mx.w)
    assert_gemm_close(y, ref, yabs)


def test_mxfp4_wide_lane_map_one_hot():
    M, N, K = 300, 512, 1024
    perm = synthetic.rng(9920).permutation(K)[:N]
    W = np.zeros((N, K), np.float32)
    W[np.arange(N), perm] = 1.0
    A = synthetic.activations(M, K, 9921)
    y = run(A, Mx(W), M)
    assert np.array_equal(y, A[:, perm])


def test_mxfp4_wide_bias_and_residual():
    M, N, K = 300, 768, 2048
    A = synthetic.activations(M, K, 9930)
    mx = Mx(synthetic.weights(N, K, 9931))
    b = synthetic.activations(1, N, 9932)[0]
    r = synthetic.activations(M, N, 9933)
    y = run(A, mx, M, bias=dev(b), resid=dev(r))
    ref, yabs = oracle.gemm(bf16_f64(A), mx.w, bf16_f64(b))
    yv, rv = bf16_f64(y), bf16_f64(r)
    assert np.all(np.abs(yv - (rv + ref)) <= 4e-3 * (yabs + np.abs(rv)) + 2.0 ** -8 * np.abs(rv + ref) + 1e-30)


@pytest.mark.parametrize("N,K", [(16384, 2048), (2048, 16384)])
def test_mxfp4_wide_full_size(N, K):
    """The encoder shapes at M = 768 in the launch configuration the bench
    times (2048 -> 16384 on 256-column tiles, the 16384-deep one split over
    K across workgroups): every output against the oracle."""
    M = 768
    print(f"mxfp4 wide full M={M} N={N} K={K}", flush=True)
    A = synthetic.activations(M, K, 9940)
    mx = Mx(synthetic.weights(N, K, 9941))
    y = run(A, mx, M)
    ref, yabs = oracle.gemm(bf16_f64(A), mx.w)
    assert_gemm_close(y, ref, yabs)
