"""GPU parity of the gated-MLP chain: the fused gate/up GELU*mul GEMM stage
against the oracle fed the GPU's own inputs, the residual stage, eager vs
graph replay (bitwise), graph purity under input mutation, and the 18-layer
chain against the oracle's fp64 chain (per-stage bounds; end-to-end error
and cosine reported)."""
import numpy as np
import pytest
import torch

import bf16_gemm_vla_amd as vla
import oracle
import synthetic
from oracle import OCP
from tests.gpu_util import Guarded, assert_gemm_close, bf16_f64, dev, host, zeros_ws

pytestmark = pytest.mark.gpu


class ChainWeights:
    def __init__(self, L, H, I, seed=0, with_down=True):
        gate, up, down = synthetic.chain_weights(L, H, I, seed)
        self.L, self.H, self.I = L, H, I
        self.wgu, self.sgu, self.wd, self.sd = [], [], [], []
        self.o_gu, self.o_sgu, self.o_d, self.o_sd = [], [], [], []
        for l in range(L):
            W = np.concatenate([gate[l], up[l]])
            q = torch.empty(2 * I * H, dtype=torch.uint8, device="cuda")
            s = torch.empty(2 * I, dtype=torch.float32, device="cuda")
            vla.vla_quantize_pack(dev(W), q, s, 2 * I, H, vla.VLA_WFMT_E4M3_OCP, vla.VLA_LAYOUT_MFMA)
            self.wgu.append(q); self.sgu.append(s)
            a, b = oracle.quantize_rows(W, OCP)
            self.o_gu.append(a); self.o_sgu.append(b)
            if not with_down:
                continue
            qd = torch.empty(H * I, dtype=torch.uint8, device="cuda")
            sd = torch.empty(H, dtype=torch.float32, device="cuda")
            vla.vla_quantize_pack(dev(down[l]), qd, sd, H, I, vla.VLA_WFMT_E4M3_OCP, vla.VLA_LAYOUT_MFMA)
            self.wd.append(qd); self.sd.append(sd)
            c, d = oracle.quantize_rows(down[l], OCP)
            self.o_d.append(c); self.o_sd.append(d)


@pytest.mark.parametrize("M,I,K", [(50, 4096, 1024), (4, 64, 128), (17, 48, 96), (300, 256, 512),
                                   (33, 4112, 1024), (40, 4128, 1024)])
def test_gelu_mul_stage(M, I, K):
    print(f"gelu_mul M={M} I={I} K={K}", flush=True)
    cw = ChainWeights(1, K, I, seed=M, with_down=False)
    A = synthetic.activations(M, K, 7000 + M)
    act, gu = Guarded(M * I * 2), Guarded(M * 2 * I * 2)
    ws = zeros_ws(vla.vla_gemm_workspace_bytes(M, 2 * I, K, 1))
    vla.vla_gemm_fp8w_gelu_mul(dev(A), cw.wgu[0], cw.sgu[0], None, act.t, gu.t, ws, ws.numel(), M, I, K)
    act.check(); gu.check()
    gu_bits = gu.numpy(np.uint16).reshape(M, 2 * I)
    # stage 1: the merged GEMM against the oracle GEMM
    ref, yabs = oracle.gemm(bf16_f64(A), oracle.dequant_rows(cw.o_gu[0], cw.o_sgu[0]))
    assert_gemm_close(gu_bits, ref, yabs)
    # stage 2: GELU*mul on the GPU's own g and u, within 1 bf16 ulp of the oracle
    want = oracle.gelu_mul(gu_bits[:, :I], gu_bits[:, I:])
    got = act.numpy(np.uint16).reshape(M, I)
    diff = np.abs(got.astype(np.int32) - want.astype(np.int32))
    same_sign = (got >> 15) == (want >> 15)
    assert np.all((diff <= 1) & same_sign | (got == want))
    # without the debug output the activation is identical
    act2 = torch.empty(M * I, dtype=torch.int16, device="cuda")
    vla.vla_gemm_fp8w_gelu_mul(dev(A), cw.wgu[0], cw.sgu[0], None, act2, None, ws, ws.numel(), M, I, K)
    assert np.array_equal(host(act2).view(np.uint16).reshape(M, I), got)


@pytest.mark.parametrize("M,I,K", [(50, 4096, 1024), (17, 48, 96), (300, 256, 512)])
def test_gelu_mul_stage_bias(M, I, K):
    """The merged gate/up GEMM adds [b_gate, b_up] in its epilogue: g and u
    against the oracle GEMM with the bias, act from the GPU's own g and u."""
    print(f"gelu_mul bias M={M} I={I} K={K}", flush=True)
    cw = ChainWeights(1, K, I, seed=M + 1, with_down=False)
    A = synthetic.activations(M, K, 7100 + M)
    b_bits = synthetic.activations(1, 2 * I, 7200 + M)[0]
    act, gu = Guarded(M * I * 2), Guarded(M * 2 * I * 2)
    ws = zeros_ws(vla.vla_gemm_workspace_bytes(M, 2 * I, K, 1))
    vla.vla_gemm_fp8w_gelu_mul(dev(A), cw.wgu[0], cw.sgu[0], dev(b_bits), act.t, gu.t, ws, ws.numel(), M, I, K)
    act.check(); gu.check()
    gu_bits = gu.numpy(np.uint16).reshape(M, 2 * I)
    ref, yabs = oracle.gemm(bf16_f64(A), oracle.dequant_rows(cw.o_gu[0], cw.o_sgu[0]), bf16_f64(b_bits))
    assert_gemm_close(gu_bits, ref, yabs)
    want = oracle.gelu_mul(gu_bits[:, :I], gu_bits[:, I:])
    got = act.numpy(np.uint16).reshape(M, I)
    diff = np.abs(got.astype(np.int32) - want.astype(np.int32))
    same_sign = (got >> 15) == (want >> 15)
    assert np.all((diff <= 1) & same_sign | (got == want))
    # every split-K counter is back at zero after the call
    assert int(host(ws[:61440]).view(np.uint32).sum()) == 0


def make_chain(L, M, H, I, seed=0):
    cw = ChainWeights(L, H, I, seed)
    x = synthetic.activations(M, H, synthetic.IDS["chain.x"] + seed)
    xin = dev(x)
    xout = torch.empty(M * H, dtype=torch.int16, device="cuda")
    nbytes = vla.vla_mlp_chain_scratch_bytes(M, H, I)
    scratch = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    return cw, x, xin, xout, scratch


def eager(cw, xin, xout, scratch, M):
    vla.vla_mlp_chain_enqueue(cw.wgu, cw.sgu, cw.wd, cw.sd, xin, xout, scratch, scratch.numel(),
                              cw.L, M, cw.H, cw.I)
    return host(xout).view(np.uint16).reshape(M, cw.H).copy()


def test_chain_small_matches_oracle_stagewise():
    L, M, H, I = 3, 50, 256, 512
    cw, x, xin, xout, scratch = make_chain(L, M, H, I, seed=1)
    got = eager(cw, xin, xout, scratch, M)
    # replay the oracle one layer at a time on the GPU's own layer input
    # (run the GPU chain with 1..L layers to get its intermediate x)
    xs = [x]
    for l in range(1, L + 1):
        sub = ChainSub(cw, l)
        xs.append(eager(sub, xin, xout, scratch, M))
    assert np.array_equal(xs[-1], got)
    for l in range(L):
        ref = oracle.mlp_chain(xs[l], [cw.o_gu[l]], [cw.o_sgu[l]], [cw.o_d[l]], [cw.o_sd[l]])
        a, b = bf16_f64(xs[l + 1]), bf16_f64(ref)
        rel = np.abs(a - b) / np.maximum(np.abs(b), 1e-3)
        assert np.percentile(rel, 99) < 2e-2 and np.max(np.abs(a - b)) < 0.05 * np.max(np.abs(b))


class ChainSub:
    """The first l layers of a ChainWeights (same device tensors)."""

    def __init__(self, cw, l):
        self.L, self.H, self.I = l, cw.H, cw.I
        self.wgu, self.sgu, self.wd, self.sd = cw.wgu[:l], cw.sgu[:l], cw.wd[:l], cw.sd[:l]


def test_chain_config_replay_eager_purity():
    """18 layers, M=50, H=1024, I=4096: graph replay == eager bitwise; replay
    after mutating x_in equals a fresh eager run; every layer close to the
    oracle's layer applied to the GPU's own layer input.

    With the configured N(0, 0.02) weights and no normalisation between
    layers, the residual stream grows quadratically and overflows bf16 near
    layer 16 on both sides; the per-layer comparison covers the layers whose
    input is still finite and below 1e4 in magnitude."""
    L, M, H, I = 18, 50, 1024, 4096
    print("chain config: building weights", flush=True)
    cw, x, xin, xout, scratch = make_chain(L, M, H, I)
    ref_eager = eager(cw, xin, xout, scratch, M)
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    print("chain config: capture", flush=True)
    h = vla.vla_mlp_chain_create(cw.wgu, cw.sgu, cw.wd, cw.sd, xin, xout, scratch, scratch.numel(),
                                 L, M, H, I, stream)
    try:
        for _ in range(3):
            xout.zero_()
            torch.cuda.synchronize()
            vla.vla_mlp_chain_replay(h, stream)
            stream.synchronize()
            assert np.array_equal(host(xout).view(np.uint16).reshape(M, H), ref_eager)
        # purity: new input in place, replay, compare with eager on the new input
        x2 = synthetic.activations(M, H, 4711)
        xin.copy_(dev(x2))
        torch.cuda.synchronize()
        vla.vla_mlp_chain_replay(h, stream)
        stream.synchronize()
        replayed = host(xout).view(np.uint16).reshape(M, H).copy()
        assert not np.array_equal(replayed, ref_eager)
        assert np.array_equal(replayed, eager(cw, xin, xout, scratch, M))
        xin.copy_(dev(x))
        torch.cuda.synchronize()
    finally:
        vla.vla_mlp_chain_destroy(h)
    with pytest.raises(RuntimeError, match="vla_mlp_chain_replay"):
        vla.vla_mlp_chain_replay(h, stream)
    # per layer: the GPU's x_l (chain truncated to l layers) through one oracle layer
    print("chain config: per-layer oracle", flush=True)
    prev = x
    checked = 0
    for l in range(L):
        cur = eager(ChainSub(cw, l + 1), xin, xout, scratch, M)
        pv = bf16_f64(prev)
        if not np.isfinite(pv).all() or np.abs(pv).max() > 1e4:
            break
        ref = oracle.mlp_chain(prev, [cw.o_gu[l]], [cw.o_sgu[l]], [cw.o_d[l]], [cw.o_sd[l]])
        a, b = bf16_f64(cur).ravel(), bf16_f64(ref).ravel()
        cos = float(a @ b / np.linalg.norm(a) / np.linalg.norm(b))
        rel = np.abs(a - b) / np.maximum(np.abs(b), 1e-3)
        print(f"layer {l}: max|x|={np.abs(b).max():.4g} cosine={cos:.7f} p99 rel={np.percentile(rel, 99):.3g}", flush=True)
        assert cos > 0.9999 and np.percentile(rel, 99) < 2e-2
        prev = cur
        checked += 1
    assert np.array_equal(prev, ref_eager) or checked >= 10
    assert checked >= 10
