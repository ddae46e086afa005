"""GPU parity of the decoder-block chain (merged gate/up GEMM with GELU*mul,
down GEMM, fused decoder boundary per layer): every layer against the oracle
fed the GPU's own layer state, the next gate bit for bit, eager vs graph
replay (bitwise), graph purity under input mutation, and the end-to-end
output against the oracle's fp64 chain (cosine similarity)."""
import numpy as np
import pytest
import torch

import bf16_gemm_vla_amd as vla
import oracle
import synthetic
from tests.gpu_util import bf16_f64, dev, host
from tests.test_gpu_chain import ChainWeights

pytestmark = pytest.mark.gpu


class Decoder:
    def __init__(self, L, M, H, I, per_row=True, seed=0, eps=1e-6):
        self.cw = ChainWeights(L, H, I, seed)
        self.L, self.M, self.H, self.I, self.per_row, self.eps = L, M, H, I, per_row, eps
        x, h, g, st = synthetic.decoder_chain_inputs(L, M, H, M if per_row else 1, seed)
        self.inputs = (x, h, g)
        self.styles = st
        self.d_in = [dev(a) for a in self.inputs]
        self.d_style = [dev(s) for s in st]
        self.d_out = [torch.empty(M * H, dtype=torch.int16, device="cuda") for _ in range(3)]
        n = vla.vla_decoder_chain_scratch_bytes(M, H, I)
        self.scratch = torch.zeros(n, dtype=torch.uint8, device="cuda")

    def args(self, layers=None):
        L = self.L if layers is None else layers
        cw = self.cw
        return (cw.wgu[:L], cw.sgu[:L], cw.wd[:L], cw.sd[:L], self.d_style[:L], self.per_row, self.eps,
                *self.d_in, *self.d_out, self.scratch, self.scratch.numel(), L, self.M, self.H, self.I)

    def eager(self, layers=None):
        vla.vla_decoder_chain_enqueue(*self.args(layers))
        return tuple(host(o).view(np.uint16).reshape(self.M, self.H).copy() for o in self.d_out)

    def oracle_layer(self, l, state):
        cw = self.cw
        return oracle.decoder_chain(*state, [cw.o_gu[l]], [cw.o_sgu[l]], [cw.o_d[l]], [cw.o_sd[l]],
                                    [self.styles[l]], self.eps, style_per_row=self.per_row)


def close(a_bits, b_bits):
    a, b = bf16_f64(a_bits).ravel(), bf16_f64(b_bits).ravel()
    cos = float(a @ b / np.linalg.norm(a) / np.linalg.norm(b))
    rel = np.abs(a - b) / np.maximum(np.abs(b), 1e-3)
    return cos, float(np.percentile(rel, 99))


def check_layers(dec, tag):
    state = dec.inputs
    for l in range(dec.L):
        got = dec.eager(l + 1)
        ref = dec.oracle_layer(l, state)
        assert np.array_equal(got[2], ref[2])                 # next gate: a copy
        for name, a, b in (("x", got[0], ref[0]), ("h", got[1], ref[1])):
            cos, p99 = close(a, b)
            print(f"{tag} layer {l} {name}: cosine={cos:.7f} p99 rel={p99:.3g}", flush=True)
            assert np.isfinite(bf16_f64(a)).all()
            assert cos > 0.9999 and p99 < 2e-2
        state = got
    return state


@pytest.mark.parametrize("per_row", [True, False])
def test_decoder_chain_small_layerwise(per_row):
    dec = Decoder(3, 50, 256, 512, per_row=per_row, seed=2)
    final = check_layers(dec, "small")
    assert all(np.array_equal(a, b) for a, b in zip(final, dec.eager()))


def test_decoder_chain_config_replay_purity_and_layers():
    """18 layers, M=50, H=1024, I=4096: graph replay == eager bitwise, replay
    after mutating the inputs equals a fresh eager run, every layer close to
    the oracle's layer on the GPU's own state, and the end-to-end output
    close to the oracle's 18-layer chain."""
    L, M, H, I = 18, 50, 1024, 4096
    print("decoder chain: building weights", flush=True)
    dec = Decoder(L, M, H, I)
    ref = dec.eager()
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    print("decoder chain: capture", flush=True)
    handle = vla.vla_decoder_chain_create(*dec.args(), stream)
    try:
        for _ in range(3):
            for o in dec.d_out:
                o.zero_()
            torch.cuda.synchronize()
            vla.vla_mlp_chain_replay(handle, stream)
            stream.synchronize()
            got = tuple(host(o).view(np.uint16).reshape(M, H) for o in dec.d_out)
            assert all(np.array_equal(a, b) for a, b in zip(got, ref))
        x2 = synthetic.activations(M, H, 4712)
        dec.d_in[0].copy_(dev(x2))
        torch.cuda.synchronize()
        vla.vla_mlp_chain_replay(handle, stream)
        stream.synchronize()
        replayed = tuple(host(o).view(np.uint16).reshape(M, H).copy() for o in dec.d_out)
        assert not np.array_equal(replayed[0], ref[0])
        fresh = dec.eager()
        assert all(np.array_equal(a, b) for a, b in zip(replayed, fresh))
        dec.d_in[0].copy_(dev(dec.inputs[0]))
        torch.cuda.synchronize()
    finally:
        vla.vla_mlp_chain_destroy(handle)
    print("decoder chain: per-layer oracle", flush=True)
    final = check_layers(dec, "config")
    assert all(np.array_equal(a, b) for a, b in zip(final, ref))
    cw = dec.cw
    e2e = oracle.decoder_chain(*dec.inputs, cw.o_gu, cw.o_sgu, cw.o_d, cw.o_sd, dec.styles, dec.eps)
    for name, a, b in (("x", ref[0], e2e[0]), ("h", ref[1], e2e[1])):
        cos, p99 = close(a, b)
        print(f"end to end {name}: cosine={cos:.7f} p99 rel={p99:.3g}", flush=True)
        assert cos > 0.999
    assert np.array_equal(ref[2], e2e[2])
