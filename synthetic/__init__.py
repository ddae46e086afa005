"""Seeded synthetic inputs shared by the HIP path's tests/benchmark and the oracle.

This module draws random numbers and nothing else: it holds none of the
method's arithmetic (no quantization, packing, GEMM or activation).  The one
rounding it does, fp32 -> bf16 for activations, is input preparation and is
done by torch's own conversion, so both sides receive identical bits.

Recipe (stated once, used everywhere):
  * generator: ``numpy.random.default_rng(SeedSequence([seed, tensor_id]))``,
    seed 0 by default; each tensor of a workload has a fixed ``tensor_id``.
  * activations: N(0, 1) drawn in fp32, rounded to bf16 (returned as uint16
    bit patterns).
  * weights: N(0, 0.02) drawn in fp32 (sigma = 0.02), one row per output
    channel (N x K).
  * decoder boundary: residual and block output N(0, 1), gate and the
    style rows (scale | shift | next gate) N(0, 0.1), all rounded to bf16
    (the pages give no distributions; modulation outputs are taken small).
The pages measure on camera observations of a public robotics benchmark and
on trained checkpoints; neither is available here, and these Gaussian
tensors of the same shapes stand in for them (no outliers).
"""
from __future__ import annotations

import numpy as np

WEIGHT_SIGMA = 0.02


def rng(tensor_id: int, seed: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, tensor_id]))


def fp32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 -> bf16 with torch's CPU conversion; return uint16 bits."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def activations(M: int, K: int, tensor_id: int, seed: int = 0) -> np.ndarray:
    """bf16 activations ~ N(0, 1), M x K, as uint16 bit patterns."""
    x = rng(tensor_id, seed).standard_normal((M, K), dtype=np.float32)
    return fp32_to_bf16_bits(x)


def weights(N: int, K: int, tensor_id: int, seed: int = 0, sigma: float = WEIGHT_SIGMA):
    """fp32 weights ~ N(0, sigma), N x K (row = output channel)."""
    w = rng(tensor_id, seed).standard_normal((N, K), dtype=np.float32)
    return (w * np.float32(sigma)).astype(np.float32)


def uniform_fp32(n: int, tensor_id: int, lo: float, hi: float, seed: int = 0) -> np.ndarray:
    return rng(tensor_id, seed).uniform(lo, hi, n).astype(np.float32)


# Tensor ids of the named workloads (fixed so every run sees the same bits).
IDS = {
    "tiny.A": 1, "tiny.W": 2,
    "skinny.up.A": 10, "skinny.up.W": 11,
    "skinny.down.A": 12, "skinny.down.W": 13,
    "wide.up.A": 20, "wide.up.W": 21,
    "wide.down.A": 22, "wide.down.W": 23,
    "dialect.W": 30,
    "chain.x": 40,
    "boundary.residual": 50, "boundary.out": 51, "boundary.gate": 52, "boundary.style": 53,
    "decoder.x": 60, "decoder.h": 61, "decoder.gate": 62,
    "decoder.style": 400,   # + layer
    "chain.gate": 100,   # + layer
    "chain.up": 200,     # + layer
    "chain.down": 300,   # + layer
}


def chain_weights(L: int, H: int, I: int, seed: int = 0):
    """fp32 gate, up (I x H) and down (H x I) weights for each of L layers."""
    gate = [weights(I, H, IDS["chain.gate"] + l, seed) for l in range(L)]
    up = [weights(I, H, IDS["chain.up"] + l, seed) for l in range(L)]
    down = [weights(H, I, IDS["chain.down"] + l, seed) for l in range(L)]
    return gate, up, down


MODULATION_SIGMA = 0.1


def boundary_inputs(M: int, D: int, style_rows: int, seed: int = 0):
    """bf16 bit patterns for the fused decoder boundary: residual, out (M x D),
    gate (M x D) and style (style_rows x 3D)."""
    def draw(shape, tid, sigma):
        x = rng(IDS[tid], seed).standard_normal(shape, dtype=np.float32) * np.float32(sigma)
        return fp32_to_bf16_bits(x)
    return (draw((M, D), "boundary.residual", 1.0), draw((M, D), "boundary.out", 1.0),
            draw((M, D), "boundary.gate", MODULATION_SIGMA),
            draw((style_rows, 3 * D), "boundary.style", MODULATION_SIGMA))


def decoder_chain_inputs(L: int, M: int, H: int, style_rows: int, seed: int = 0):
    """bf16 bit patterns for the decoder-block chain: residual x and normalized
    input h ~ N(0, 1), gate ~ N(0, 0.1) (M x H), and one style array
    (style_rows x 3H, N(0, 0.1)) per layer."""
    def draw(shape, tid, sigma):
        x = rng(tid, seed).standard_normal(shape, dtype=np.float32) * np.float32(sigma)
        return fp32_to_bf16_bits(x)
    return (draw((M, H), IDS["decoder.x"], 1.0), draw((M, H), IDS["decoder.h"], 1.0),
            draw((M, H), IDS["decoder.gate"], MODULATION_SIGMA),
            [draw((style_rows, 3 * H), IDS["decoder.style"] + l, MODULATION_SIGMA) for l in range(L)])
