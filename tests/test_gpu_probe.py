"""GPU checks of the measurement probes: the matrix-core rate probe does
exactly the multiply-adds it is credited with (every lane's accumulator sum
equals the count the rate is computed from), on every instruction form, with
each of its four chains on its own operand set."""
import numpy as np
import pytest
import torch

import bf16_gemm_vla_amd as vla

pytestmark = pytest.mark.gpu

# name, form, (m, n, k), bytes of 1.0 / 2.0 / 4.0 / 8.0 in the operand type
FORMS = [
    ("bf16_32x32x16", vla.VLA_MFMA_BF16_32X32X16, (32, 32, 16), "bf16"),
    ("bf16_16x16x32", vla.VLA_MFMA_BF16_16X16X32, (16, 16, 32), "bf16"),
    ("fp8_32x32x64", vla.VLA_MFMA_FP8_32X32X64, (32, 32, 64), "fp8"),
    ("fp8_16x16x128", vla.VLA_MFMA_FP8_16X16X128, (16, 16, 128), "fp8"),
]


def power_of_two_word(e, dt):
    """A 32-bit operand word whose every element is 2^e (bf16 pairs or E4M3 quads)."""
    if dt == "bf16":
        h = (127 + e) << 7
        return h | (h << 16)
    b = (7 + e) << 3          # OCP E4M3: bias 7, three mantissa bits
    return b * 0x01010101


@pytest.mark.parametrize("name,form,mnk,dt", FORMS, ids=[f[0] for f in FORMS])
def test_mfma_rate_probe_counts(name, form, mnk, dt):
    m, n, k = mnk
    words = np.zeros((256, 64), dtype=np.uint32)
    for j in range(4):            # set j: A = 1, B = 2^j
        words[:, 16 * j:16 * j + 8] = power_of_two_word(0, dt)
        words[:, 16 * j + 8:16 * j + 16] = power_of_two_word(j, dt)
    ops = torch.from_numpy(words.view(np.int32)).cuda()
    blocks, iters = 3, 37
    out = torch.full((blocks * 256,), -1.0, dtype=torch.float32, device="cuda")
    vla.vla_probe_mfma_rate(form, ops, iters, out, blocks)
    torch.cuda.synchronize()
    got = out.cpu().numpy().reshape(blocks, 4, 64)
    # each output element of chain j gathers k products 1 * 2^j per iteration;
    # a wave holds m*n outputs per chain spread over its 64 lanes
    per_wave = iters * m * n * k * (1 + 2 + 4 + 8)
    assert np.all(got.sum(axis=2, dtype=np.float64) == per_wave), name
    per_lane = iters * (m * n // 64) * k * (1 + 2 + 4 + 8)
    assert np.all(got == per_lane), name



def test_mfma_rate_probe_clocks():
    """The optional clock output: one (cycles, 100 MHz ticks) pair per
    workgroup, nothing written past them, and a plausible shader clock."""
    words = np.zeros((256, 64), dtype=np.uint32)
    for j in range(4):
        words[:, 16 * j:16 * j + 8] = power_of_two_word(0, "bf16")
        words[:, 16 * j + 8:16 * j + 16] = power_of_two_word(j, "bf16")
    ops = torch.from_numpy(words.view(np.int32)).cuda()
    blocks, iters = 8, 4096
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    clocks = torch.full((2 * blocks + 2,), -7, dtype=torch.int64, device="cuda")
    vla.vla_probe_mfma_rate(vla.VLA_MFMA_BF16_32X32X16, ops, iters, out, blocks, clocks=clocks)
    torch.cuda.synchronize()
    c = clocks.cpu().numpy()
    assert np.all(c[2 * blocks:] == -7)
    cycles, ticks = c[0:2 * blocks:2].astype(np.float64), c[1:2 * blocks:2].astype(np.float64)
    # four chains of 32-cycle instructions, one wave per SIMD: at least the
    # instructions' own cycles
    assert np.all(cycles >= iters * 4 * 32), cycles
    assert np.all(ticks > 0)
    ghz = cycles / (ticks * 10.0)
    assert np.all((ghz > 0.5) & (ghz < 3.0)), ghz
    assert np.all(out.cpu().numpy() == iters * (32 * 32 // 64) * 16 * 15)
