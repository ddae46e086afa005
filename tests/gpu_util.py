"""Shared helpers for the GPU parity tests: device buffers with canary guard
bands, bf16 bit conversions and the GEMM tolerance check."""
from __future__ import annotations

import numpy as np
import torch

import oracle

GUARD = 4096          # bytes of canary before and after every output buffer
CANARY = 0xA5


class Guarded:
    """A device byte buffer with canary bands on both sides of the payload."""

    def __init__(self, nbytes: int, fill: int | None = None):
        self.n = nbytes
        self.raw = torch.full((GUARD + nbytes + GUARD,), CANARY, dtype=torch.uint8, device="cuda")
        if fill is not None:
            self.raw[GUARD:GUARD + nbytes].fill_(fill)

    @property
    def t(self) -> torch.Tensor:
        return self.raw[GUARD:GUARD + self.n]

    def ptr(self) -> int:
        return self.t.data_ptr()

    def check(self) -> None:
        torch.cuda.synchronize()
        head = self.raw[:GUARD].cpu().numpy()
        tail = self.raw[GUARD + self.n:].cpu().numpy()
        assert np.all(head == CANARY), "write before the buffer (canary corrupted)"
        assert np.all(tail == CANARY), "write past the end of the buffer (canary corrupted)"

    def numpy(self, dtype) -> np.ndarray:
        torch.cuda.synchronize()
        return self.t.cpu().numpy().view(dtype)


def dev(a: np.ndarray) -> torch.Tensor:
    """Upload a numpy array (uint16 bf16 bits go up as int16)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a.copy()).cuda()


def host(t: torch.Tensor, dtype=None) -> np.ndarray:
    torch.cuda.synchronize()
    a = t.cpu().numpy()
    return a.view(dtype) if dtype is not None else a


def bf16_f64(bits) -> np.ndarray:
    return oracle.bf16_value(bits)


def assert_gemm_close(y_bits: np.ndarray, y_ref: np.ndarray, yabs: np.ndarray, tol: float = 4e-3):
    """|y - y_ref| <= tol * sum_k |a w| elementwise (the bound the path promises)."""
    y = bf16_f64(y_bits)
    err = np.abs(y - y_ref)
    bound = tol * yabs
    bad = err > bound
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(
            f"{bad.sum()} of {bad.size} outputs outside {tol}*sum|a*w|; first at {tuple(i)}: "
            f"y={y[tuple(i)]} ref={y_ref[tuple(i)]} bound={bound[tuple(i)]}")
    return float((err / np.maximum(yabs, 1e-30)).max())


def zeros_ws(nbytes: int) -> torch.Tensor:
    return torch.zeros(max(nbytes, 256), dtype=torch.uint8, device="cuda")
