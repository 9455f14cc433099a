"""Helpers for the GPU parity tests: device transfer and the acceptance bound."""
from __future__ import annotations

import numpy as np
import torch

import oracle

DEV = torch.device("cuda:0")


def to_dev(a: np.ndarray) -> torch.Tensor:
    """numpy -> device tensor: uint16 arrays are bf16 bit patterns, float32 stays float32."""
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def x_as_f32(x: np.ndarray) -> np.ndarray:
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32)
    return x


def max_abs_w(fmt: int, W: np.ndarray, N: int, K: int, chunk: int = 4096) -> float:
    """max |w| over the whole dequantised weight tensor (chunked to bound memory)."""
    m = 0.0
    Wr = W.reshape(N, -1)
    for n0 in range(0, N, chunk):
        n1 = min(N, n0 + chunk)
        m = max(m, float(np.abs(oracle.dequant(fmt, np.ascontiguousarray(Wr[n0:n1]), n1 - n0, K)).max()))
    return m


def bound(x: np.ndarray, rows, wmax: float) -> np.ndarray:
    """|dy| <= 1e-3 * ||x_row||_2 * max|w|, ||x_row|| of the unquantised row in fp64; [len(rows), 1]."""
    xf = x_as_f32(x[rows]).astype(np.float64)
    return 1e-3 * np.sqrt((xf ** 2).sum(1))[:, None] * wmax


def check(y_gpu: np.ndarray, y_ref: np.ndarray, tol: np.ndarray, what: str) -> float:
    err = np.abs(y_gpu.astype(np.float64) - y_ref)
    ratio = float(np.max(err / tol)) if err.size else 0.0
    assert np.all(np.isfinite(y_gpu)), f"{what}: non-finite output"
    assert np.all(err <= tol), f"{what}: max err/tol {ratio:.3g}"
    return ratio
