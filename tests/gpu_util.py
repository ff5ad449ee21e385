"""Helpers for the GPU parity tests: numpy inputs -> device tensors, tolerances."""
from __future__ import annotations

import numpy as np
import torch


def dev():
    return torch.device("cuda", 0)


def bf16_tensor(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns -> torch.bfloat16 device tensor (same bits)."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).copy())
    return t.view(torch.bfloat16).to(dev())


def words_tensor(words: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(words).view(np.int32).copy()).to(dev())


def f32_tensor(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32).copy()).to(dev())


def i32_tensor(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32).copy()).to(dev())


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def assert_close(gpu: np.ndarray, ref: np.ndarray, what: str = "") -> None:
    """|gpu - oracle| <= 1e-2 * max|oracle| + 1e-3, element by element."""
    tol = 1e-2 * float(np.abs(ref).max()) + 1e-3
    err = np.abs(gpu - ref)
    worst = float(err.max())
    assert worst <= tol, f"{what}: max |gpu - oracle| = {worst:.3e} > tol {tol:.3e}"
