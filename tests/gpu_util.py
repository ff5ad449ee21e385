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


def interleave_gate_up(wg: dict, wu: dict) -> dict:
    """Rows of [gate; up] regrouped per 64 outputs (gate rows 64c..64c+63, then the
    matching up rows), the row order the SwiGLU epilogue of vq_qmm_packed expects."""
    I, K, bits = wg["N"], wg["K"], wg["bits"]
    G = K // 64
    out = {}
    for key, width in (("wq", K * bits // 32), ("scales", G), ("biases", G)):
        g = np.asarray(wg[key]).reshape(I, width)
        u = np.asarray(wu[key]).reshape(I, width)
        blocks = [np.concatenate([g[64 * c: 64 * c + 64], u[64 * c: 64 * c + 64]]) for c in range(I // 64)]
        out[key] = np.ascontiguousarray(np.concatenate(blocks))
    out.update(N=2 * I, K=K, bits=bits, group_size=64)
    return out


def stack_gate_up(wg: dict, wu: dict) -> dict:
    """The [gate; up] matrix of the oracle composition (gate rows first)."""
    I, K, bits = wg["N"], wg["K"], wg["bits"]
    G = K // 64
    out = {}
    for key, width in (("wq", K * bits // 32), ("scales", G), ("biases", G)):
        out[key] = np.ascontiguousarray(np.concatenate([np.asarray(wg[key]).reshape(I, width),
                                                        np.asarray(wu[key]).reshape(I, width)]))
    out.update(N=2 * I, K=K, bits=bits, group_size=64)
    return out
