"""Oracle: skinny weight-only-quantized matmul (test infrastructure only).

What is computed (page "Speculative decoding and MTP on Apple silicon", Facts:
the claim that the stock quantized matmul re-reads the weight matrix for every
row of the M = 2..8 verify window, measured on the (M,5120)@(17408,5120)^T
shape; page "The fastest way to run local LLMs on a Mac", section "Why native
MTP doubles decode": the verify pass runs all drafted rows through one pass
over the weights):

    Y[m, n] = sum_k X[m, k] * W[n, k],
    W[n, k] = s[n, g(k)] * q[n, k] + b[n, g(k)],   g(k) = k // group_size.

Readings where the pages are silent (they name 4-bit and 8-bit affine packs
but give no formula or layout):
  * "affine" is w = s*q + b with unsigned codes q in [0, 2**bits);
  * groups of ``group_size`` consecutive inputs along K share one bf16 scale
    and one bf16 bias;
  * 4-bit codes: element k of row n is the nibble at bits 4*(k%8)..4*(k%8)+3 of
    32-bit word k//8 of that row (low nibble first, little-endian words);
    8-bit codes: byte k of row n.

The oracle dequantises explicitly into a float64 matrix and multiplies with
numpy in float64: no blocking, fusion or reordering.
"""
from __future__ import annotations

import numpy as np


def bf16_to_f64(bits) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float64 exactly."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def unpack_codes(wq, bits: int, N: int, K: int) -> np.ndarray:
    """Integer codes q[N, K] from the packed words (see module docstring)."""
    words = np.ascontiguousarray(np.asarray(wq, dtype=np.uint32)).reshape(N, K * bits // 32)
    if bits == 4:
        q = np.empty((N, K), dtype=np.int64)
        for j in range(8):  # nibble j of word w holds element 8*w + j
            q[:, j::8] = (words >> np.uint32(4 * j)) & np.uint32(0xF)
        return q
    if bits == 8:
        return words.view(np.uint8).reshape(N, K).astype(np.int64)
    raise ValueError("bits must be 4 or 8")


def dequantize(wq, scales, biases, bits: int, group_size: int, N: int, K: int,
               rows=None) -> np.ndarray:
    """Explicit float64 weights W[n, k] = s[n, k//gs] * q[n, k] + b[n, k//gs].

    ``rows`` optionally restricts the result to a subset of output rows n.
    """
    G = K // group_size
    q = unpack_codes(wq, bits, N, K)
    s = bf16_to_f64(scales).reshape(N, G)
    b = bf16_to_f64(biases).reshape(N, G)
    if rows is not None:
        q, s, b = q[rows], s[rows], b[rows]
    g = np.arange(K) // group_size
    return s[:, g] * q + b[:, g]


def skinny_qmm(x, wq, scales, biases, bits: int, group_size: int, M: int, N: int, K: int,
               cols=None) -> np.ndarray:
    """float64 Y[M, N] (or Y[:, cols]) = X @ W^T with X the bf16 rows widened exactly."""
    X = bf16_to_f64(x).reshape(M, K)
    W = dequantize(wq, scales, biases, bits, group_size, N, K, rows=cols)
    return X @ W.T


def algorithmic_bytes(M: int, N: int, K: int, bits: int, group_size: int = 64,
                      out_bytes: int = 2) -> int:
    """Bytes one call must move at minimum: packed codes + bf16 scale/bias + X + Y."""
    return N * K * bits // 8 + 4 * N * (K // group_size) + 2 * M * K + out_bytes * M * N
