"""Oracle: 8-bit KV cache — the append that quantizes rows into it, and multi-row
attention that reads it (test infrastructure only).

The pages use KV-quantized caches together with speculative decoding (page
"Speculative decoding and MTP on Apple silicon", Facts: an 8-bit KV cache runs
with speculation and saves memory) but fix no format. Readings, following the
affine group quantization the pages use for weights:
  * every cached key or value row of a KV head is cut into groups of 64 along the
    head dimension; group g of position j holds codes q in [0, 255] and one bf16
    (scale, bias) pair: x ~ scale * q + bias;
  * quantizing a bf16 row (the append): per group, mn = min x, mx = max x (exact),
    scale32 = (mx - mn) / 255 in float32, code = rint((x - mn) / scale32) in
    float32 (round half to even), clamped to [0, 255]; a group with mx == mn gets
    codes 0 and scale 0; the stored scale is bf16(scale32) (round to nearest
    even) and the stored bias is mn (a bf16 value already). The integer codes are
    decided in float32 on both sides, so they must agree exactly;
  * attention reads the dequantized values s * q + b (float64 here) and is
    otherwise the definition in oracle/attn.py, causal or with a tree mask.
"""
from __future__ import annotations

import numpy as np

from .attn import visible_keys
from .qmm import bf16_to_f64

GROUP = 64


def _bf16_rne(x32: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def quantize_rows(x_bits: np.ndarray):
    """Quantize bf16 rows [..., D] (D a multiple of 64).

    Returns (codes uint8 [..., D], sb uint16 [..., D/64, 2]) with sb[..., g, 0] the
    bf16 scale and sb[..., g, 1] the bf16 bias of group g."""
    x = (np.asarray(x_bits, np.uint16).astype(np.uint32) << 16).view(np.float32)
    shape = x.shape
    D = shape[-1]
    g = x.reshape(-1, D // GROUP, GROUP)
    mn = g.min(axis=-1)
    mx = g.max(axis=-1)
    scale32 = ((mx - mn) / np.float32(255.0)).astype(np.float32)
    flat = scale32 == 0
    safe = np.where(flat, np.float32(1.0), scale32).astype(np.float32)
    q = np.rint(((g - mn[..., None]).astype(np.float32) / safe[..., None]).astype(np.float32))
    q = np.clip(q, 0, 255)
    q[flat] = 0
    sb = np.stack([_bf16_rne(scale32), _bf16_rne(mn)], axis=-1)
    return (q.astype(np.uint8).reshape(shape),
            sb.reshape(shape[:-1] + (D // GROUP, 2)))


def dequantize(codes: np.ndarray, sb: np.ndarray) -> np.ndarray:
    """float64 s * q + b for codes [..., D] and sb [..., D/64, 2]."""
    D = codes.shape[-1]
    s = bf16_to_f64(sb[..., 0])
    b = bf16_to_f64(sb[..., 1])
    q = codes.astype(np.float64).reshape(codes.shape[:-1] + (D // GROUP, GROUP))
    return (s[..., None] * q + b[..., None]).reshape(codes.shape)


def int8_attention(q, k_codes, k_sb, v_codes, v_sb, M: int, Hq: int, Hkv: int, D: int, T: int,
                   T_cap: int, scale: float, mask=None, pairs=None) -> np.ndarray:
    """float64 o[M, Hq, D] (or the listed (m, h) rows) of attention over the
    dequantized caches k_codes/v_codes [Hkv, T_cap, D], k_sb/v_sb [Hkv, T_cap, D/64, 2];
    causal among the drafted rows, or the tree mask of oracle/attn.py."""
    G = Hq // Hkv
    Q = bf16_to_f64(q).reshape(M, Hq, D)
    Kf = dequantize(np.asarray(k_codes)[:, :T], np.asarray(k_sb)[:, :T])
    Vf = dequantize(np.asarray(v_codes)[:, :T], np.asarray(v_sb)[:, :T])
    chain = np.array([(1 << (i + 1)) - 1 for i in range(M)], dtype=np.uint64)
    msk = chain if mask is None else mask
    todo = [(m, h) for m in range(M) for h in range(Hq)] if pairs is None else list(pairs)
    res = np.empty((len(todo), D))
    for i, (m, h) in enumerate(todo):
        idx = visible_keys(M, T, msk, m)
        s = scale * (Kf[h // G, idx, :] @ Q[m, h, :])
        e = np.exp(s - s.max())
        res[i] = (e / e.sum()) @ Vf[h // G, idx, :]
    return res.reshape(M, Hq, D) if pairs is None else res


def algorithmic_bytes(M: int, Hq: int, Hkv: int, D: int, T: int) -> int:
    """Codes and (scale, bias) pairs of K and V read once per KV head, q in and out (bf16)."""
    return 2 * Hkv * T * (D + 4 * (D // GROUP)) + 4 * M * Hq * D
