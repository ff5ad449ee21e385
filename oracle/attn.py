"""Oracle: multi-row decode attention over a GQA KV cache (test infrastructure only).

What is computed (page "Speculative decoding and MTP on Apple silicon", Facts:
the claim that stock decode attention re-reads the whole KV cache once per
query row for 2-8 rows and that a multi-row kernel reads each KV tile once;
page "The fastest way to run local LLMs on a Mac", section "Why token 1,000 is
faster than token 100,000": the full-attention layers read a KV cache that
grows with context):

For query row i in [0, M), query head h, KV head kv = h // G (G = Hq // Hkv):
    s_ij = scale * <q[i, h], k[kv, j]>                  for j <= T - M + i
    w_ij = exp(s_ij - max_j s_ij) / sum_j exp(s_ij - max_j s_ij)
    o[i, h] = sum_j w_ij * v[kv, j]

Readings where the pages are silent:
  * causal among the drafted rows, bottom-right aligned: the M verify rows are
    the last M of the T valid positions, so row i sees every committed position
    and drafted rows 0..i;
  * grouped-query attention maps consecutive query heads onto one KV head;
  * no rotary embedding, window, sink or gate inside the attention call.

float64 throughout; softmax subtracts the row maximum.
"""
from __future__ import annotations

import numpy as np

from .qmm import bf16_to_f64


def _kv(cache, Hkv: int, T_cap: int, D: int, T: int) -> np.ndarray:
    return bf16_to_f64(cache).reshape(Hkv, T_cap, D)[:, :T, :]


def attention_weights(q, k_cache, M: int, Hq: int, Hkv: int, D: int, T: int, T_cap: int,
                      scale: float, m: int, h: int) -> np.ndarray:
    """float64 softmax weights w[j] (length T, zero where masked) of row m, head h."""
    G = Hq // Hkv
    Q = bf16_to_f64(q).reshape(M, Hq, D)
    Kc = _kv(k_cache, Hkv, T_cap, D, T)
    limit = T - M + m  # last visible key index (inclusive)
    s = scale * (Kc[h // G, : limit + 1, :] @ Q[m, h, :])
    e = np.exp(s - s.max())
    w = np.zeros(T)
    w[: limit + 1] = e / e.sum()
    return w


def multirow_attention(q, k_cache, v_cache, M: int, Hq: int, Hkv: int, D: int, T: int,
                       T_cap: int, scale: float, pairs=None) -> np.ndarray:
    """float64 output o[M, Hq, D] (or, with ``pairs=[(m, h), ...]``, o for those rows only).

    Follows the definition in the module docstring one (row, head) at a time.
    """
    Vc = _kv(v_cache, Hkv, T_cap, D, T)
    G = Hq // Hkv
    if pairs is None:
        out = np.empty((M, Hq, D))
        for m in range(M):
            for h in range(Hq):
                w = attention_weights(q, k_cache, M, Hq, Hkv, D, T, T_cap, scale, m, h)
                out[m, h] = w @ Vc[h // G]
        return out
    res = np.empty((len(pairs), D))
    for i, (m, h) in enumerate(pairs):
        w = attention_weights(q, k_cache, M, Hq, Hkv, D, T, T_cap, scale, m, h)
        res[i] = w @ Vc[h // G]
    return res


# ------------------------------------------------------------------ tree verify
# Tree verify (page "Speculative decoding and MTP on Apple silicon", Facts: the
# full-attention layers of a tree verify run with tree-attention masks): the M
# verify rows are the nodes of a draft tree instead of a chain. Readings where
# the page is silent:
#   * the nodes occupy the last M of the T valid positions, node i at T - M + i;
#   * node i sees every committed position (j < T - M) and node t iff bit t of
#     mask[i] is set — its ancestors; a node always sees itself, and bits at or
#     above M are ignored;
#   * the chain mask (bits 0..i for node i) is the causal case above.

def visible_keys(M: int, T: int, mask, m: int) -> np.ndarray:
    """Key indices row m sees, in increasing order."""
    bits = int(mask[m]) | (1 << m)
    return np.array(list(range(T - M)) + [T - M + t for t in range(M) if (bits >> t) & 1], dtype=np.int64)


def tree_attention_weights(q, k_cache, M: int, Hq: int, Hkv: int, D: int, T: int, T_cap: int,
                           scale: float, mask, m: int, h: int) -> np.ndarray:
    """float64 softmax weights w[j] (length T, zero where not visible) of row m, head h."""
    G = Hq // Hkv
    Q = bf16_to_f64(q).reshape(M, Hq, D)
    Kc = _kv(k_cache, Hkv, T_cap, D, T)
    idx = visible_keys(M, T, mask, m)
    s = scale * (Kc[h // G, idx, :] @ Q[m, h, :])
    e = np.exp(s - s.max())
    w = np.zeros(T)
    w[idx] = e / e.sum()
    return w


def tree_attention(q, k_cache, v_cache, M: int, Hq: int, Hkv: int, D: int, T: int, T_cap: int,
                   scale: float, mask, pairs=None) -> np.ndarray:
    """float64 output o[M, Hq, D] of tree verify (or the listed (m, h) rows only)."""
    Vc = _kv(v_cache, Hkv, T_cap, D, T)
    G = Hq // Hkv
    todo = [(m, h) for m in range(M) for h in range(Hq)] if pairs is None else list(pairs)
    res = np.empty((len(todo), D))
    for i, (m, h) in enumerate(todo):
        w = tree_attention_weights(q, k_cache, M, Hq, Hkv, D, T, T_cap, scale, mask, m, h)
        res[i] = w @ Vc[h // G]
    return res.reshape(M, Hq, D) if pairs is None else res


def algorithmic_bytes(M: int, Hq: int, Hkv: int, D: int, T: int) -> int:
    """K and V rows read once per KV head, plus Q in and O out (bf16)."""
    return 4 * Hkv * T * D + 4 * M * Hq * D
