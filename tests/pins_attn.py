"""Pins for the multi-row attention oracle (module passed in, for mutation tests)."""
from __future__ import annotations

import math
import struct

import numpy as np

from synth import attn_inputs, f32_to_bf16_bits


def _f(bits) -> float:
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def attn_bruteforce(q, k, v, M, Hq, Hkv, D, T, T_cap, scale):
    """Pure-Python loops with math.exp."""
    G = Hq // Hkv
    out = np.zeros((M, Hq, D))
    for i in range(M):
        for h in range(Hq):
            kv = h // G
            limit = T - M + i
            s = []
            for j in range(limit + 1):
                s.append(scale * sum(_f(q[i, h, d]) * _f(k[kv, j, d]) for d in range(D)))
            mx = max(s)
            e = [math.exp(t - mx) for t in s]
            z = sum(e)
            for d in range(D):
                out[i, h, d] = sum(e[j] / z * _f(v[kv, j, d]) for j in range(limit + 1))
    return out


def attn_textbook(q, k, v, M, Hq, Hkv, D, T, T_cap, scale):
    """softmax(scale * Q K^T + mask) V with each KV head repeated for its G query heads."""
    G = Hq // Hkv
    wid = lambda a: (np.asarray(a, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    Q = wid(q).reshape(M, Hq, D).transpose(1, 0, 2)                    # [Hq, M, D]
    Kr = np.repeat(wid(k).reshape(Hkv, T_cap, D)[:, :T], G, axis=0)    # [Hq, T, D]
    Vr = np.repeat(wid(v).reshape(Hkv, T_cap, D)[:, :T], G, axis=0)
    S = scale * Q @ Kr.transpose(0, 2, 1)                               # [Hq, M, T]
    mask = np.arange(T)[None, :] > (T - M + np.arange(M))[:, None]      # [M, T]
    S = np.where(mask[None], -np.inf, S)
    S = S - S.max(axis=-1, keepdims=True)
    W = np.exp(S)
    W /= W.sum(axis=-1, keepdims=True)
    return (W @ Vr).transpose(1, 0, 2)                                  # [M, Hq, D]


def _small(seed, M=3, Hq=4, Hkv=2, D=8, T=10, T_cap=12):
    q, k, v = attn_inputs(200 + seed, M, Hq, Hkv, D, T_cap)
    return q, k, v, dict(M=M, Hq=Hq, Hkv=Hkv, D=D, T=T, T_cap=T_cap, scale=1 / math.sqrt(D))


def pin_rows_sum_to_one(mod):
    q, k, v, a = _small(0, M=4, Hq=6, Hkv=2, D=16, T=40, T_cap=48)
    for m in range(a["M"]):
        for h in range(a["Hq"]):
            w = mod.attention_weights(q, k, a["M"], a["Hq"], a["Hkv"], a["D"], a["T"], a["T_cap"], a["scale"], m, h)
            assert abs(w.sum() - 1.0) <= 1e-12
            assert np.all(w[a["T"] - a["M"] + m + 1:] == 0.0) and np.all(w[: a["T"] - a["M"] + m + 1] > 0)


def pin_bruteforce(mod):
    for seed in (1, 2):
        q, k, v, a = _small(seed)
        ref = attn_bruteforce(q, k, v, **a)
        got = mod.multirow_attention(q, k, v, **a)
        assert np.allclose(got, ref, rtol=0, atol=1e-12)


def pin_textbook(mod):
    for seed, shape in ((3, dict(M=4, Hq=2, Hkv=2, D=64, T=256, T_cap=256)),
                        (4, dict(M=5, Hq=12, Hkv=2, D=32, T=70, T_cap=80))):
        q, k, v, a = _small(seed, **shape)
        ref = attn_textbook(q, k, v, **a)
        assert np.allclose(mod.multirow_attention(q, k, v, **a), ref, rtol=0, atol=1e-12)
        pairs = [(0, 0), (a["M"] - 1, a["Hq"] - 1), (a["M"] // 2, 1)]
        got = mod.multirow_attention(q, k, v, **a, pairs=pairs)
        assert np.allclose(got, np.stack([ref[m, h] for m, h in pairs]), rtol=0, atol=1e-12)


def pin_special_cases(mod):
    # M = 1: ordinary single-token decode attention over all T keys.
    q, k, v, a = _small(5, M=1, T=9)
    wid = lambda x: (np.asarray(x, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    Q, Kc, Vc = wid(q)[0], wid(k), wid(v)
    for h in range(a["Hq"]):
        s = a["scale"] * Kc[h // 2, :9] @ Q[h]
        w = np.exp(s - s.max()); w /= w.sum()
        assert np.allclose(mod.multirow_attention(q, k, v, **a)[0, h], w @ Vc[h // 2, :9], atol=1e-12)
    # identical keys: every visible key gets the same weight -> mean of the visible values.
    q, k, v, a = _small(6, M=3, T=7)
    k[:] = k[:, :1, :]
    out = mod.multirow_attention(q, k, v, **a)
    Vc = wid(v)
    for m in range(3):
        for h in range(a["Hq"]):
            assert np.allclose(out[m, h], Vc[h // 2, : 7 - 3 + m + 1].mean(axis=0), atol=1e-12)
    # T = M = 1: the only visible value.
    q, k, v, a = _small(7, M=1, T=1)
    out = mod.multirow_attention(q, k, v, **a)
    for h in range(a["Hq"]):
        assert np.array_equal(out[0, h], wid(v)[h // 2, 0])
    # very large scale with a unique best key: the value of that key.
    q, k, v, a = _small(8, M=2, T=12)
    a["scale"] = 1e6
    out = mod.multirow_attention(q, k, v, **a)
    Q, Kc, Vc = wid(q), wid(k), wid(v)
    for m in range(2):
        for h in range(a["Hq"]):
            s = Kc[h // 2, : 12 - 2 + m + 1] @ Q[m, h]
            assert np.allclose(out[m, h], Vc[h // 2, int(np.argmax(s))], atol=1e-9)


def pin_causality(mod):
    """Changing keys/values a row cannot see leaves that row bit-identical."""
    q, k, v, a = _small(9, M=4, T=20, T_cap=20)
    base = mod.multirow_attention(q, k, v, **a)
    for m in range(a["M"]):
        k2, v2 = k.copy(), v.copy()
        lim = a["T"] - a["M"] + m
        if lim + 1 >= a["T"]:
            continue
        k2[:, lim + 1:, :] = f32_to_bf16_bits(np.full(k2[:, lim + 1:, :].shape, 3.0, np.float32))
        v2[:, lim + 1:, :] = f32_to_bf16_bits(np.full(v2[:, lim + 1:, :].shape, -7.0, np.float32))
        out = mod.multirow_attention(q, k2, v2, **a)
        assert np.array_equal(out[m], base[m])
        assert not np.array_equal(out[a["M"] - 1], base[a["M"] - 1])


# ------------------------------------------------------------------ tree verify
def tree_bruteforce(q, k, v, M, Hq, Hkv, D, T, T_cap, scale, mask):
    """Pure-Python loops with math.exp: row i sees keys j < T - M, and key T - M + t
    when t == i or bit t of mask[i] is set (t < M)."""
    G = Hq // Hkv
    out = np.zeros((M, Hq, D))
    for i in range(M):
        vis = [j for j in range(T - M)]
        for t in range(M):
            if t == i or (int(mask[i]) >> t) & 1:
                vis.append(T - M + t)
        for h in range(Hq):
            kv = h // G
            s = [scale * sum(_f(q[i, h, d]) * _f(k[kv, j, d]) for d in range(D)) for j in vis]
            mx = max(s)
            e = [math.exp(t - mx) for t in s]
            z = sum(e)
            for d in range(D):
                out[i, h, d] = sum(e[n] / z * _f(v[kv, j, d]) for n, j in enumerate(vis))
    return out


def tree_textbook(q, k, v, M, Hq, Hkv, D, T, T_cap, scale, mask):
    """softmax(scale * Q K^T + tree mask) V, the [M, T] mask built with numpy bit operations."""
    G = Hq // Hkv
    wid = lambda a: (np.asarray(a, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    Q = wid(q).reshape(M, Hq, D).transpose(1, 0, 2)
    Kr = np.repeat(wid(k).reshape(Hkv, T_cap, D)[:, :T], G, axis=0)
    Vr = np.repeat(wid(v).reshape(Hkv, T_cap, D)[:, :T], G, axis=0)
    S = scale * Q @ Kr.transpose(0, 2, 1)
    bits = (np.asarray(mask, np.uint64)[:, None] >> np.arange(M, dtype=np.uint64)[None, :]) & 1
    seen = np.concatenate([np.ones((M, T - M), bool), (bits == 1) | np.eye(M, dtype=bool)], axis=1)
    S = np.where(seen[None], S, -np.inf)
    S = S - S.max(axis=-1, keepdims=True)
    W = np.exp(S)
    W /= W.sum(axis=-1, keepdims=True)
    return (W @ Vr).transpose(1, 0, 2)


def pin_tree_chain_is_causal(mod):
    """The chain mask is the causal case, value for value."""
    from synth import chain_masks
    q, k, v, a = _small(11, M=5, Hq=6, Hkv=2, D=16, T=30, T_cap=32)
    got = mod.tree_attention(q, k, v, **a, mask=chain_masks(a["M"]))
    assert np.allclose(got, mod.multirow_attention(q, k, v, **a), rtol=0, atol=1e-15)


def pin_tree_bruteforce(mod):
    from synth import tree_masks
    for seed, M in ((12, 5), (13, 4)):
        q, k, v, a = _small(seed, M=M, Hq=4, Hkv=2, D=8, T=12, T_cap=14)
        mask = tree_masks(seed, M)
        ref = tree_bruteforce(q, k, v, **a, mask=mask)
        assert np.allclose(mod.tree_attention(q, k, v, **a, mask=mask), ref, rtol=0, atol=1e-12)


def pin_tree_textbook(mod):
    """Random trees and arbitrary masks (self bit missing, bits at or above M set)."""
    from synth import tree_masks
    for seed, shape in ((14, dict(M=8, Hq=12, Hkv=2, D=32, T=90, T_cap=96)),
                        (15, dict(M=16, Hq=4, Hkv=4, D=16, T=16, T_cap=16))):
        q, k, v, a = _small(seed, **shape)
        for mask in (tree_masks(seed, a["M"]), np.array([0, 0xFFFF0001, 5, 2, 0xF0] * 4, np.uint32)[: a["M"]]):
            ref = tree_textbook(q, k, v, **a, mask=mask)
            assert np.allclose(mod.tree_attention(q, k, v, **a, mask=mask), ref, rtol=0, atol=1e-12)
            pairs = [(0, 0), (a["M"] - 1, a["Hq"] - 1)]
            got = mod.tree_attention(q, k, v, **a, mask=mask, pairs=pairs)
            assert np.allclose(got, np.stack([ref[m, h] for m, h in pairs]), rtol=0, atol=1e-12)


def pin_tree_self_only_is_decode(mod):
    """A node that sees only itself among the drafted rows is single-row decode
    attention over the context followed by its own key and value."""
    q, k, v, a = _small(16, M=4, Hq=4, Hkv=2, D=16, T=24, T_cap=24)
    M, T = a["M"], a["T"]
    mask = np.array([1 << i for i in range(M)], np.uint32)
    got = mod.tree_attention(q, k, v, **a, mask=mask)
    for i in range(M):
        keep = list(range(T - M)) + [T - M + i]
        k1, v1 = k[:, keep], v[:, keep]
        one = mod.multirow_attention(q[i:i + 1], k1, v1, 1, a["Hq"], a["Hkv"], a["D"], len(keep), len(keep),
                                     a["scale"])
        assert np.allclose(got[i], one[0], rtol=0, atol=1e-13)


def pin_tree_weights(mod):
    """Weights sum to one, are zero exactly on the keys the node does not see."""
    from synth import tree_masks
    q, k, v, a = _small(17, M=8, Hq=4, Hkv=2, D=16, T=40, T_cap=40)
    mask = tree_masks(17, a["M"])
    for m in range(a["M"]):
        w = mod.tree_attention_weights(q, k, a["M"], a["Hq"], a["Hkv"], a["D"], a["T"], a["T_cap"], a["scale"],
                                       mask, m, 1)
        assert abs(w.sum() - 1.0) <= 1e-12
        seen = [t for t in range(a["M"]) if (int(mask[m]) >> t) & 1]
        tail = w[a["T"] - a["M"]:]
        assert np.all(tail[seen] > 0) and np.all(np.delete(tail, seen) == 0) and np.all(w[: a["T"] - a["M"]] > 0)


PINS = [pin_rows_sum_to_one, pin_bruteforce, pin_textbook, pin_special_cases, pin_causality,
        pin_tree_chain_is_causal, pin_tree_bruteforce, pin_tree_textbook, pin_tree_self_only_is_decode,
        pin_tree_weights]
