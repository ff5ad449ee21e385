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


PINS = [pin_rows_sum_to_one, pin_bruteforce, pin_textbook, pin_special_cases, pin_causality]
