"""Pins for the 8-bit KV oracle (module passed in, for mutation tests)."""
from __future__ import annotations

import math
import struct

import numpy as np

import oracle.attn as oattn
from synth import attn_inputs, f32_to_bf16_bits, tree_masks


def _f(bits) -> float:
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def _wid(a):
    return (np.asarray(a, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _grid_rows(seed, shape, step_exp=-6):
    """bf16 rows whose every 64-group is b + s*q with s = 2**step_exp, b a bf16
    value, q integers in [0, 255] reaching 0 and 255: the quantizer must return
    exactly (q, s, b)."""
    g = np.random.default_rng(seed)
    D = shape[-1]
    n = int(np.prod(shape[:-1])) * (D // 64)
    q = g.integers(0, 256, size=(n, 64))
    q[:, 0], q[:, 1] = 0, 255
    # b = k*s with k in [-256, 0]: every b + s*q = (k + q)*s has |k + q| <= 256,
    # which bf16 (8 significant bits) holds exactly
    b = -g.integers(0, 257, size=n) * 2.0 ** step_exp
    x = b[:, None] + q * 2.0 ** step_exp
    bits = f32_to_bf16_bits(x.astype(np.float32))
    assert np.array_equal(_wid(bits), x), "grid values must be exact in bf16"
    return bits.reshape(shape), q.reshape(shape).astype(np.uint8), b


def pin_quantize_exact_grid(mod):
    bits, q, b = _grid_rows(1, (3, 5, 128))
    codes, sb = mod.quantize_rows(bits)
    assert np.array_equal(codes, q)
    assert np.all(_wid(sb[..., 0]) == 2.0 ** -6)
    assert np.array_equal(_wid(sb[..., 1]).reshape(-1), b)
    assert np.array_equal(mod.dequantize(codes, sb), _wid(bits))


def pin_quantize_bounds(mod):
    """Random rows: codes span [0, 255] with the min at 0 and the max at 255, and the
    dequantized value is within half a step (of the bf16 scale) plus the scale's
    own rounding of the input."""
    x = attn_inputs(30, 1, 1, 4, 256, 40)[1]          # [4, 40, 256] bf16 ~ N(0, 1)
    codes, sb = mod.quantize_rows(x)
    xf = _wid(x).reshape(4, 40, 4, 64)
    cg = codes.reshape(4, 40, 4, 64)
    assert np.all(cg.min(axis=-1) == 0) and np.all(cg.max(axis=-1) == 255)
    assert np.array_equal(np.take_along_axis(cg, xf.argmin(axis=-1)[..., None], -1)[..., 0], np.zeros((4, 40, 4)))
    s = _wid(sb[..., 0])
    err = np.abs(mod.dequantize(codes, sb).reshape(4, 40, 4, 64) - xf)
    span = xf.max(-1) - xf.min(-1)
    assert np.all(err <= 0.5 * s[..., None] * (1 + 2 ** -6) + span[..., None] * 2 ** -8)
    assert np.all(mod.dequantize(codes, sb).reshape(4, 40, 4, 64).min(-1) == xf.min(-1))


def pin_quantize_constant_and_scalar(mod):
    """A constant group: codes 0, scale 0, bias = the value (dequantizes exactly).
    One group checked element by element with Python floats: float32 division,
    round half to even."""
    x = np.full((2, 64), f32_to_bf16_bits(np.array([1.75], np.float32))[0], np.uint16)
    x[1] = f32_to_bf16_bits(np.linspace(-3, 5, 64).astype(np.float32))
    codes, sb = mod.quantize_rows(x)
    assert np.all(codes[0] == 0) and _wid(sb[0, 0, 0]) == 0 and _wid(sb[0, 0, 1]) == 1.75
    row = [_f(v) for v in x[1]]
    mn, mx = min(row), max(row)
    s32 = np.float32(np.float32(mx - mn) / np.float32(255))
    for i, v in enumerate(row):
        t = np.float32(np.float32(np.float32(v) - np.float32(mn)) / s32)
        assert codes[1, i] == int(min(255, max(0, round(float(t)))))   # round(): half to even
    assert sb[1, 0, 0] == f32_to_bf16_bits(np.array([s32], np.float32))[0]


def _cache(seed, M, Hq, Hkv, D, T):
    q, k, v = attn_inputs(seed, M, Hq, Hkv, D, T)
    kc, ks = __import__("oracle.kv8", fromlist=["x"]).quantize_rows(k)
    vc, vs = __import__("oracle.kv8", fromlist=["x"]).quantize_rows(v)
    return q, kc, ks, vc, vs


def pin_int8_attention_exact_grid(mod):
    """Caches whose values lie on the quantization grid: int8 attention is the
    bf16 attention of oracle/attn.py on the same values (causal and tree)."""
    M, Hq, Hkv, D, T = 4, 6, 2, 64, 30
    q = attn_inputs(31, M, Hq, Hkv, D, T)[0]
    kb, kq, _ = _grid_rows(2, (Hkv, T, D), step_exp=-7)
    vb, vq_, _ = _grid_rows(3, (Hkv, T, D), step_exp=-5)
    kc, ks = mod.quantize_rows(kb)
    vc, vs = mod.quantize_rows(vb)
    got = mod.int8_attention(q, kc, ks, vc, vs, M, Hq, Hkv, D, T, T, 0.125)
    assert np.allclose(got, oattn.multirow_attention(q, kb, vb, M, Hq, Hkv, D, T, T, 0.125), rtol=0, atol=1e-13)
    mask = tree_masks(31, M)
    got = mod.int8_attention(q, kc, ks, vc, vs, M, Hq, Hkv, D, T, T, 0.125, mask=mask)
    assert np.allclose(got, oattn.tree_attention(q, kb, vb, M, Hq, Hkv, D, T, T, 0.125, mask), rtol=0, atol=1e-13)


def pin_int8_attention_bruteforce(mod):
    """Pure-Python loops: dequantize element by element, then causal softmax attention."""
    M, Hq, Hkv, D, T = 3, 4, 2, 64, 7
    q, kc, ks, vc, vs = _cache(32, M, Hq, Hkv, D, T)
    G = Hq // Hkv
    deq = lambda c, sb, kv, j, d: _f(sb[kv, j, d // 64, 0]) * int(c[kv, j, d]) + _f(sb[kv, j, d // 64, 1])
    got = mod.int8_attention(q, kc, ks, vc, vs, M, Hq, Hkv, D, T, T, 0.2)
    for i in range(M):
        for h in (0, Hq - 1):
            kv = h // G
            s = [0.2 * sum(_f(q[i, h, d]) * deq(kc, ks, kv, j, d) for d in range(D)) for j in range(T - M + i + 1)]
            mx = max(s)
            e = [math.exp(t - mx) for t in s]
            z = sum(e)
            for d in (0, 17, D - 1):
                ref = sum(e[j] / z * deq(vc, vs, kv, j, d) for j in range(len(e)))
                assert abs(got[i, h, d] - ref) <= 1e-12


def pin_int8_attention_rows_sum(mod):
    """All values of V equal c in a head: the output is c whatever the weights."""
    M, Hq, Hkv, D, T = 4, 4, 2, 64, 20
    q, kc, ks, vc, vs = _cache(33, M, Hq, Hkv, D, T)
    vc = np.full_like(vc, 200)
    vs = vs.copy()
    vs[..., 0] = f32_to_bf16_bits(np.array([0.25], np.float32))[0]
    vs[..., 1] = f32_to_bf16_bits(np.array([-3.0], np.float32))[0]
    got = mod.int8_attention(q, kc, ks, vc, vs, M, Hq, Hkv, D, T, T, 0.3)
    assert np.allclose(got, 0.25 * 200 - 3.0, rtol=0, atol=1e-12)


PINS = [pin_quantize_exact_grid, pin_quantize_bounds, pin_quantize_constant_and_scalar,
        pin_int8_attention_exact_grid, pin_int8_attention_bruteforce, pin_int8_attention_rows_sum]
