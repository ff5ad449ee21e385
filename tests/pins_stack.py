"""Pins for the verify-step composition oracle (oracle/stack.py), each taking the
oracle module as an argument so that the mutation tests can run them against
deliberately broken copies.

What pins it, other than itself:
  * a hand-derived one-layer fixture whose every value is exact
    (tests/golden/stack_hand.json, derivation written out there);
  * hand values of the bf16 rounding (ties to even, negative ties, subnormals,
    the case where a detour through float32 would round twice), and bit-level
    agreement with the float32 -> bf16 rounding of the input generator where the
    two must agree (inputs that are float32 values);
  * per-element Python loops written here from the definitions: RMSNorm with
    math.sqrt, SiLU with math.exp, bf16 rounding by integer arithmetic on the
    float64 bits, the quantized products by dequantising code by code from the
    hex text of the packed words, attention with math.exp (the attention pins'
    brute force), and the layer order of the reading, including where the new
    K/V rows are appended;
  * the layer schedule written out by hand (attention on layers 3, 7, ..., 63).
"""
from __future__ import annotations

import json
import math
import os
import struct

import numpy as np

from synth import attn_inputs, f32_to_bf16_bits, qmm_activations, qmm_weights
from tests.pins_attn import attn_bruteforce
from tests.pins_qmm import _bf16_scalar, _code_bruteforce

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
EPS = 1e-6


# ------------------------------------------------------------- loop references
def bf16_round_int(x: float) -> float:
    """Nearest bf16 value, ties to even, by integer arithmetic on the float64 bits:
    keep the top 8 of the 53 significand bits and round on the 45 dropped ones
    (normal bf16 range and zero only)."""
    if x == 0.0:
        return x
    u = struct.unpack("<Q", struct.pack("<d", float(x)))[0]
    sign, exp, man = u >> 63, (u >> 52) & 0x7FF, u & ((1 << 52) - 1)
    assert abs(x) >= 2.0 ** -126 and exp < 2047, x
    sig = (1 << 52) | man
    keep, drop, half = sig >> 45, sig & ((1 << 45) - 1), 1 << 44
    if drop > half or (drop == half and keep & 1):
        keep += 1
    val = keep * 2.0 ** (exp - 1023 - 7)
    return -val if sign else val


def _bits_of(x: float) -> int:
    """bf16 bit pattern of a value that is already a bf16 value."""
    return struct.unpack("<I", struct.pack("<f", x))[0] >> 16


def rms_loop(rows):
    out = []
    for r in rows:
        d = math.sqrt(sum(v * v for v in r) / len(r) + EPS)
        out.append([v / d for v in r])
    return out


def silu_loop(g: float) -> float:
    if -g > 700.0:          # exp(-g) overflows; silu(g) -> -0
        return -0.0
    return g / (1.0 + math.exp(-g))


def _dequant_rows(w):
    """W[n][k] as Python floats, code by code from the hex text of the words."""
    N, K, bits, gs = w["N"], w["K"], w["bits"], w["group_size"]
    words = np.asarray(w["wq"]).reshape(-1)
    s = np.asarray(w["scales"]).reshape(N, K // gs)
    b = np.asarray(w["biases"]).reshape(N, K // gs)
    return [[_bf16_scalar(s[n, k // gs]) * _code_bruteforce(words, bits, K, n, k) + _bf16_scalar(b[n, k // gs])
             for k in range(K)] for n in range(N)]


def qmm_loop(rows, w, rnd=True):
    W = _dequant_rows(w)
    out = []
    for r in rows:
        y = [sum(r[k] * Wn[k] for k in range(len(r))) for Wn in W]
        out.append([bf16_round_int(v) for v in y] if rnd else y)
    return out


def layer_loop(h, w, attn, kv, ctx, Hq, Hkv, D, inter):
    """One block of the reading, element by element; kv = {"k", "v"} float
    arrays [Hkv, T_cap, D] updated in place."""
    M = len(h)
    a = [[bf16_round_int(v) for v in r] for r in rms_loop(h)]
    qkv = qmm_loop(a, w["qkv"])
    q = [r[: Hq * D] for r in qkv]
    if attn:
        for m in range(M):
            for j in range(Hkv):
                for d in range(D):
                    kv["k"][j, ctx + m, d] = qkv[m][Hq * D + j * D + d]
                    kv["v"][j, ctx + m, d] = qkv[m][(Hq + Hkv) * D + j * D + d]
        T_cap = kv["k"].shape[1]
        to_bits = np.vectorize(_bits_of, otypes=[np.uint32])
        qb = to_bits(np.array(q)).astype(np.uint16).reshape(M, Hq, D)
        kb = to_bits(kv["k"]).astype(np.uint16)
        vb = to_bits(kv["v"]).astype(np.uint16)
        o = attn_bruteforce(qb, kb, vb, M, Hq, Hkv, D, ctx + M, T_cap, 1.0 / math.sqrt(D))
        c = [[bf16_round_int(float(v)) for v in o[m].reshape(-1)] for m in range(M)]
    else:
        c = q
    oo = qmm_loop(c, w["o"])
    h = [[bf16_round_int(h[m][n] + oo[m][n]) for n in range(len(h[m]))] for m in range(M)]
    a2 = [[bf16_round_int(v) for v in r] for r in rms_loop(h)]
    gu = qmm_loop(a2, w["gate_up"])
    act = [[bf16_round_int(silu_loop(r[i]) * r[inter + i]) for i in range(inter)] for r in gu]
    dn = qmm_loop(act, w["down"])
    return [[bf16_round_int(h[m][n] + dn[m][n]) for n in range(len(h[m]))] for m in range(M)]


# --------------------------------------------------------------------- inputs
def _pack_words(codes, bits):
    """uint32 words of integer codes [N, K] (low field first)."""
    codes = np.asarray(codes, dtype=np.uint64)
    N, K = codes.shape
    per = 32 // bits
    words = np.zeros((N, K // per), dtype=np.uint64)
    for j in range(per):
        words |= codes[:, j::per] << np.uint64(bits * j)
    return words.astype(np.uint32)


def hand_fixture():
    with open(os.path.join(GOLDEN, "stack_hand.json")) as f:
        fx = json.load(f)
    mats = {}
    for name, spec in fx["matrices"].items():
        N, K = spec["N"], spec["K"]
        codes = np.zeros((N, K), dtype=np.int64)
        sc = np.zeros((N, K // 64), dtype=np.uint16)
        bi = np.zeros((N, K // 64), dtype=np.uint16)
        for row in spec["rows"]:
            if row[0] in ("even", "odd"):
                ns = range(0 if row[0] == "even" else 1, N, 2)
                pat, code, s, b = row[1:]
            else:
                ns = range(row[0], row[1])
                pat, code, s, b = row[2:]
            ks = {"all": range(K), "even_k": range(0, K, 2), "odd_k": range(1, K, 2),
                  "k_ge_32": range(32, K)}[pat]
            for n in ns:
                for k in ks:
                    codes[n, k] = code
                sc[n, :] = int(s, 16)
                bi[n, :] = int(b, 16)
        mats[name] = {"wq": _pack_words(codes, 4), "scales": sc, "biases": bi, "bits": 4, "group_size": 64,
                      "N": N, "K": K}
    return fx, mats


def small_stack(seed: int, bits: int, layers: int, M: int = 3, hidden: int = 64, inter: int = 64,
                Hq: int = 2, Hkv: int = 1, D: int = 32, n_attn: int = 1, ctx: int = 5):
    """Tiny stack with activations of order 1 (zero-mean scales)."""
    Eq2 = (2 ** bits - 1) * (2 ** (bits + 1) - 1) / 6.0        # E[q^2] of uniform codes
    Ls = []
    for li in range(layers):
        lw = {}
        for j, (name, N, K) in enumerate((("qkv", (Hq + 2 * Hkv) * D, hidden), ("o", hidden, Hq * D),
                                          ("gate_up", 2 * inter, hidden), ("down", hidden, inter))):
            lw[name] = qmm_weights(400 + seed, N, K, bits, layer=10 * li + j, scale_mean=0.0,
                                   scale_std=1.0 / math.sqrt(K * Eq2), bias_std=0.01)
        Ls.append(lw)
    T_cap = ctx + M + 2
    kvs = []
    for a in range(n_attn):
        _, k, v = attn_inputs(400 + seed, M, Hq, Hkv, D, T_cap, extra=a)
        kvs.append({"k": _wide(k), "v": _wide(v)})
    h = _wide(qmm_activations(400 + seed, M, hidden))
    return Ls, kvs, h, dict(ctx=ctx, Hq=Hq, Hkv=Hkv, D=D, inter=inter)


def _wide(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _copy_kv(kv):
    return {"k": kv["k"].copy(), "v": kv["v"].copy()}


# ----------------------------------------------------------------------- pins
def pin_round_bf16_hand(mod):
    with open(os.path.join(GOLDEN, "stack_hand.json")) as f:
        cases = json.load(f)["round_bf16_cases"]
    for name, x, want in cases:
        got = float(mod.round_bf16(np.array([x]))[0])
        assert got == want, (name, got, want)
        assert float(mod.round_bf16(np.array([-x]))[0]) == -want, name


def pin_round_bf16_bits(mod):
    """float32 inputs: the oracle's bits equal the generator's float32 -> bf16 rounding
    (a single rounding either way), including exact ties; float64 inputs: equal to
    the integer rounding of the float64 bits."""
    rng = np.random.default_rng(11)
    f = (rng.standard_normal(20000) * np.exp(rng.uniform(-30, 30, 20000))).astype(np.float32)
    ties = ((rng.integers(0x3F800000 >> 16, 0x4F800000 >> 16, 2000).astype(np.uint32) << 16) | 0x8000)
    f = np.concatenate([f, ties.view(np.float32), -ties.view(np.float32)])
    assert np.array_equal(mod.to_bf16_bits(f.astype(np.float64)), f32_to_bf16_bits(f))
    x = rng.standard_normal(3000) * np.exp(rng.uniform(-20, 20, 3000))
    got = mod.round_bf16(x)
    assert all(float(g) == bf16_round_int(float(v)) for g, v in zip(got, x))


def pin_rmsnorm(mod):
    rng = np.random.default_rng(12)
    h = rng.standard_normal((3, 40)) * np.array([[1.0], [1e-3], [50.0]])
    ref = np.array(rms_loop(h.tolist()))
    assert np.allclose(mod.rmsnorm(h), ref, rtol=1e-14, atol=0)
    assert np.allclose(mod.rmsnorm(np.array([[3.0, 4.0]])), [[3 / math.sqrt(12.5 + EPS), 4 / math.sqrt(12.5 + EPS)]],
                       rtol=1e-15, atol=0)
    tiny = mod.rmsnorm(np.full((1, 8), 1e-3))            # eps is inside the root: 1e-3 / sqrt(2e-6)
    assert abs(float(tiny[0, 0]) - 1e-3 / math.sqrt(2e-6)) < 1e-12


def pin_silu(mod):
    rng = np.random.default_rng(13)
    g = rng.standard_normal(500) * 6
    u = rng.standard_normal(500)
    ref = np.array([silu_loop(a) * b for a, b in zip(g, u)])
    assert np.allclose(mod.silu_mul(g, u), ref, rtol=1e-14, atol=1e-300)
    x = np.linspace(-30, 30, 121)
    ones = np.ones_like(x)
    assert np.allclose(mod.silu_mul(x, ones) - mod.silu_mul(-x, ones), x, rtol=0, atol=1e-13)
    assert float(mod.silu_mul(np.array([2.0]), np.array([3.0]))[0]) == 6.0 / (1.0 + math.exp(-2.0))
    big = mod.silu_mul(np.array([-1000.0, 1000.0]), np.array([1.0, 1.0]))
    assert big[0] == 0.0 and big[1] == 1000.0


def pin_hand_layer(mod):
    fx, mats = hand_fixture()
    s = fx["shape"]
    h0 = np.full((s["M"], s["hidden"]), fx["h0"])
    h = mod.layer_forward(h0, mats, s["attention"], None, 0, s["Hq"], s["Hkv"], s["D"], s["inter"])
    want = np.where(np.arange(s["hidden"]) % 2 == 0, fx["expected_h_even"], fx["expected_h_odd"])
    assert np.array_equal(h[0], want), h[0]
    # the same fixture through the per-element loops (they must agree with the hand values too)
    assert layer_loop(h0.tolist(), mats, False, None, 0, s["Hq"], s["Hkv"], s["D"], s["inter"])[0] == want.tolist()


def pin_layer_bruteforce(mod):
    for seed, bits, attn in ((0, 4, True), (1, 8, True), (2, 4, False)):
        Ls, kvs, h, a = small_stack(seed, bits, 1)
        kv_o, kv_b = _copy_kv(kvs[0]), _copy_kv(kvs[0])
        got = mod.layer_forward(h, Ls[0], attn, kv_o if attn else None, **a)
        ref = np.array(layer_loop(h.tolist(), Ls[0], attn, kv_b, **a))
        assert np.allclose(got, ref, rtol=1e-12, atol=0), (seed, bits, attn, np.abs(got - ref).max())
        assert np.array_equal(kv_o["k"], kv_b["k"]) and np.array_equal(kv_o["v"], kv_b["v"]), "appended rows"
        assert np.abs(got).max() < 20.0           # activations of order 1


def pin_append_position(mod):
    """An attention layer writes its new K/V rows at ctx .. ctx+M-1 and nothing else."""
    Ls, kvs, h, a = small_stack(3, 4, 1, M=2, ctx=4)
    kv = _copy_kv(kvs[0])
    mod.layer_forward(h, Ls[0], True, kv, **a)
    M, ctx, Hq, Hkv, D = 2, a["ctx"], a["Hq"], a["Hkv"], a["D"]
    rms = [[bf16_round_int(v) for v in r] for r in rms_loop(h.tolist())]
    qkv = np.array(qmm_loop(rms, Ls[0]["qkv"]))
    for m in range(M):
        assert np.array_equal(kv["k"][:, ctx + m, :], qkv[m, Hq * D:(Hq + Hkv) * D].reshape(Hkv, D))
        assert np.array_equal(kv["v"][:, ctx + m, :], qkv[m, (Hq + Hkv) * D:].reshape(Hkv, D))
    untouched = [j for j in range(kv["k"].shape[1]) if not ctx <= j < ctx + M]
    assert np.array_equal(kv["k"][:, untouched], kvs[0]["k"][:, untouched])
    assert np.array_equal(kv["v"][:, untouched], kvs[0]["v"][:, untouched])


def pin_schedule(mod):
    assert [l for l in range(64) if mod.is_attention_layer(l)] == [3, 7, 11, 15, 19, 23, 27, 31, 35, 39, 43, 47,
                                                                     51, 55, 59, 63]
    assert [l for l in range(8) if mod.is_attention_layer(l, 2)] == [1, 3, 5, 7]


def pin_stack_forward(mod):
    """Four layers, attention on layer 3 (every 4) -- each layer's output against the loops."""
    Ls, kvs, h, a = small_stack(4, 4, 4, M=2)
    kv_o, kv_b = _copy_kv(kvs[0]), _copy_kv(kvs[0])
    outs = mod.stack_forward(h, Ls, [kv_o], attn_every=4, **a)
    assert len(outs) == 4
    cur = h.tolist()
    for li in range(4):
        cur = layer_loop(cur, Ls[li], li == 3, kv_b if li == 3 else None, **a)
        assert np.allclose(outs[li], np.array(cur), rtol=1e-12, atol=0), li
    assert np.array_equal(kv_o["k"], kv_b["k"])


def pin_lm_head(mod):
    rng = np.random.default_rng(14)
    h = _wide(f32_to_bf16_bits(rng.standard_normal((2, 64)).astype(np.float32)))
    w = qmm_weights(450, 40, 64, 4)
    a = [[bf16_round_int(v) for v in r] for r in rms_loop(h.tolist())]
    ref = np.array(qmm_loop(a, w, rnd=False))
    got = mod.lm_head_logits(h, w)
    assert np.allclose(got, ref, rtol=1e-12, atol=0)
    cols = [0, 7, 39]
    assert np.array_equal(mod.lm_head_logits(h, w, cols=cols), got[:, cols])


PINS = [pin_round_bf16_hand, pin_round_bf16_bits, pin_rmsnorm, pin_silu, pin_hand_layer, pin_layer_bruteforce,
        pin_append_position, pin_schedule, pin_stack_forward, pin_lm_head]
