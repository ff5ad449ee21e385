"""Oracle: one verify step through a synthetic dense stack (test infrastructure only).

Composition of the three kernels into the verify pass the pages describe
(page "The fastest way to run local LLMs on a Mac", sections "Decode is a
memory-bandwidth problem" and "Why native MTP doubles decode": one batched
forward over the last committed token plus the drafted tokens reads every
weight once; section "Why token 1,000 is faster than token 100,000": only the
full-attention layers keep a KV cache; page "Speculative decoding and MTP on
Apple silicon", Facts: three of four layers of the hybrid model are recurrent).

Readings (the pages give no layer definition):
  * pre-norm blocks: h += o(attn(qkv(rms(h)))); h += down(silu(gate) * up)
    with gate|up = gate_up(rms(h)) (gate rows first); RMSNorm with unit weight
    and eps = 1e-6 inside the square root;
  * attention runs on every fourth layer (layers 3, 7, ..., 63 of 64; in
    general layer l when l mod every = every - 1); the recurrent layers are out
    of scope, so on the other layers the query slice of the fused q|k|v output
    feeds the o projection directly;
  * the M new K/V rows are written at cache positions ctx .. ctx+M-1 before the
    attention call, which then sees T = ctx + M keys;
  * activations are stored as bf16 between kernels (bf16 activations on every
    pass: page "The fastest way to run local LLMs on a Mac", section "Why exact
    acceptance matters"), so this oracle rounds to bf16 (nearest, ties to even,
    straight from float64) at the same points -- the RMSNorm outputs, every
    projection output, the SwiGLU output and the residual stream after each add
    -- and computes everything else in float64;
  * the final RMSNorm output goes through the lm_head projection to float32
    logits, which feed the acceptance step.

Pinned by tests/pins_stack.py: a hand-derived one-layer fixture whose values
are exact, per-element Python loops (math.sqrt, math.exp, an integer bf16
rounding of the float64 bits, dequantise-then-loop products and attention) on
tiny stacks with an attention layer, and bit-level agreement of the bf16
rounding with the float32 route where the two must agree.
"""
from __future__ import annotations

import numpy as np

from . import attn as _attn
from . import qmm as _qmm

RMS_EPS = 1e-6


def round_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bf16 value, ties to even.

    |x| = f * 2**e with f in [0.5, 1); a bf16 value has 8 significant bits, so
    its spacing at |x| is 2**(e - 8) (never below the smallest subnormal step
    2**-133); x / spacing is rounded to an integer, ties to even (np.rint).
    Zeros, infinities and NaNs pass through.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    step = np.ldexp(1.0, np.maximum(e - 8, -133))
    with np.errstate(invalid="ignore"):
        r = np.rint(x / step) * step
    return np.where(np.isfinite(x), r, x)


def to_bf16_bits(x) -> np.ndarray:
    """bf16 bit patterns of float64 values (rounded as in ``round_bf16``)."""
    f = round_bf16(x).astype(np.float32)   # exact: a bf16 value is a float32 value
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def rmsnorm(h: np.ndarray, eps: float = RMS_EPS) -> np.ndarray:
    """h / sqrt(mean(h**2) + eps) per row (unit weight)."""
    return h / np.sqrt(np.mean(h * h, axis=-1, keepdims=True) + eps)


def silu_mul(gate: np.ndarray, up: np.ndarray) -> np.ndarray:
    """silu(gate) * up = gate / (1 + exp(-gate)) * up (exp may overflow to inf for
    very negative gates; the quotient is then the correct limit, -0)."""
    with np.errstate(over="ignore"):
        return gate / (1.0 + np.exp(-gate)) * up


def is_attention_layer(layer: int, every: int = 4) -> bool:
    """Layers every-1, 2*every-1, ... are the full-attention layers."""
    return layer % every == every - 1


def qmm_bf16(a: np.ndarray, w: dict) -> np.ndarray:
    """Quantized projection of bf16-valued float64 rows, result rounded to bf16."""
    M, K = a.shape
    bits = to_bf16_bits(a)
    y = _qmm.skinny_qmm(bits, w["wq"], w["scales"], w["biases"], w["bits"], w["group_size"],
                        M, w["N"], K)
    return round_bf16(y)


def layer_forward(h: np.ndarray, w: dict, attn_layer: bool, kv: dict | None, ctx: int,
                  Hq: int, Hkv: int, D: int, inter: int) -> np.ndarray:
    """One pre-norm block on bf16-valued float64 rows h [M, hidden].

    ``w`` holds packs "qkv", "o", "gate_up", "down" (dicts as from the input
    generator; gate_up holds the inter gate rows, then the inter up rows).
    ``kv`` holds float64-valued caches "k", "v" [Hkv, T_cap, D] (bf16 values)
    and is updated in place on attention layers.
    """
    M = h.shape[0]
    a = round_bf16(rmsnorm(h))
    qkv = qmm_bf16(a, w["qkv"])
    q = qkv[:, : Hq * D]
    if attn_layer:
        k_new = qkv[:, Hq * D: (Hq + Hkv) * D].reshape(M, Hkv, D)
        v_new = qkv[:, (Hq + Hkv) * D:].reshape(M, Hkv, D)
        kv["k"][:, ctx: ctx + M, :] = k_new.transpose(1, 0, 2)
        kv["v"][:, ctx: ctx + M, :] = v_new.transpose(1, 0, 2)
        T_cap = kv["k"].shape[1]
        o = _attn.multirow_attention(to_bf16_bits(q), to_bf16_bits(kv["k"]), to_bf16_bits(kv["v"]),
                                     M, Hq, Hkv, D, ctx + M, T_cap, 1.0 / np.sqrt(D))
        ctx_in = round_bf16(o.reshape(M, Hq * D))
    else:
        ctx_in = q
    h = round_bf16(h + qmm_bf16(ctx_in, w["o"]))
    a2 = round_bf16(rmsnorm(h))
    gu = qmm_bf16(a2, w["gate_up"])
    act = round_bf16(silu_mul(gu[:, :inter], gu[:, inter:]))
    h = round_bf16(h + qmm_bf16(act, w["down"]))
    return h


def stack_forward(h: np.ndarray, layers: list, kvs: list, ctx: int, Hq: int, Hkv: int, D: int,
                  inter: int, attn_every: int = 4) -> list:
    """The layers of the stack in order on h [M, hidden]; ``kvs`` holds one cache
    dict per attention layer, in layer order (updated in place). Returns the
    hidden rows after every layer (the last entry is the stack's output)."""
    out, ai = [], 0
    for li, w in enumerate(layers):
        attn = is_attention_layer(li, attn_every)
        h = layer_forward(h, w, attn, kvs[ai] if attn else None, ctx, Hq, Hkv, D, inter)
        ai += int(attn)
        out.append(h)
    return out


def lm_head_logits(h: np.ndarray, w: dict, cols=None) -> np.ndarray:
    """float64 logits (or the chosen columns) of the final RMSNorm output."""
    a = round_bf16(rmsnorm(h))
    M, K = a.shape
    return _qmm.skinny_qmm(to_bf16_bits(a), w["wq"], w["scales"], w["biases"], w["bits"],
                           w["group_size"], M, w["N"], K, cols=cols)
