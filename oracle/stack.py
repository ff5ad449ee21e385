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
    with gate|up = gate_up(rms(h)); RMSNorm with unit weight and eps = 1e-6;
  * attention runs on every fourth layer (layers 3, 7, ..., 63 of 64); the
    recurrent layers are out of scope, so on the other layers the query slice
    of the fused q|k|v output feeds the o projection directly;
  * the M new K/V rows are written at cache positions ctx .. ctx+M-1 before the
    attention call, which then sees T = ctx + M keys;
  * activations are stored as bf16 between kernels (bf16 activations on every
    pass: page "The fastest way to run local LLMs on a Mac", section "Why exact
    acceptance matters"), so this oracle rounds to bf16 at the same points and
    computes everything else in float64;
  * the final RMSNorm output goes through the lm_head projection to float32
    logits, which feed the acceptance step.
"""
from __future__ import annotations

import numpy as np

from . import attn as _attn
from . import qmm as _qmm

RMS_EPS = 1e-6


def round_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bf16 value (via float32, ties to even)."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint32) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def to_bf16_bits(x) -> np.ndarray:
    """bf16 bit patterns of float64 values (rounded as in ``round_bf16``)."""
    f = round_bf16(x).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def rmsnorm(h: np.ndarray, eps: float = RMS_EPS) -> np.ndarray:
    """h / sqrt(mean(h**2) + eps) per row (unit weight)."""
    return h / np.sqrt(np.mean(h * h, axis=-1, keepdims=True) + eps)


def silu_mul(gate: np.ndarray, up: np.ndarray) -> np.ndarray:
    """silu(gate) * up = gate / (1 + exp(-gate)) * up."""
    return gate / (1.0 + np.exp(-gate)) * up


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
    generator). ``kv`` holds float64-valued caches "k", "v" [Hkv, T_cap, D]
    (bf16 values) and is updated in place on attention layers.
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


def lm_head_logits(h: np.ndarray, w: dict, cols=None) -> np.ndarray:
    """float64 logits (or the chosen columns) of the final RMSNorm output."""
    a = round_bf16(rmsnorm(h))
    M, K = a.shape
    return _qmm.skinny_qmm(to_bf16_bits(a), w["wq"], w["scales"], w["biases"], w["bits"],
                           w["group_size"], M, w["N"], K, cols=cols)
