"""Seeded synthetic inputs for the verify pass (weights, activations, KV cache,
draft/target logits, uniforms).

This module is shared by the tests, the benchmark and the CPU oracle's callers.
It holds no arithmetic of the method itself: it only draws random numbers,
rounds them to the storage formats (bf16 bit patterns, packed integer words,
24-bit uniforms) and returns plain numpy arrays. Random numbers that the method
consumes (the acceptance uniforms) are drawn here and passed in as inputs.

Seeding: every array comes from ``numpy.random.default_rng`` on a
``SeedSequence(seed, spawn_key=(config, stream))`` so that each named stream of
each configuration is reproducible on its own.
"""
from __future__ import annotations

import numpy as np

# Named random streams. The integer ids are part of the seeding recipe.
STREAMS = {
    "W": 1, "S": 2, "B": 3, "X": 4,
    "Q": 5, "K": 6, "V": 7,
    "plogit": 8, "qlogit": 9, "draft-u": 10, "accept-u": 11, "tree": 12,
}

U_BITS = 24  # uniforms are k * 2**-24, k uniform in [0, 2**24)


def rng(config: int, stream: str, seed: int = 0, extra: int = 0) -> np.random.Generator:
    """Generator for one named stream of one configuration."""
    key = (int(config), STREAMS[stream], int(extra))
    return np.random.default_rng(np.random.SeedSequence(seed, spawn_key=key))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest even); return uint16 bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def bf16_normal(g: np.random.Generator, shape, mean: float = 0.0, std: float = 1.0) -> np.ndarray:
    """Normal(mean, std) samples rounded to bf16 bit patterns."""
    return f32_to_bf16_bits((g.standard_normal(shape) * std + mean).astype(np.float32))


# --------------------------------------------------------------------------- QMM
def qmm_weights(config: int, N: int, K: int, bits: int = 4, group_size: int = 64,
                seed: int = 0, layer: int = 0, scale_mean: float = 0.02, scale_std: float = 0.005,
                bias_std: float = 0.01):
    """Quantized weight pack of one linear layer W[N, K].

    * codes: uniform integers in [0, 2**bits); drawn as uniform random 32-bit
      words, which makes every 4-bit or 8-bit field uniform. Stored as
      ``uint32[N, K * bits // 32]`` (the packing convention is documented in
      include/vq.h).
    * scales ~ N(0.02, 0.005), biases ~ N(0, 0.01), bf16, ``[N, K // group_size]``
      (the distribution of the dense-layer configurations; other means and
      spreads give stacks whose activations stay O(1)).
    """
    assert K % group_size == 0 and (K * bits) % 32 == 0
    words = rng(config, "W", seed, layer).integers(0, 2**32, size=(N, K * bits // 32),
                                                   dtype=np.uint64).astype(np.uint32)
    G = K // group_size
    scales = bf16_normal(rng(config, "S", seed, layer), (N, G), scale_mean, scale_std)
    biases = bf16_normal(rng(config, "B", seed, layer), (N, G), 0.0, bias_std)
    return {"wq": words, "scales": scales, "biases": biases,
            "bits": bits, "group_size": group_size, "N": N, "K": K}


def qmm_activations(config: int, M: int, K: int, seed: int = 0, extra: int = 0) -> np.ndarray:
    """bf16 activation rows X[M, K] ~ N(0, 1)."""
    return bf16_normal(rng(config, "X", seed, extra), (M, K))


# --------------------------------------------------------------------- attention
def attn_inputs(config: int, M: int, Hq: int, Hkv: int, D: int, T_cap: int,
                seed: int = 0, extra: int = 0):
    """Query rows q[M, Hq, D] and a KV cache k, v [Hkv, T_cap, D], all bf16 ~ N(0, 1)."""
    q = bf16_normal(rng(config, "Q", seed, extra), (M, Hq, D))
    k = bf16_normal(rng(config, "K", seed, extra), (Hkv, T_cap, D))
    v = bf16_normal(rng(config, "V", seed, extra), (Hkv, T_cap, D))
    return q, k, v


def tree_masks(config: int, M: int, seed: int = 0, extra: int = 0) -> np.ndarray:
    """Ancestor masks of a random draft tree of M nodes in topological order:
    node 0 is the root, node i > 0 hangs under a uniformly drawn earlier node, and
    mask[i] has bit t set for every node t on the path from the root to i
    (i included). uint32 [M]."""
    g = rng(config, "tree", seed, extra)
    mask = np.zeros(M, dtype=np.uint32)
    for i in range(M):
        parent = int(g.integers(0, i)) if i > 0 else -1
        mask[i] = (int(mask[parent]) if parent >= 0 else 0) | (1 << i)
    return mask


def chain_masks(M: int) -> np.ndarray:
    """The masks of a chain (node i under node i - 1): bits 0..i."""
    return np.array([(1 << (i + 1)) - 1 for i in range(M)], dtype=np.uint32)


# -------------------------------------------------------------------- acceptance
def accept_logits(config: int, K: int, V: int, std: float = 2.0, seed: int = 0, extra: int = 0):
    """Target logits [K+1, V] and draft logits [K, V], float32 ~ N(0, std)."""
    pl = (rng(config, "plogit", seed, extra).standard_normal((K + 1, V)) * std).astype(np.float32)
    ql = (rng(config, "qlogit", seed, extra).standard_normal((K, V)) * std).astype(np.float32)
    return pl, ql


def accept_logits_correlated(config: int, K: int, V: int, std: float = 2.0, noise: float = 0.5,
                             seed: int = 0, extra: int = 0):
    """Target logits [K+1, V] ~ N(0, std) and draft logits [K, V] equal to the target
    rows plus N(0, noise): a draft that agrees with the target most of the time, so
    that long accepted prefixes and the bonus draw are exercised."""
    pl = (rng(config, "plogit", seed, extra).standard_normal((K + 1, V)) * std).astype(np.float32)
    ql = (pl[:K].astype(np.float64)
          + rng(config, "qlogit", seed, extra).standard_normal((K, V)) * noise).astype(np.float32)
    return pl, ql


def uniforms24(config: int, shape, stream: str = "accept-u", seed: int = 0, extra: int = 0) -> np.ndarray:
    """float32 uniforms k * 2**-24 with k uniform in [0, 2**24) (exact in float32)."""
    k = rng(config, stream, seed, extra).integers(0, 2**U_BITS, size=shape, dtype=np.int64)
    return (k.astype(np.float64) * 2.0**-U_BITS).astype(np.float32)


def random_words_torch(n_words: int, seed: int, device):
    """Bulk uniform 32-bit words generated on a torch device (for multi-GB weight
    stacks that only the benchmark uses; parity tests draw from numpy above)."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    return torch.randint(-(2**31), 2**31, (n_words,), dtype=torch.int32,
                         device=device, generator=gen)


def bf16_normal_torch(shape, mean: float, std: float, seed: int, device):
    """Normal(mean, std) bf16 tensor generated on a torch device (benchmark stacks)."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    t = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    return (t * std + mean).to(torch.bfloat16)
