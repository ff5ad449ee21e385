"""Pins for the QMM oracle: checks against things other than the oracle itself.

Each pin takes the oracle module as an argument so that the mutation tests can
run the same pins against deliberately broken copies of the oracle.
"""
from __future__ import annotations

import json
import os
import struct

import numpy as np

from synth import qmm_activations, qmm_weights

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bf16_scalar(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def _code_bruteforce(words, bits: int, K: int, n: int, k: int) -> int:
    """Code q[n, k] read from the hex text of the packed words (an independent route)."""
    per_row = K * bits // 32
    if bits == 4:
        w = int(words[n * per_row + k // 8])
        hexs = f"{w:08x}"          # most significant nibble first
        return int(hexs[7 - (k % 8)], 16)
    w = int(words[n * per_row + k // 4])
    hexs = f"{w:08x}"
    byte = k % 4
    return int(hexs[6 - 2 * byte: 8 - 2 * byte], 16)


def qmm_bruteforce(x, wq, scales, biases, bits, gs, M, N, K):
    """Triple loop in Python floats (float64)."""
    words = np.asarray(wq).reshape(-1)
    s = np.asarray(scales).reshape(N, K // gs)
    b = np.asarray(biases).reshape(N, K // gs)
    X = np.asarray(x).reshape(M, K)
    y = [[0.0] * N for _ in range(M)]
    for n in range(N):
        w = [_bf16_scalar(s[n, k // gs]) * _code_bruteforce(words, bits, K, n, k) + _bf16_scalar(b[n, k // gs])
             for k in range(K)]
        for m in range(M):
            acc = 0.0
            for k in range(K):
                acc += _bf16_scalar(X[m, k]) * w[k]
            y[m][n] = acc
    return np.array(y)


def _case(seed, bits, M=3, N=5, K=192, gs=64):
    w = qmm_weights(100 + seed, N, K, bits, gs)
    x = qmm_activations(100 + seed, M, K)
    return x, w


def pin_golden(mod):
    with open(os.path.join(GOLDEN, "qmm_hand.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        words = np.array([int(v, 16) for v in c["words"]], dtype=np.uint32)
        sc = np.array([int(v, 16) for v in c["scales_bf16"]], dtype=np.uint16)
        bi = np.array([int(v, 16) for v in c["biases_bf16"]], dtype=np.uint16)
        x = np.array([[int(v, 16) for v in row] for row in c["x_bf16"]], dtype=np.uint16)
        y = mod.skinny_qmm(x, words, sc, bi, c["bits"], c["group_size"], c["M"], c["N"], c["K"])
        assert np.array_equal(y, np.array(c["expected_y"])), (c["name"], y)


def pin_bruteforce(mod):
    for seed, bits in ((0, 4), (1, 8), (2, 4)):
        x, w = _case(seed, bits)
        M, N, K = x.shape[0], w["N"], w["K"]
        ref = qmm_bruteforce(x, w["wq"], w["scales"], w["biases"], bits, 64, M, N, K)
        got = mod.skinny_qmm(x, w["wq"], w["scales"], w["biases"], bits, 64, M, N, K)
        assert np.allclose(got, ref, rtol=0, atol=1e-12 * max(1.0, np.abs(ref).max())), (bits, got, ref)


def pin_factorized(mod):
    """y = sum_g s_g * sum_{k in g} q*x + b_g * sum_{k in g} x (closed-form regrouping)."""
    for seed, bits in ((3, 4), (4, 8)):
        x, w = _case(seed, bits, M=2, N=4, K=256)
        M, N, K, gs = 2, 4, 256, 64
        words = w["wq"].reshape(-1)
        y = np.zeros((M, N))
        for n in range(N):
            for g in range(K // gs):
                s = _bf16_scalar(w["scales"][n, g])
                b = _bf16_scalar(w["biases"][n, g])
                for m in range(M):
                    qx = sum(_code_bruteforce(words, bits, K, n, k) * _bf16_scalar(x[m, k])
                             for k in range(g * gs, (g + 1) * gs))
                    sx = sum(_bf16_scalar(x[m, k]) for k in range(g * gs, (g + 1) * gs))
                    y[m, n] += s * qx + b * sx
        got = mod.skinny_qmm(x, w["wq"], w["scales"], w["biases"], bits, gs, M, N, K)
        assert np.allclose(got, y, rtol=0, atol=1e-10 * max(1.0, np.abs(y).max()))


def pin_integer_exact(mod):
    """s = 1, b = 0 and small integer activations: an exact integer matmul."""
    rng = np.random.default_rng(5)
    for bits in (4, 8):
        M, N, K, gs = 3, 6, 128, 64
        words = rng.integers(0, 2**32, size=(N, K * bits // 32), dtype=np.uint64).astype(np.uint32)
        ones = np.full((N, K // gs), 0x3F80, dtype=np.uint16)
        zeros = np.zeros((N, K // gs), dtype=np.uint16)
        xi = rng.integers(-8, 9, size=(M, K))
        xb = np.array([[struct.unpack("<I", struct.pack("<f", float(v)))[0] >> 16 for v in row] for row in xi],
                      dtype=np.uint16)
        q = [[_code_bruteforce(words.reshape(-1), bits, K, n, k) for k in range(K)] for n in range(N)]
        ref = [[sum(int(xi[m, k]) * q[n][k] for k in range(K)) for n in range(N)] for m in range(M)]
        got = mod.skinny_qmm(xb, words, ones, zeros, bits, gs, M, N, K)
        assert np.array_equal(got, np.array(ref, dtype=np.float64)), bits


def pin_zero_codes(mod):
    """q = 0 everywhere: y = sum_g b_g * sum_{k in g} x."""
    x, w = _case(6, 4, M=2, N=3, K=192)
    M, N, K, gs = 2, 3, 192, 64
    words = np.zeros_like(w["wq"])
    got = mod.skinny_qmm(x, words, w["scales"], w["biases"], 4, gs, M, N, K)
    ref = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            for g in range(K // gs):
                ref[m, n] += _bf16_scalar(w["biases"][n, g]) * sum(_bf16_scalar(x[m, k]) for k in range(g * gs, (g + 1) * gs))
    assert np.allclose(got, ref, rtol=0, atol=1e-12 * max(1.0, np.abs(ref).max()))


def pin_row_independence(mod):
    x, w = _case(7, 4, M=5, N=7, K=128)
    M, N, K = 5, 7, 128
    full = mod.skinny_qmm(x, w["wq"], w["scales"], w["biases"], 4, 64, M, N, K)
    for m in range(M):
        one = mod.skinny_qmm(x[m:m + 1], w["wq"], w["scales"], w["biases"], 4, 64, 1, N, K)
        assert np.array_equal(full[m], one[0])


PINS = [pin_golden, pin_bruteforce, pin_factorized, pin_integer_exact, pin_zero_codes, pin_row_independence]
