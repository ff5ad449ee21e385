"""GPU parity of vq_skinny_qmm against the float64 oracle."""
import numpy as np
import pytest
import torch

import oracle.qmm as oq
from synth import qmm_activations, qmm_weights
from tests.gpu_util import assert_close, bf16_tensor, dev, to_f64, words_tensor

pytestmark = pytest.mark.gpu


def _run(vq, w, x_bits, out_dtype=torch.bfloat16, ldx_pad=0):
    M, K = x_bits.shape
    x = bf16_tensor(x_bits)
    if ldx_pad:
        wide = torch.zeros((M, K + ldx_pad), dtype=torch.bfloat16, device=dev())
        wide[:, :K] = x
        x = wide[:, :K]
    y = vq.skinny_qmm(x, words_tensor(w["wq"]), bf16_tensor(w["scales"]), bf16_tensor(w["biases"]), w["bits"],
                      w["N"], w["K"], out_dtype=out_dtype)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("M", list(range(1, 17)))
def test_config0_all_rows(vq, bits, M):
    """Config 0: W 512x1024, group 64, M = 1..16 (covers both row paddings)."""
    w = qmm_weights(0, 512, 1024, bits)
    x = qmm_activations(0, M, 1024)
    ref = oq.skinny_qmm(x, w["wq"], w["scales"], w["biases"], bits, 64, M, 512, 1024)
    assert_close(to_f64(_run(vq, w, x)), ref, f"bits={bits} M={M}")


@pytest.mark.parametrize("bits,M,N,K", [
    (4, 3, 200, 64 * 3),        # ragged N, three groups
    (4, 5, 33, 64 * 17),        # one column over a tile; a chunk boundary inside K
    (8, 7, 130, 64 * 21),
    (4, 16, 256, 8192),         # many K splits -> cross-workgroup reduction
    (8, 9, 96, 8192),
    (4, 1, 4000, 64),           # single group
    (8, 12, 1000, 1088),
    # plan rules for long K: narrow outputs take full 16-group ranges (ragged last
    # range), wider ones at least three blocks per range
    (4, 4, 300, 64 * 97),
    (8, 8, 5120, 64 * 75),
    (4, 4, 8256, 64 * 70),
])
def test_ragged_and_split_shapes(vq, bits, M, N, K):
    w = qmm_weights(11, N, K, bits, layer=N)
    x = qmm_activations(11, M, K, extra=K)
    ref = oq.skinny_qmm(x, w["wq"], w["scales"], w["biases"], bits, 64, M, N, K)
    assert_close(to_f64(_run(vq, w, x)), ref, f"{bits}-bit M={M} N={N} K={K}")
    assert_close(to_f64(_run(vq, w, x, out_dtype=torch.float32, ldx_pad=24)), ref, "f32 out, padded ldx")


def test_deterministic(vq):
    w = qmm_weights(12, 512, 8192, 4)
    x = qmm_activations(12, 8, 8192)
    a = _run(vq, w, x, out_dtype=torch.float32)
    for _ in range(3):
        b = _run(vq, w, x, out_dtype=torch.float32)
        assert torch.equal(a, b)


PROJ = {"q": (6144, 5120), "k": (1024, 5120), "o": (5120, 6144), "gate": (17408, 5120),
        "down": (5120, 17408), "qkv": (8192, 5120), "gate_up": (34816, 5120)}


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("name", list(PROJ))
def test_config1_projection_sampled(vq, bits, name):
    """Config 1 shapes at every M of the sweep; 64 sampled output columns each."""
    N, K = PROJ[name]
    w = qmm_weights(1, N, K, bits, layer=list(PROJ).index(name))
    cols = np.random.default_rng(N + K).choice(N, size=64, replace=False)
    cols = np.concatenate([cols, [0, N - 1]])
    for M in (1, 2, 3, 4, 6, 8, 12, 16):
        x = qmm_activations(1, M, K, extra=M)
        ref = oq.skinny_qmm(x, w["wq"], w["scales"], w["biases"], bits, 64, M, N, K, cols=cols)
        y = to_f64(_run(vq, w, x))
        assert_close(y[:, cols], ref, f"{name} {bits}-bit M={M}")


def test_lm_head_sampled_f32(vq):
    N, K = 248320, 5120
    w = qmm_weights(3, N, K, 4, layer=999)
    cols = np.concatenate([np.random.default_rng(5).choice(N, 48, replace=False), [0, N - 1]])
    x = qmm_activations(3, 4, K)
    ref = oq.skinny_qmm(x, w["wq"], w["scales"], w["biases"], 4, 64, 4, N, K, cols=cols)
    y = to_f64(_run(vq, w, x, out_dtype=torch.float32))
    assert_close(y[:, cols], ref, "lm_head")
