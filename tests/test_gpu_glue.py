"""GPU parity of the element-wise glue of the unfused verify-step composition
(include/vq_glue.h): RMSNorm and the residual add against the oracle's
definitions. The fused step folds both into the projections; these entry
points stay for callers that compose the step from separate calls."""
import numpy as np
import pytest
import torch

import oracle.stack as ostack
from synth import qmm_activations
from tests.gpu_util import assert_close, bf16_tensor, to_f64

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,N,pad", [(1, 5120, 0), (4, 5120, 64), (16, 17408, 0), (3, 300, 8), (8, 65536, 0)])
def test_rmsnorm_bf16(vq, M, N, pad):
    xb = qmm_activations(40, M, N + pad, extra=N)
    x = bf16_tensor(xb)[:, :N]                       # row stride N + pad
    out = torch.full((M, N + 2 * pad), float("nan"), dtype=torch.bfloat16, device=x.device)
    y = vq.rmsnorm(x, out=out[:, :N], eps=1e-6)
    torch.cuda.synchronize()
    ref = ostack.round_bf16(ostack.rmsnorm(to_f64(x)))
    got = to_f64(y)
    assert_close(got, ref, f"rmsnorm M={M} N={N}")
    # float32 arithmetic then one rounding: within one bf16 step of the oracle
    step = np.ldexp(1.0, np.frexp(np.abs(ref))[1] - 8)
    assert np.all(np.abs(got - ref) <= step), float(np.max(np.abs(got - ref) / step))
    if pad:
        assert torch.isnan(out[:, N:].float()).all(), "wrote past the rows"


@pytest.mark.parametrize("n", [1, 7, 4096, 5120 * 16, 1 << 20])
def test_add_bf16(vq, n):
    a_bits = qmm_activations(41, 1, n, extra=n)[0]
    b_bits = qmm_activations(42, 1, n, extra=n)[0]
    a, b = bf16_tensor(a_bits), bf16_tensor(b_bits)
    ref = ostack.round_bf16(to_f64(a) + to_f64(b))
    y = vq.add_(a.clone(), b)                        # in place: y aliases a
    torch.cuda.synchronize()
    got = to_f64(y)
    # a + b of two bf16 values is exact in float32 unless their exponents are far
    # apart; then one float32 rounding precedes the bf16 one
    exact = np.abs(to_f64(a)) * 2.0 ** -16 < np.abs(to_f64(b))
    exact &= np.abs(to_f64(b)) * 2.0 ** -16 < np.abs(to_f64(a))
    assert np.array_equal(got[exact], ref[exact])
    assert_close(got, ref, f"add n={n}")
