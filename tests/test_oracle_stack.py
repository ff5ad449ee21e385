"""The verify-step composition oracle against its pins, and the pins against
planted mistakes."""
import pytest

import oracle.stack as ostack
from tests import pins_stack
from tests.mutation import caught, mutant


@pytest.mark.parametrize("pin", pins_stack.PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(ostack)


# Dropping the rounding of a value that only feeds a projection (the RMSNorm
# outputs, the SwiGLU output, the attention output) is not a mistake this oracle
# can make: its projections take their inputs as bf16 bit patterns, so those
# roundings happen either way. The roundings that do change results -- the
# residual adds, the projection outputs, the bf16 rounding itself -- are below.
MUTANTS = [
    ("eps outside the square root", "np.sqrt(np.mean(h * h, axis=-1, keepdims=True) + eps)",
     "(np.sqrt(np.mean(h * h, axis=-1, keepdims=True)) + eps)"),
    ("norm over the wrong axis", "np.mean(h * h, axis=-1, keepdims=True)", "np.mean(h * h, axis=0, keepdims=True)"),
    ("gate and up swapped", "silu_mul(gu[:, :inter], gu[:, inter:])", "silu_mul(gu[:, inter:], gu[:, :inter])"),
    ("attention residual not rounded", 'h = round_bf16(h + qmm_bf16(ctx_in, w["o"]))',
     'h = h + qmm_bf16(ctx_in, w["o"])'),
    ("MLP residual not rounded", 'h = round_bf16(h + qmm_bf16(act, w["down"]))', 'h = h + qmm_bf16(act, w["down"])'),
    ("attention on the first layer of every four", "return layer % every == every - 1", "return layer % every == 0"),
    ("new rows appended one position late", 'kv["k"][:, ctx: ctx + M, :] = k_new', 'kv["k"][:, ctx + 1: ctx + M + 1, :] = k_new'),
    ("keys and values swapped", 'v_new = qkv[:, (Hq + Hkv) * D:]', 'v_new = qkv[:, Hq * D: (Hq + Hkv) * D]'),
    ("silu with the wrong sign", "np.exp(-gate)", "np.exp(gate)"),
    ("ties rounded away from zero", "np.rint(x / step)", "np.trunc(x / step + np.copysign(0.5, x))"),
    ("one significant bit too few", "np.maximum(e - 8, -133)", "np.maximum(e - 7, -133)"),
    ("projection outputs not rounded", "    return round_bf16(y)\n", "    return y\n"),
    ("lm_head without the final norm", "a = round_bf16(rmsnorm(h))\n    M, K", "a = round_bf16(h)\n    M, K"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(name, old, new):
    assert caught(pins_stack.PINS, mutant("stack", old, new)), name
