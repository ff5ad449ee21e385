"""The 8-bit KV oracle against its pins, and the pins against planted mistakes."""
import pytest

import oracle.kv8 as okv
from tests import pins_kv8
from tests.mutation import caught, mutant


@pytest.mark.parametrize("pin", pins_kv8.PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(okv)


MUTANTS = [
    ("step over 256 levels", "(mx - mn) / np.float32(255.0)", "(mx - mn) / np.float32(256.0)"),
    ("bias from the maximum", "_bf16_rne(mn)], axis=-1)", "_bf16_rne(mx)], axis=-1)"),
    ("codes truncated", "q = np.rint(", "q = np.floor("),
    ("scale truncated to bf16", "sb = np.stack([_bf16_rne(scale32),",
     "sb = np.stack([(scale32.view(np.uint32) >> 16).astype(np.uint16),"),
    ("groups of 32", "q = codes.astype(np.float64).reshape(codes.shape[:-1] + (D // GROUP, GROUP))",
     "q = codes.astype(np.float64).reshape(codes.shape[:-1] + (D // 32, 32))[..., ::2, :].repeat(2, -2)"),
    ("scale and bias swapped", "s = bf16_to_f64(sb[..., 0])\n    b = bf16_to_f64(sb[..., 1])",
     "s = bf16_to_f64(sb[..., 1])\n    b = bf16_to_f64(sb[..., 0])"),
    ("signed codes", "q = codes.astype(np.float64)", "q = codes.astype(np.int8).astype(np.float64)"),
    ("values read from the key cache", "Vf = dequantize(np.asarray(v_codes)[:, :T], np.asarray(v_sb)[:, :T])",
     "Vf = dequantize(np.asarray(k_codes)[:, :T], np.asarray(k_sb)[:, :T])"),
    ("one key too many", "idx = visible_keys(M, T, msk, m)", "idx = visible_keys(M, T, msk << np.uint64(1) | msk, m)"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(name, old, new):
    assert caught(pins_kv8.PINS, mutant("kv8", old, new)), name
