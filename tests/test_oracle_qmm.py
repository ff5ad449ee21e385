"""The QMM oracle against its pins, and the pins against planted mistakes."""
import pytest

import oracle.qmm as oq
from tests import pins_qmm
from tests.mutation import caught, mutant


@pytest.mark.parametrize("pin", pins_qmm.PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(oq)


MUTANTS = [
    ("high nibble first", "q[:, j::8] = (words >> np.uint32(4 * j))", "q[:, j::8] = (words >> np.uint32(4 * (7 - j)))"),
    ("groups along the wrong index", "g = np.arange(K) // group_size", "g = np.arange(K) % (K // group_size)"),
    ("dropped bias", "return s[:, g] * q + b[:, g]", "return s[:, g] * q"),
    ("scale and bias swapped", "s = bf16_to_f64(scales).reshape(N, G)", "s = bf16_to_f64(biases).reshape(N, G)"),
    ("sign of bias", "return s[:, g] * q + b[:, g]", "return s[:, g] * q - b[:, g]"),
    ("8-bit byte order", "return words.view(np.uint8).reshape(N, K).astype(np.int64)",
     "return words.byteswap().view(np.uint8).reshape(N, K).astype(np.int64)"),
    ("bf16 widened from the wrong half", "b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16",
     "b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 15"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(name, old, new):
    assert caught(pins_qmm.PINS, mutant("qmm", old, new)), name
