"""The attention oracle against its pins, and the pins against planted mistakes."""
import pytest

import oracle.attn as oa
from tests import pins_attn
from tests.mutation import caught, mutant


@pytest.mark.parametrize("pin", pins_attn.PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(oa)


MUTANTS = [
    ("mask one key too many", "limit = T - M + m  #", "limit = T - M + m + 1  #"),
    ("mask one key too few", "limit = T - M + m  #", "limit = T - M + m - 1  #"),
    ("GQA heads interleaved", "s = scale * (Kc[h // G, : limit + 1, :] @ Q[m, h, :])",
     "s = scale * (Kc[h % Hkv, : limit + 1, :] @ Q[m, h, :])"),
    ("values of the wrong head", "out[m, h] = w @ Vc[h // G]", "out[m, h] = w @ Vc[h % Hkv]"),
    ("scale dropped", "s = scale * (Kc", "s = 1.0 * (Kc"),
    ("top-left causal alignment", "limit = T - M + m  #", "limit = m  #"),
    ("tree: mask bit off by one", "if (bits >> t) & 1]", "if (bits >> (t + 1)) & 1]"),
    ("tree: node does not see itself", "bits = int(mask[m]) | (1 << m)", "bits = int(mask[m])"),
    ("tree: last committed key dropped", "list(range(T - M)) + [T - M + t", "list(range(T - M - 1)) + [T - M + t"),
    ("tree: mask read by column", "bits = int(mask[m]) | (1 << m)",
     "bits = sum(((int(mask[t]) >> m) & 1) << t for t in range(M)) | (1 << m)"),
    ("tree: bits at or above M used", "for t in range(M) if (bits >> t) & 1]",
     "for t in range(M + 1) if (bits >> t) & 1 and T - M + t < T] + ([T - 1] if (bits >> M) & 1 else [])"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(name, old, new):
    assert caught(pins_attn.PINS, mutant("attn", old, new)), name
