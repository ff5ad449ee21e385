"""The acceptance oracle against its pins, the distribution identity over 10**6
trials, and the pins against planted mistakes."""
import pytest

import oracle.accept as oacc
from tests import pins_accept
from tests.mutation import caught, mutant


@pytest.mark.parametrize("pin", pins_accept.PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(oacc)


@pytest.mark.parametrize("name,cfg", [
    ("config0: V=1000 K=3 logits N(0,2), no truncation", dict(config=0, K=3, V=1000, T=1.0, top_k=0, top_p=1.0)),
    ("V=1000 K=3 T=1.0 top-k 20 + top-p 0.95", dict(config=4, K=3, V=1000, T=1.0, top_k=20, top_p=0.95)),
    ("config3: V=248320 K=3 T=0.7 top-p 0.95", dict(config=3, K=3, V=248320, T=0.7, top_k=0, top_p=0.95)),
    ("config4: V=248320 K=7 T=1.0 top-k 20 + top-p 0.95", dict(config=4, K=7, V=248320, T=1.0, top_k=20, top_p=0.95)),
    ("correlated drafts V=1000 K=3", dict(config=0, K=3, V=1000, T=1.0, top_k=0, top_p=1.0, corr=0.5)),
    ("correlated drafts config3 V=248320 K=3 T=0.7 top-p 0.95", dict(config=3, K=3, V=248320, T=0.7, top_k=0, top_p=0.95, corr=0.3)),
    ("correlated drafts config4 V=248320 K=7 T=1.0 top-k 20 + top-p 0.95", dict(config=4, K=7, V=248320, T=1.0, top_k=20, top_p=0.95, corr=0.3)),
])
def test_distribution_1e6_trials(name, cfg):
    pvals, _, _ = pins_accept.chisquare_trials(oacc, n_trials=10**6, **cfg)
    if cfg.get("corr") is not None:
        assert cfg["K"] in pvals, f"bonus position not reached often enough: {pvals}"


MUTANTS = [
    ("p and q swapped in the accept test", "if not (mus[i] * int(mQ[d]) * ZP < int(mP[d]) * ZQ * 2**U_BITS):",
     "if not (mus[i] * int(mP[d]) * ZQ < int(mQ[d]) * ZP * 2**U_BITS):"),
    ("crossing token dropped by top-p", "if before * 2**TOPP_BITS < thr:", "if (before + mt) * 2**TOPP_BITS < thr:"),
    ("ties to the higher id", "order = np.lexsort((np.arange(V), -p32.astype(np.float64)))",
     "order = np.lexsort((-np.arange(V), -p32.astype(np.float64)))"),
    ("residual (q - p)+", "r = [max(0, int(a) * ZQ - int(b) * ZP) for a, b in zip(mP, mQ)]\n        R = sum(r)\n        if R == 0:\n            r, R = [int(a) for a in mP], ZP\n    else:",
     "r = [max(0, int(b) * ZP - int(a) * ZQ) for a, b in zip(mP, mQ)]\n        R = sum(r)\n        if R == 0:\n            r, R = [int(a) for a in mP], ZP\n    else:"),
    ("inverse CDF off by one", "return bisect_right(list(accumulate(int(v) for v in r)), tau)",
     "return bisect_right(list(accumulate(int(v) for v in r)), tau + 1)"),
    ("bonus drawn from the first row", "    else:\n        r, R = [int(a) for a in mP], ZP\n    t = inverse_cdf",
     "    else:\n        r, R = [int(a) for a in rowsP[0][0]], rowsP[0][1]\n    t = inverse_cdf"),
    ("top-k after top-p", "n_top = V if (top_k <= 0 or top_k >= V) else int(top_k)      # step 3",
     "n_top = V      # step 3"),
    ("accept test not strict", "if not (mus[i] * int(mQ[d]) * ZP < int(mP[d]) * ZQ * 2**U_BITS):",
     "if not (mus[i] * int(mQ[d]) * ZP <= int(mP[d]) * ZQ * 2**U_BITS):"),
    ("drafts emitted after the rejection too", "tokens = [int(d) for d in drafts[:j]] + [t] + [INVALID] * (K - j)",
     "tokens = [int(d) for d in drafts[:j]] + [t] + [int(d) for d in drafts[j + 1:]]"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(name, old, new):
    assert caught(pins_accept.PINS, mutant("accept", old, new)), name
