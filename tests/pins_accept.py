"""Pins for the acceptance oracle (module passed in, for mutation tests)."""
from __future__ import annotations

import json
import os
from fractions import Fraction
from itertools import product

import numpy as np
from scipy import stats

from synth import accept_logits, accept_logits_correlated, uniforms24

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
F32 = np.float32


def _golden():
    with open(os.path.join(GOLDEN, "accept_hand.json")) as f:
        return json.load(f)


def pin_truncation_golden(mod):
    for c in _golden()["truncation"]:
        p = np.array(c["p"], dtype=F32)
        kept, Z = mod.truncate(p, c["top_k"], c["top_p"])
        assert sorted(int(t) for t in np.nonzero(kept)[0]) == c["kept"], c
        for t in c["kept"]:  # kept masses are floor(p * 2**40), exactly
            assert int(kept[t]) == int(Fraction(float(p[t])) * 2**40), c
        assert Z == sum(int(kept[t]) for t in c["kept"])


def pin_accept_golden(mod):
    for c in _golden()["accept"]:
        P = np.array(c["P"], dtype=F32)
        Q = np.array(c["Q"], dtype=F32).reshape(len(c["drafts"]), P.shape[1])
        toks, n = mod.spec_accept(P, Q, c["drafts"], np.array(c["uniforms"], dtype=F32), c["top_k"], c["top_p"])
        assert (toks, n) == (c["tokens"], c["n_accepted"]), (c["why"], toks, n)


# Dyadic fixtures: every decision threshold and every CDF edge of the 24-bit
# uniforms lands on a multiple of 2**22, so the rule is constant on each of the
# four cells [c/4, (c+1)/4) of every uniform and exact enumeration is finite.
DYADIC = [
    dict(P=[[1/2, 1/4, 1/8, 1/8], [1/4, 1/4, 1/4, 1/4]], Q=[[1/4, 1/2, 1/8, 1/8]]),
    dict(P=[[1/2, 1/4, 1/4], [0, 1/2, 1/2], [1/4, 1/4, 1/2]], Q=[[1/4, 1/4, 1/2], [1/2, 1/4, 1/4]]),
]


def pin_dyadic_exact(mod):
    """Closed form: the emitted token at position i, given that every earlier draft
    was accepted, is distributed exactly as p~_i (and the first one as p~_0)."""
    for fx in DYADIC:
        P = np.array(fx["P"], dtype=F32)
        Q = np.array(fx["Q"], dtype=F32)
        K, V = Q.shape
        reach = [Fraction(0)] * (K + 1)
        emit = [[Fraction(0)] * V for _ in range(K + 1)]
        cells = [Fraction(c, 4) for c in range(4)]
        for drafts in product(range(V), repeat=K):
            pd = Fraction(1)
            for i, d in enumerate(drafts):
                pd *= Fraction(float(Q[i, d]))
            if pd == 0:
                continue
            for us in product(cells, repeat=K + 1):
                w = pd / 4 ** (K + 1)
                toks, n = mod.spec_accept(P, Q, list(drafts), np.array([float(u) for u in us], dtype=F32))
                assert n >= 0
                for i in range(n + 1):
                    reach[i] += w
                    emit[i][toks[i]] += w
        for i in range(K + 1):
            for x in range(V):
                assert emit[i][x] == reach[i] * Fraction(float(P[i, x])), (fx, i, x)
        assert reach[1] == sum(min(Fraction(float(P[0, x])), Fraction(float(Q[0, x]))) for x in range(V))


def _rows(seed, K, V, T=1.0):
    import oracle.accept as real  # input rows only: probabilities rounded to float32
    pl, ql = accept_logits(300 + seed, K, V)
    return real.probs_f32(pl, T), real.probs_f32(ql, T)


def pin_special_cases(mod):
    rng = np.random.default_rng(11)
    K, V = 3, 40
    P, Q = _rows(1, K, V)
    # p = q: every draft from q~ is accepted and the bonus comes from p~_K.
    for tk, tp in ((0, 1.0), (8, 0.9)):
        for _ in range(20):
            us = uniforms24(400, (2 * K + 1,), extra=int(rng.integers(1 << 30)))
            drafts = [mod.sample_truncated(P[i], tk, tp, us[K + 1 + i]) for i in range(K)]
            toks, n = mod.spec_accept(P, P[:K], drafts, us[: K + 1], tk, tp)
            assert n == K and toks[:K] == drafts
            assert toks[K] == mod.sample_truncated(P[K], tk, tp, us[K])
    # disjoint supports: reject at 0 and draw from p~_0.
    Pd = P.copy(); Pd[:, 1::2] = 0
    Qd = Q.copy(); Qd[:, 0::2] = 0
    for _ in range(20):
        us = uniforms24(401, (K + 2,), extra=int(rng.integers(1 << 30)))
        drafts = [mod.sample_truncated(Qd[i], 0, 1.0, us[K + 1]) for i in range(K)]
        toks, n = mod.spec_accept(Pd, Qd, drafts, us[: K + 1])
        assert n == 0 and toks[0] == mod.sample_truncated(Pd[0], 0, 1.0, us[K]) and toks[0] % 2 == 0
    # top_k = 1 on both sides: greedy verification (longest argmax-matching prefix + one token).
    am = lambda row: int(np.lexsort((np.arange(V), -row.astype(np.float64)))[0])
    for _ in range(30):
        drafts = [am(P[i]) if rng.random() < 0.6 else int(rng.integers(V)) for i in range(K)]
        us = uniforms24(402, (K + 1,), extra=int(rng.integers(1 << 30)))
        toks, n = mod.spec_accept(P, Q, drafts, us, 1, 1.0)
        j = next((i for i in range(K) if drafts[i] != am(P[i])), K)
        assert n == j and toks[: j + 1] == drafts[:j] + [am(P[j])]
    # top_p = 1, top_k = 0: identity truncation.
    kept, Z = mod.truncate(P[0], 0, 1.0)
    m = np.array([int(Fraction(float(v)) * 2**40) for v in P[0]], dtype=np.int64)
    assert np.array_equal(kept, m) and Z == int(m.sum())
    # extreme uniforms of the final draw (K = 0): first / last token of positive mass.
    Pz = P[:1].copy(); Pz[0, :3] = 0; Pz[0, -2:] = 0
    assert mod.spec_accept(Pz, np.zeros((0, V), F32), [], np.array([0.0], F32))[0] == [3]
    assert mod.spec_accept(Pz, np.zeros((0, V), F32), [], np.array([1 - 2**-24], F32))[0] == [V - 3]
    # the smallest representable mass (2**-40) at the front is still drawn at u = 0.
    Pt = np.array([[2.0**-40, 0.25, 0.75]], F32)
    assert mod.spec_accept(Pt, np.zeros((0, 3), F32), [], np.array([0.0], F32))[0] == [0]
    assert mod.spec_accept(Pt, np.zeros((0, 3), F32), [], np.array([2.0**-24], F32))[0] == [1]
    # invalid entries.
    bad = ([-1] * (K + 1), -1)
    us = np.full(K + 1, 0.5, F32)
    d = [0, 1, 2]
    Pn = P.copy(); Pn[2, 5] = np.nan
    assert mod.spec_accept(Pn, Q, d, us) == bad
    Pn = P.copy(); Pn[0, 5] = -1e-9
    assert mod.spec_accept(Pn, Q, d, us) == bad
    Qn = Q.copy(); Qn[1, 0] = 1.5
    assert mod.spec_accept(P, Qn, d, us) == bad
    assert mod.spec_accept(P, Q, [0, V, 1], us) == bad
    assert mod.spec_accept(P, Q, d, np.array([0.5, 1.0, 0.5, 0.5], F32)) == bad
    Pn = P.copy(); Pn[3] = 0
    assert mod.spec_accept(Pn, Q, d, us) == bad


def pin_shared_rows_match(mod):
    """The vectorised shared-rows path equals the per-trial rule."""
    rng = np.random.default_rng(12)
    for tk, tp, T in ((0, 1.0, 1.0), (10, 0.9, 0.7), (3, 0.5, 1.0)):
        K, V = 3, 60
        P, Q = _rows(2, K, V, T)
        sr = mod.SharedRows(P, Q, tk, tp)
        B = 300
        us = uniforms24(403, (B, 2 * K + 1), extra=tk)
        drafts = np.array([[mod.sample_truncated(Q[i], tk, tp, us[b, K + 1 + i]) if b % 3 else int(rng.integers(V))
                            for i in range(K)] for b in range(B)])
        toks, n = sr.run(drafts, us[:, : K + 1])
        for b in range(B):
            t1, n1 = mod.spec_accept(P, Q, list(drafts[b]), us[b, : K + 1], tk, tp)
            assert (list(toks[b]), int(n[b])) == (t1, n1), (tk, tp, b)


PINS = [pin_truncation_golden, pin_accept_golden, pin_dyadic_exact, pin_special_cases, pin_shared_rows_match]


# ------------------------------------------------------------ distribution check
def make_trials(mod, config, K, V, T, top_k, top_p, n_trials, seed=0, corr=None):
    """Shared rows (oracle float32 probabilities of synthetic logits), drafts drawn
    from q~ per position, and the acceptance uniforms of ``n_trials`` verifies."""
    if corr is None:
        pl, ql = accept_logits(config, K, V, seed=seed)
    else:
        pl, ql = accept_logits_correlated(config, K, V, noise=corr, seed=seed)
    P, Q = mod.probs_f32(pl, T), mod.probs_f32(ql, T)
    sr = mod.SharedRows(P, Q, top_k, top_p)
    assert sr.valid
    u_d = uniforms24(config, (n_trials, K), stream="draft-u", seed=seed)
    u_a = uniforms24(config, (n_trials, K + 1), stream="accept-u", seed=seed)
    mu_d = np.floor(u_d.astype(np.float64) * 2**24).astype(np.int64)
    drafts = np.empty((n_trials, K), dtype=np.int64)
    for i in range(K):
        kept, Z = sr.rowsQ[i]
        drafts[:, i] = np.searchsorted(mod.cdf_edges(kept, Z), mu_d[:, i], side="right")
    return dict(P=P, Q=Q, logits=(pl, ql), sr=sr, drafts=drafts, uniforms=u_a)


def check_distribution(sr, toks, n, K, V, alpha=1e-3, min_reach=2000):
    """Chi-square of the emitted tokens against p~ per position (positions reached by
    at least ``min_reach`` trials) and the position-0 acceptance rate against
    sum_x min(p~_0, q~_0) within 4 sigma. Returns the p-values by position."""
    toks = np.asarray(toks, dtype=np.int64)
    n = np.asarray(n, dtype=np.int64)
    n_trials = n.size
    assert np.all(n >= 0)
    pvals = {}
    for i in range(K + 1):
        sel = n >= i
        if sel.sum() < min_reach:
            continue
        obs = np.bincount(toks[sel, i], minlength=V).astype(np.float64)
        kept, Z = sr.rowsP[i]
        exp = kept.astype(np.float64) / Z * sel.sum()
        assert obs[exp == 0].sum() == 0, "token emitted outside the truncated support"
        order = np.argsort(exp)
        small = exp[order] < 5
        o = np.concatenate([obs[order][~small], [obs[order][small].sum()]])
        e = np.concatenate([exp[order][~small], [exp[order][small].sum()]])
        keep = e > 0
        o, e = o[keep], e[keep]
        e *= o.sum() / e.sum()
        pvals[i] = float(stats.chisquare(o, e).pvalue)
    if K > 0:
        kP, ZP = sr.rowsP[0]
        kQ, ZQ = sr.rowsQ[0]
        rate = sum(min(Fraction(int(a), ZP), Fraction(int(b), ZQ)) for a, b in zip(kP, kQ) if a and b)
        obs_rate = float((n >= 1).mean())
        sigma = np.sqrt(float(rate) * (1 - float(rate)) / n_trials)
        assert abs(obs_rate - float(rate)) <= 4 * sigma + 1e-12, (obs_rate, float(rate))
    assert 0 in pvals and all(pv > alpha for pv in pvals.values()), pvals
    return pvals


def chisquare_trials(mod, config, K, V, T, top_k, top_p, n_trials, seed=0, alpha=1e-3,
                     corr=None, min_reach=2000):
    """10**6-trial distribution check of the oracle itself (see ``check_distribution``)."""
    tr = make_trials(mod, config, K, V, T, top_k, top_p, n_trials, seed, corr)
    toks, n = tr["sr"].run(tr["drafts"], tr["uniforms"])
    return check_distribution(tr["sr"], toks, n, K, V, alpha, min_reach), None, None
