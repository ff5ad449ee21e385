"""Oracle: exact Leviathan–Chen acceptance with identical truncation (test infrastructure only).

The method (page "The fastest way to run local LLMs on a Mac", section "Why
exact acceptance matters"; page "Speculative decoding and MTP on Apple
silicon", Facts, the claims on Leviathan–Chen rejection sampling and on
truncating draft and verify distributions identically): a drafted token d is
accepted with probability min(1, p(d)/q(d)), p the target's and q the draft's
probability; at the first rejection a replacement is drawn from the normalised
positive part of p - q; the same top-k / top-p truncation is applied to both
distributions. When every draft is accepted one more token is drawn from the
target row that follows the last draft (the verify pass yields "two to three
tokens" per pass at depth three).

The pages give the rule in words only. The arithmetic below is this
library's reading of it, chosen so that a parallel GPU implementation can
reproduce every decision bit for bit (integer addition is associative, float
addition is not):

  1. (logits input only) p = softmax(logits / temperature) in float32. That
     stage is compared within a tolerance; the stages below take float32
     probabilities as given.
  2. Order each row by (probability descending, token id ascending).
  3. top-k (0 < k < V): keep the first k tokens of that order.
  4. Masses m(x) = floor(p(x) * 2**40) (exact: p has a 24-bit significand);
     Zk = sum of the masses kept by top-k.
  5. top-p: tp = max(1, floor(top_p * 2**24)); walking the order, token t is
     kept iff (mass of the kept tokens before t) * 2**24 < tp * Zk. So the
     token that crosses the threshold is kept and top_p = 1 keeps every token
     of positive mass. Z = sum of kept masses; p~(x) = m(x) / Z if kept else 0.
     Target and draft rows are truncated by the same rule with the same
     parameters, each on its own probabilities.
  6. Accept draft d_i iff mu_i * mQ_i(d) * ZP_i < mP_i(d) * ZQ_i * 2**24 with
     mu_i = floor(u_i * 2**24); this is u_i < p~_i(d) / q~_i(d) on 24-bit
     uniforms. Stop at the first rejection j.
  7. At a rejection j: r(x) = max(0, mP_j(x) * ZQ_j - mQ_j(x) * ZP_j), which is
     (p~_j - q~_j)+ scaled by ZP_j * ZQ_j. If every draft was accepted:
     r = mP_K (the bonus row). If r is identically zero (only possible when
     p~_j == q~_j and the draft lies outside both supports) the token is drawn
     from p~_j.
  8. Inverse CDF in token-id order: R = sum r, tau = floor(mu_K * R / 2**24);
     the token is the smallest t with r(0) + ... + r(t) > tau.
  9. Emit d_0 .. d_{j-1} and the drawn token; n_accepted = j; unused output
     slots are -1.

An entry is invalid (all outputs -1, n_accepted = -1) when any of its rows
holds a NaN, a probability < 0 or > 1, or keeps zero total mass; when a draft id
lies outside [0, V); or when a uniform lies outside [0, 1).

Python integers carry every product exactly; float arithmetic appears only in
step 1 and in the exact conversions of steps 4-6.
"""
from __future__ import annotations

from bisect import bisect_right
from itertools import accumulate

import numpy as np

MASS_BITS = 40
U_BITS = 24
TOPP_BITS = 24
INVALID = -1


# ----------------------------------------------------------------------- step 1
def softmax_f64(logits, temperature: float) -> np.ndarray:
    """float64 softmax(logits / temperature) along the last axis (max-subtracted)."""
    z = np.asarray(logits, dtype=np.float32).astype(np.float64) / np.float64(np.float32(temperature))
    z = z - z.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)


def probs_f32(logits, temperature: float = 1.0) -> np.ndarray:
    """float64 softmax rounded to float32: the probability rows fed to the exact stages."""
    return softmax_f64(logits, temperature).astype(np.float32)


# ------------------------------------------------------------------- steps 2-5
def masses(p32) -> np.ndarray | None:
    """m(x) = floor(p(x) * 2**40) as int64, or None if the row is not a valid probability row."""
    p = np.asarray(p32, dtype=np.float32).astype(np.float64)
    if not np.all((p >= 0.0) & (p <= 1.0)):  # NaN fails both comparisons
        return None
    return np.floor(np.ldexp(p, MASS_BITS)).astype(np.int64)


def topp_fixed(top_p: float) -> int:
    """tp = max(1, floor(top_p * 2**24)) for a float32 top_p in (0, 1]."""
    return max(1, int(np.floor(np.float64(np.float32(top_p)) * 2.0**TOPP_BITS)))


def truncate(p32, top_k: int, top_p: float):
    """Kept masses (int64 [V], zero off the kept set) and their total Z (int).

    Returns (None, 0) for an invalid row. Z == 0 means nothing of positive mass
    was kept, which also makes the entry invalid.
    """
    p32 = np.asarray(p32, dtype=np.float32)
    m = masses(p32)
    if m is None:
        return None, 0
    V = m.size
    order = np.lexsort((np.arange(V), -p32.astype(np.float64)))  # step 2
    n_top = V if (top_k <= 0 or top_k >= V) else int(top_k)      # step 3
    top = order[:n_top]
    top_m = [int(v) for v in m[top]]
    Zk = sum(top_m)                                               # step 4
    thr = topp_fixed(top_p) * Zk                                   # step 5
    kept = np.zeros(V, dtype=np.int64)
    before = 0
    for t, mt in zip(top, top_m):
        if before * 2**TOPP_BITS < thr:
            kept[t] = mt
        before += mt
    return kept, int(kept.sum())


# ----------------------------------------------------------------- steps 6-9
def mu24(u) -> int | None:
    """mu = floor(u * 2**24) for a float32 uniform u in [0, 1), else None."""
    u = np.float64(np.float32(u))
    if not (0.0 <= u < 1.0):
        return None
    return int(np.floor(u * 2.0**U_BITS))


def inverse_cdf(r, R: int, mu: int) -> int:
    """Smallest t with r[0] + ... + r[t] > floor(mu * R / 2**24) (token-id order)."""
    tau = (mu * R) >> U_BITS
    return bisect_right(list(accumulate(int(v) for v in r)), tau)


def spec_accept(P, Q, drafts, uniforms, top_k: int = 0, top_p: float = 1.0):
    """One verify step.

    P: float32 [K+1, V] target probabilities; Q: float32 [K, V] draft
    probabilities; drafts: K token ids; uniforms: K+1 float32 values in [0, 1).
    Returns (tokens: list of K+1 ints, n_accepted: int).
    """
    P = np.asarray(P, dtype=np.float32)
    K = len(drafts)
    V = P.shape[-1]
    Q = np.asarray(Q, dtype=np.float32).reshape(K, V)
    bad = ([INVALID] * (K + 1), INVALID)
    rowsP = [truncate(P[i], top_k, top_p) for i in range(K + 1)]
    rowsQ = [truncate(Q[i], top_k, top_p) for i in range(K)]
    if any(kept is None or Z == 0 for kept, Z in rowsP + rowsQ):
        return bad
    mus = [mu24(u) for u in uniforms]
    if len(mus) != K + 1 or any(mu is None for mu in mus):
        return bad
    if any(not (0 <= int(d) < V) for d in drafts):
        return bad

    j = K
    for i in range(K):                                            # step 6
        d = int(drafts[i])
        mP, ZP = rowsP[i]
        mQ, ZQ = rowsQ[i]
        if not (mus[i] * int(mQ[d]) * ZP < int(mP[d]) * ZQ * 2**U_BITS):
            j = i
            break

    mP, ZP = rowsP[j]
    if j < K:                                                     # step 7
        mQ, ZQ = rowsQ[j]
        r = [max(0, int(a) * ZQ - int(b) * ZP) for a, b in zip(mP, mQ)]
        R = sum(r)
        if R == 0:
            r, R = [int(a) for a in mP], ZP
    else:
        r, R = [int(a) for a in mP], ZP
    t = inverse_cdf(r, R, mus[K])                                 # step 8
    tokens = [int(d) for d in drafts[:j]] + [t] + [INVALID] * (K - j)
    return tokens, j


def cdf_edges(r, R: int) -> np.ndarray:
    """int64 e[t] = ceil((r[0] + ... + r[t]) * 2**24 / R).

    The inverse CDF of step 8 returns the number of t with e[t] <= mu: for an
    integer running sum C, C > floor(mu * R / 2**24) holds exactly when
    C * 2**24 > mu * R, i.e. when mu < ceil(C * 2**24 / R).
    """
    one = 2**U_BITS
    return np.array([-(-(c * one) // R) for c in accumulate(int(v) for v in r)], dtype=np.int64)


def sample_truncated(p32, top_k: int, top_p: float, u) -> int:
    """One draw from the truncated distribution p~ by the inverse CDF of step 8
    (used to draw synthetic drafts from q~ in tests)."""
    kept, Z = truncate(p32, top_k, top_p)
    return inverse_cdf(kept, Z, mu24(u))


# ------------------------------------------------- batch of trials, shared rows
class SharedRows:
    """Precomputation for many verify trials that share the same P and Q rows.

    Equivalent to calling ``spec_accept`` per trial. The per-token comparisons
    are rewritten with exact integer ceilings so they vectorise:
      * accept: mu*X < Y  <=>  mu < ceil(Y / X) for X > 0; for X == 0 it is Y > 0;
      * inverse CDF: the smallest t with C_t > floor(mu*R/2**24) is the number
        of t with ceil(C_t * 2**24 / R) <= mu (C_t the running sum of r).
    """

    def __init__(self, P, Q, top_k: int = 0, top_p: float = 1.0):
        P = np.asarray(P, dtype=np.float32)
        self.K = P.shape[0] - 1
        self.V = P.shape[1]
        Q = np.asarray(Q, dtype=np.float32).reshape(self.K, self.V)
        self.rowsP = [truncate(P[i], top_k, top_p) for i in range(self.K + 1)]
        self.rowsQ = [truncate(Q[i], top_k, top_p) for i in range(self.K)]
        self.valid = all(k is not None and Z > 0 for k, Z in self.rowsP + self.rowsQ)
        if not self.valid:
            return
        one = 2**U_BITS
        self.accept_limit = []  # per position: int64 [V], accept iff mu < limit[d]
        for i in range(self.K):
            mP, ZP = self.rowsP[i]
            mQ, ZQ = self.rowsQ[i]
            lim = np.empty(self.V, dtype=np.int64)
            for d in range(self.V):
                X = int(mQ[d]) * ZP
                Y = int(mP[d]) * ZQ * one
                lim[d] = (one if Y > 0 else 0) if X == 0 else min(one, -(-Y // X))
            self.accept_limit.append(lim)
        self.edges = []  # per position j: int64 [V], token = #(edges <= mu)
        for j in range(self.K + 1):
            mP, ZP = self.rowsP[j]
            if j < self.K:
                mQ, ZQ = self.rowsQ[j]
                r = [max(0, int(a) * ZQ - int(b) * ZP) for a, b in zip(mP, mQ)]
                R = sum(r)
                if R == 0:
                    r, R = [int(a) for a in mP], ZP
            else:
                r, R = [int(a) for a in mP], ZP
            self.edges.append(cdf_edges(r, R))

    def run(self, drafts, uniforms):
        """drafts int [B, K], uniforms float32 [B, K+1] -> (tokens [B, K+1], n_accepted [B])."""
        drafts = np.asarray(drafts, dtype=np.int64).reshape(-1, self.K)
        uniforms = np.asarray(uniforms, dtype=np.float32).reshape(-1, self.K + 1)
        B = drafts.shape[0]
        tokens = np.full((B, self.K + 1), INVALID, dtype=np.int64)
        n_acc = np.full(B, INVALID, dtype=np.int64)
        if not self.valid:
            return tokens, n_acc
        u = uniforms.astype(np.float64)
        ok = np.all((u >= 0.0) & (u < 1.0), axis=1) & np.all((drafts >= 0) & (drafts < self.V), axis=1)
        mu = np.floor(np.where((u >= 0.0) & (u < 1.0), u, 0.0) * 2.0**U_BITS).astype(np.int64)
        dr = np.clip(drafts, 0, self.V - 1)
        j = np.full(B, self.K, dtype=np.int64)
        alive = np.ones(B, dtype=bool)
        for i in range(self.K):
            acc = mu[:, i] < self.accept_limit[i][dr[:, i]]
            newly = alive & ~acc
            j[newly] = i
            alive &= acc
        for jj in range(self.K + 1):
            sel = j == jj
            if not sel.any():
                continue
            tokens[sel, jj] = np.searchsorted(self.edges[jj], mu[sel, self.K], side="right")
            for i in range(jj):
                tokens[sel, i] = drafts[sel, i]
        n_acc[:] = j
        tokens[~ok] = INVALID
        n_acc[~ok] = INVALID
        return tokens, n_acc
