"""GPU parity of vq_spec_accept: bit-exact decisions and tokens against the
exact-integer oracle given the same float32 probabilities and uniforms, the
10**6-trial distribution check on the GPU's own outputs, and the float32
softmax of logits mode within tolerance."""
import numpy as np
import pytest
import torch

import oracle.accept as oacc
from synth import accept_logits, accept_logits_correlated, uniforms24
from tests import pins_accept
from tests.gpu_util import f32_tensor, i32_tensor

pytestmark = pytest.mark.gpu


def _entries(config, B, K, V, T, top_k, top_p, corr=None):
    """B independent verifies: rows, drafts drawn from q~, uniforms (numpy)."""
    P = np.empty((B, K + 1, V), np.float32)
    Q = np.empty((B, K, V), np.float32)
    D = np.empty((B, K), np.int64)
    U = uniforms24(config, (B, K + 1), stream="accept-u", extra=7)
    ud = uniforms24(config, (B, K), stream="draft-u", extra=7)
    for b in range(B):
        if corr is None:
            pl, ql = accept_logits(config, K, V, extra=b)
        else:
            pl, ql = accept_logits_correlated(config, K, V, noise=corr, extra=b)
        P[b], Q[b] = oacc.probs_f32(pl, T), oacc.probs_f32(ql, T)
        for i in range(K):
            D[b, i] = oacc.sample_truncated(Q[b, i], top_k, top_p, ud[b, i])
    return P, Q, D, U


def _gpu(vq, P, Q, D, U, **kw):
    toks, n = vq.spec_accept(f32_tensor(P), f32_tensor(Q) if Q.size else None,
                             i32_tensor(D) if D.size else None, f32_tensor(U), **kw)
    torch.cuda.synchronize()
    return toks.cpu().numpy().astype(np.int64), n.cpu().numpy().astype(np.int64)


def _oracle(P, Q, D, U, top_k, top_p):
    res = [oacc.spec_accept(P[b], Q[b], list(D[b]), U[b], top_k, top_p) for b in range(P.shape[0])]
    return np.array([r[0] for r in res], np.int64), np.array([r[1] for r in res], np.int64)


TRUNC = [(0, 1.0), (20, 0.95), (0, 0.95), (5, 1.0), (1, 1.0), (50, 0.5)]


@pytest.mark.parametrize("top_k,top_p", TRUNC)
@pytest.mark.parametrize("corr", [None, 0.5])
def test_config0_entries_bit_exact(vq, top_k, top_p, corr):
    P, Q, D, U = _entries(0, 48, 3, 1000, 1.0, top_k, top_p, corr)
    got = _gpu(vq, P, Q, D, U, top_k=top_k, top_p=top_p)
    ref = _oracle(P, Q, D, U, top_k, top_p)
    assert np.array_equal(got[1], ref[1]) and np.array_equal(got[0], ref[0])


@pytest.mark.parametrize("K,T,top_k,top_p", [(3, 0.7, 0, 0.95), (7, 1.0, 20, 0.95)])
def test_full_vocab_entries_bit_exact(vq, K, T, top_k, top_p):
    """Configs 3 and 4 sampler settings at V = 248320."""
    P, Q, D, U = _entries(3 if K == 3 else 4, 3, K, 248320, T, top_k, top_p, corr=0.3)
    got = _gpu(vq, P, Q, D, U, top_k=top_k, top_p=top_p)
    ref = _oracle(P, Q, D, U, top_k, top_p)
    assert np.array_equal(got[1], ref[1]) and np.array_equal(got[0], ref[0])


def test_invalid_entries_and_edges(vq):
    K, V = 3, 1000
    P, Q, D, U = _entries(0, 8, K, V, 1.0, 0, 1.0)
    P[1, 2, 17] = np.nan
    Q[2, 0, 3] = -1e-8
    D[3, 1] = V
    U[4, 3] = 1.0
    P[5, 1, :] = 0.0
    Q[6, 2, 9] = 1.5
    got = _gpu(vq, P, Q, D, U)
    ref = _oracle(P, Q, D, U, 0, 1.0)
    assert np.array_equal(got[1], ref[1]) and np.array_equal(got[0], ref[0])
    assert list(got[1][1:7]) == [-1] * 6 and got[1][0] >= 0 and got[1][7] >= 0


def test_k0_plain_sampling(vq):
    P, Q, D, U = _entries(0, 16, 0, 1000, 1.0, 0, 1.0)
    got = _gpu(vq, P, Q, D, U, top_k=10, top_p=0.9)
    ref = _oracle(P, Q, D, U, 10, 0.9)
    assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1])


def test_tiny_vocab_and_hand_examples(vq):
    import json, os
    with open(os.path.join(os.path.dirname(__file__), "golden", "accept_hand.json")) as f:
        cases = json.load(f)["accept"]
    for c in cases:
        P = np.array([c["P"]], np.float32)
        K = len(c["drafts"])
        Q = np.array(c["Q"], np.float32).reshape(1, K, P.shape[2])
        D = np.array([c["drafts"]], np.int64).reshape(1, K)
        U = np.array([c["uniforms"]], np.float32)
        toks, n = _gpu(vq, P, Q, D, U, top_k=c["top_k"], top_p=c["top_p"])
        assert list(toks[0]) == c["tokens"] and int(n[0]) == c["n_accepted"], c["why"]


@pytest.mark.parametrize("name,cfg", [
    ("config0", dict(config=0, K=3, V=1000, T=1.0, top_k=0, top_p=1.0)),
    ("config0 correlated", dict(config=0, K=3, V=1000, T=1.0, top_k=0, top_p=1.0, corr=0.5)),
    ("config4 V=248320 K=7 top-k 20 top-p 0.95", dict(config=4, K=7, V=248320, T=1.0, top_k=20, top_p=0.95, corr=0.3)),
])
def test_shared_rows_1e6_trials(vq, name, cfg):
    """10**6 trials of one verify: GPU tokens bit-exact against the oracle and
    distributed as p~ per position (chi-square)."""
    tr = pins_accept.make_trials(oacc, n_trials=10**6, **cfg)
    toks, n = vq.spec_accept(f32_tensor(tr["P"]), f32_tensor(tr["Q"]), i32_tensor(tr["drafts"]),
                             f32_tensor(tr["uniforms"]), top_k=cfg["top_k"], top_p=cfg["top_p"])
    torch.cuda.synchronize()
    toks, n = toks.cpu().numpy().astype(np.int64), n.cpu().numpy().astype(np.int64)
    rt, rn = tr["sr"].run(tr["drafts"], tr["uniforms"])
    assert np.array_equal(n, rn) and np.array_equal(toks, rt)
    pins_accept.check_distribution(tr["sr"], toks, n, cfg["K"], cfg["V"])


@pytest.mark.parametrize("V,T,top_k,top_p", [(1000, 1.0, 0, 1.0), (248320, 0.7, 0, 0.95), (248320, 1.0, 20, 0.95)])
def test_logits_mode(vq, V, T, top_k, top_p):
    """float32 softmax against the float64 oracle; tokens valid and, over 10**6
    shared-row trials, distributed as the oracle's p~."""
    K = 3
    tr = pins_accept.make_trials(oacc, config=3, K=K, V=V, T=T, top_k=top_k, top_p=top_p, n_trials=10**6, corr=0.3)
    pl, ql = tr["logits"]
    probs = torch.empty((1, 2 * K + 1, V), dtype=torch.float32, device="cuda")
    toks, n = vq.spec_accept(f32_tensor(pl), f32_tensor(ql), i32_tensor(tr["drafts"]), f32_tensor(tr["uniforms"]),
                             logits=True, temperature=T, top_k=top_k, top_p=top_p, probs_out=probs)
    torch.cuda.synchronize()
    ref = np.concatenate([oacc.softmax_f64(pl, T), oacc.softmax_f64(ql, T)])
    got = probs[0].cpu().numpy().astype(np.float64)
    err = np.abs(got - ref)
    assert err.max() <= 1e-2 * ref.max() + 1e-3
    assert np.all(err <= 1e-4 * ref + 1e-12), float((err / (ref + 1e-30)).max())
    toks, n = toks.cpu().numpy().astype(np.int64), n.cpu().numpy().astype(np.int64)
    pins_accept.check_distribution(tr["sr"], toks, n, K, V)


@pytest.mark.parametrize("top_k,top_p", [(20, 0.95), (0, 0.95), (0, 1.0)])
def test_many_entries_per_row_path(vq, top_k, top_p):
    """Enough verifies that every row gets its own workgroup (no chunked stages)."""
    P, Q, D, U = _entries(0, 160, 3, 500, 1.0, top_k, top_p, corr=0.5)
    got = _gpu(vq, P, Q, D, U, top_k=top_k, top_p=top_p)
    ref = _oracle(P, Q, D, U, top_k, top_p)
    assert np.array_equal(got[1], ref[1]) and np.array_equal(got[0], ref[0])


@pytest.mark.parametrize("top_k,top_p", [(0, 0.9), (30000, 0.9), (0, 1.0), (100, 1.0)])
def test_crowded_rows(vq, top_k, top_p):
    """Uniform target rows put every key in one histogram bin: more keys than the
    chunked selects gather, so those rows take the single-workgroup path."""
    K, V = 2, 40000
    P, Q, D, U = _entries(5, 4, K, V, 1.0, top_k, top_p)
    P[0, :, :] = oacc.probs_f32(np.zeros((K + 1, V), np.float32), 1.0)
    P[2, 1, :] = P[0, 1, :]
    Q[3, 0, :] = oacc.probs_f32(np.zeros((1, V), np.float32), 1.0)[0]
    got = _gpu(vq, P, Q, D, U, top_k=top_k, top_p=top_p)
    ref = _oracle(P, Q, D, U, top_k, top_p)
    assert np.array_equal(got[1], ref[1]) and np.array_equal(got[0], ref[0])


@pytest.mark.parametrize("B,K", [(1, 7), (150, 7)])   # chunked stages; one workgroup per row (2250 rows)
def test_huge_logits_stay_valid(vq, B, K):
    """Logits of magnitude ~1.5e4 (float32 ulp ~0.002 after scaling): every computed
    probability stays in [0, 1], every entry is valid, and the tokens are the
    oracle's on the device's own probabilities."""
    V, T, top_k, top_p = 248320, 1.0, 20, 0.95
    g = np.random.default_rng(B)
    pl = (15000.0 + 60.0 * g.standard_normal((B, K + 1, V))).astype(np.float32)
    ql = (g.standard_normal((B, K, V)) * 2.0).astype(np.float32)
    drafts = np.stack([[int(np.argmax(ql[b, i])) for i in range(K)] for b in range(B)]).astype(np.int32)
    us = np.asarray(g.integers(0, 2 ** 24, size=(B, K + 1)) * 2.0 ** -24, np.float32)
    probs = torch.empty((B, 2 * K + 1, V), dtype=torch.float32, device="cuda")
    toks, n = vq.spec_accept(f32_tensor(pl), f32_tensor(ql), i32_tensor(drafts), f32_tensor(us), logits=True,
                             temperature=T, top_k=top_k, top_p=top_p, probs_out=probs)
    torch.cuda.synchronize()
    pr = probs.cpu().numpy()
    assert np.all(pr >= 0) and np.all(pr <= 1), float(pr.max())
    n = n.cpu().numpy()
    assert np.all(n >= 0)
    toks = toks.cpu().numpy()
    for b in range(min(B, 8)):
        rt, rn = oacc.spec_accept(pr[b, : K + 1].astype(np.float64), pr[b, K + 1:].astype(np.float64),
                                  list(drafts[b]), us[b], top_k, top_p)
        assert list(toks[b]) == rt and int(n[b]) == rn


def _structured_row(kind: str, V: int, rng) -> np.ndarray:
    """float32 probability rows whose keys crowd the first histogram levels:
    one_hot: a few head tokens, every other probability exactly 0 (the zeros
      share every key bit above the token id: three levels deep);
    flat_tail: half the mass on a few tokens, the rest uniform over the tail;
    l1_spread: 20000 tokens whose probabilities share the top key bits and
      differ in mantissa bits 11..6 (separated at level 1), the rest 0;
    l2_spread: 30000 tokens differing only in mantissa bits 5..0 (level 2);
    two_bins: 20000 tokens at 2^-15, 20000 at 2^-17, the rest 0."""
    p = np.zeros(V, np.float32)
    ids = rng.permutation(V)
    if kind == "one_hot":
        p[ids[0]] = 0.9
        p[ids[1:6]] = 0.02
    elif kind == "flat_tail":
        p[ids[:4]] = 0.125
        p[ids[4:]] = np.float32(0.5 / (V - 4))
    elif kind == "l1_spread":
        j = rng.integers(0, 64, 20000)
        p[ids[:20000]] = (2.0 ** -16 * (1.0 + j * 2.0 ** -17)).astype(np.float32)
    elif kind == "l2_spread":
        j = rng.integers(0, 64, 30000)
        p[ids[:30000]] = (2.0 ** -16 * (1.0 + j * 2.0 ** -23)).astype(np.float32)
    elif kind == "two_bins":
        p[ids[:20000]] = 2.0 ** -15
        p[ids[20000:40000]] = 2.0 ** -17
    else:
        raise ValueError(kind)
    return p


@pytest.mark.parametrize("kind,top_k,top_p", [
    ("one_hot", 20, 0.95), ("one_hot", 20, 1.0), ("flat_tail", 0, 0.95), ("flat_tail", 20, 0.95),
    ("l1_spread", 5000, 0.95), ("l1_spread", 5000, 0.9999), ("l1_spread", 0, 0.5),
    ("l2_spread", 7000, 0.95), ("l2_spread", 7000, 0.99999), ("two_bins", 25000, 0.5), ("two_bins", 30000, 1.0),
])
def test_refined_regions(vq, kind, top_k, top_p):
    """Rows whose crossing bin holds more keys than one gather: the chunked
    pipeline narrows it by one or two more histogram levels (and the top-p walk
    after top-k crosses at those levels); a top-p walk after a top-k wider than
    the gather buffer may still end in the single-workgroup rows kernel
    (two_bins, top-k 25000). Bit-exact against the oracle at V = 248320, K = 7."""
    K, V, B = 7, 248320, 2
    rng = np.random.default_rng(sum(map(ord, kind)) + top_k)
    P = np.stack([np.stack([_structured_row(kind, V, rng) for _ in range(K + 1)]) for _ in range(B)])
    Q = np.stack([np.stack([_structured_row(kind, V, rng) for _ in range(K)]) for _ in range(B)])
    Q[0] = P[0, :K]          # entry 0: q = p, every draft accepted, then the bonus draw
    ud = uniforms24(9, (B, K), stream="draft-u")
    U = uniforms24(9, (B, K + 1))
    D = np.array([[oacc.sample_truncated(Q[b, i], top_k, top_p, ud[b, i]) for i in range(K)] for b in range(B)])
    # a draft the target may reject (drawn from another row's support)
    D[1, 0] = int(np.argmax(P[0, 3]))
    got = _gpu(vq, P, Q, D, U, top_k=top_k, top_p=top_p)
    ref = _oracle(P, Q, D, U, top_k, top_p)
    assert np.array_equal(got[1], ref[1]) and np.array_equal(got[0], ref[0]), (got, ref)


def _small_k_row(kind: str, V: int, rng) -> np.ndarray:
    if kind == "random":
        p = rng.random(V) ** 8
        return (p / p.sum()).astype(np.float32)
    if kind == "flat":
        return np.full(V, np.float32(1.0 / V))
    if kind == "periodic":  # every 4096-element chunk holds the same values
        p = np.tile(rng.random(4096) ** 8, -(-V // 4096))[:V]
        return (p / p.sum()).astype(np.float32)
    return _structured_row(kind, V, rng)


@pytest.mark.parametrize("V,top_k,top_p,kind", [
    (3 * 4096 + 5, 20, 0.95, "random"),     # last chunk shorter than top_k
    (3 * 4096 + 5, 64, 1.0, "random"),
    (100, 64, 0.9, "random"),               # a single chunk
    (65, 64, 1.0, "random"),                # every key but one kept
    (5000, 63, 0.8, "flat"),                # equal probabilities: the ids decide
    (248320, 20, 0.95, "flat"),
    (248320, 1, 1.0, "one_hot"),
    (248320, 64, 0.95, "one_hot"),          # fewer nonzero than top_k: zeros in id order
    (248320, 65, 0.95, "one_hot"),          # just above the per-chunk candidate path
    (40000, 50, 0.5, "random"),
    # every chunk's top values tie with every other chunk's: about 19 (63)
    # candidates per chunk survive the chunk bound, more than the merge ranks
    # directly, so the row goes through the digit-by-digit select
    (248320, 20, 0.95, "periodic"),
    (248320, 64, 0.9, "periodic"),
])
def test_small_top_k(vq, V, top_k, top_p, kind):
    """Top-k of at most 64 goes through per-chunk candidates and one select per
    row over them: short and single chunks, ties broken by id across chunks,
    rows with fewer nonzero probabilities than top_k. Bit-exact, K = 3."""
    K, B = 3, 3
    rng = np.random.default_rng(V + 7 * top_k + sum(map(ord, kind)))
    P = np.stack([np.stack([_small_k_row(kind, V, rng) for _ in range(K + 1)]) for _ in range(B)])
    Q = np.stack([np.stack([_small_k_row(kind, V, rng) for _ in range(K)]) for _ in range(B)])
    Q[0] = P[0, :K]          # every draft accepted, then the bonus draw
    ud = uniforms24(11, (B, K), stream="draft-u")
    U = uniforms24(11, (B, K + 1))
    D = np.array([[oacc.sample_truncated(Q[b, i], top_k, top_p, ud[b, i]) for i in range(K)] for b in range(B)])
    got = _gpu(vq, P, Q, D, U, top_k=top_k, top_p=top_p)
    ref = _oracle(P, Q, D, U, top_k, top_p)
    assert np.array_equal(got[1], ref[1]) and np.array_equal(got[0], ref[0]), (got, ref)


def test_small_top_k_invalid_rows(vq):
    """Invalid probabilities and an all-zero row under top-k 20: the entries they
    touch report -1, the others match the oracle."""
    K, V = 3, 10000
    P, Q, D, U = _entries(0, 6, K, V, 1.0, 20, 0.95)
    P[1, 2, 17] = np.nan
    Q[2, 0, 3] = -1e-8
    P[3, 1, :] = 0.0
    Q[4, 2, 9999] = 1.5
    got = _gpu(vq, P, Q, D, U, top_k=20, top_p=0.95)
    ref = _oracle(P, Q, D, U, 20, 0.95)
    assert np.array_equal(got[1], ref[1]) and np.array_equal(got[0], ref[0])
    assert list(got[1][1:5]) == [-1] * 4 and got[1][0] >= 0 and got[1][5] >= 0
