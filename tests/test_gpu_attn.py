"""GPU parity of vq_multirow_attn against the float64 oracle."""
import math

import numpy as np
import pytest
import torch

import oracle.attn as oa
from synth import attn_inputs
from tests.gpu_util import assert_close, bf16_tensor, i32_tensor, to_f64

pytestmark = pytest.mark.gpu


def _run(vq, q, k, v, T, scale):
    out = vq.multirow_attn(bf16_tensor(q), bf16_tensor(k), bf16_tensor(v), T, scale)
    torch.cuda.synchronize()
    return to_f64(out)


@pytest.mark.parametrize("M,Hq,Hkv,D,T,T_cap", [
    (4, 2, 2, 64, 256, 256),       # config 0
    (5, 12, 2, 64, 256, 260),      # GQA 6:1, T_cap > T
    (1, 8, 8, 128, 100, 128),      # single row, ragged T
    (3, 8, 2, 128, 67, 70),        # T not a multiple of the tile
    (2, 24, 4, 256, 40, 40),       # config-2 heads, short context
    (6, 24, 4, 256, 300, 320),     # 36 rows per KV head: two row tiles
    (16, 24, 4, 256, 90, 96),      # 96 rows: three row tiles
    (16, 8, 1, 256, 130, 130),     # 128 rows: four row tiles
    (16, 16, 2, 128, 16, 16),      # T == M: every row sees a different prefix
    (7, 4, 4, 64, 5000, 5000),     # many key ranges -> combine kernel
])
def test_shapes_full(vq, M, Hq, Hkv, D, T, T_cap):
    q, k, v = attn_inputs(0 if (M, T) == (4, 256) else 20, M, Hq, Hkv, D, T_cap, extra=T)
    scale = 1 / math.sqrt(D)
    ref = oa.multirow_attention(q, k, v, M, Hq, Hkv, D, T, T_cap, scale)
    assert_close(_run(vq, q, k, v, T, scale), ref, f"M={M} Hq={Hq} Hkv={Hkv} D={D} T={T}")


@pytest.mark.parametrize("ctx", [8192, 32768])
@pytest.mark.parametrize("M", [2, 3, 4, 5, 6, 7, 8])
def test_config2_sampled(vq, ctx, M):
    """Config 2: Hq=24, Hkv=4, D=256, KV at ctx committed positions + M drafted rows."""
    Hq, Hkv, D = 24, 4, 256
    T = ctx + M
    q, k, v = attn_inputs(2, M, Hq, Hkv, D, T, extra=ctx)
    out = _run(vq, q, k, v, T, 1 / 16)
    rng = np.random.default_rng(ctx + M)
    pairs = [(m, int(h)) for m in range(M) for h in rng.choice(Hq, 3, replace=False)]
    ref = oa.multirow_attention(q, k, v, M, Hq, Hkv, D, T, T, 1 / 16, pairs=pairs)
    got = np.stack([out[m, h] for m, h in pairs])
    assert_close(got, ref, f"ctx={ctx} M={M}")


@pytest.mark.parametrize("M", [8, 2])
def test_config4_context_sampled(vq, M):
    """The 8-bit step's attention shape: 8 rows over 131072 committed positions
    (T = 131080, 129 key ranges of 32 tiles per KV head and the combine), on
    sampled (row, head) pairs; and 2 rows (one row tile: queries in registers,
    two K/V buffers, two workgroups per compute unit)."""
    Hq, Hkv, D, ctx = 24, 4, 256, 131072
    T = ctx + M
    q, k, v = attn_inputs(4, M, Hq, Hkv, D, T, extra=ctx)
    out = _run(vq, q, k, v, T, 1 / 16)
    rng = np.random.default_rng(ctx + M)
    pairs = [(m, int(h)) for m in range(M) for h in rng.choice(Hq, 2, replace=False)]
    ref = oa.multirow_attention(q, k, v, M, Hq, Hkv, D, T, T, 1 / 16, pairs=pairs)
    got = np.stack([out[m, h] for m, h in pairs])
    assert_close(got, ref, f"ctx={ctx} M={M}")


def test_deterministic(vq):
    q, k, v = attn_inputs(21, 8, 24, 4, 256, 8200)
    a = _run(vq, q, k, v, 8200, 1 / 16)
    for _ in range(2):
        assert np.array_equal(a, _run(vq, q, k, v, 8200, 1 / 16))


@pytest.mark.parametrize("M,Hq,Hkv,D,T,T_cap", [
    (4, 2, 2, 64, 256, 260),       # config 0 with the append
    (8, 4, 2, 64, 1026, 1030),     # the appended rows straddle two key ranges
    (16, 16, 2, 128, 16, 20),      # T == M: every key is appended
    (4, 24, 4, 256, 4100, 4100),   # 27B heads
])
def test_append_fused(vq, M, Hq, Hkv, D, T, T_cap):
    """vq_multirow_attn_append: the M new rows (taken from a fused q|k|v-like row
    layout) land at cache positions T-M .. T-1 and the output equals the
    attention over the appended cache, bit for bit with the separate append."""
    q, k, v = attn_inputs(22, M, Hq, Hkv, D, T_cap, extra=T)
    rng = np.random.default_rng(T)
    new = rng.standard_normal((M, 2 * Hkv * D + 16)).astype(np.float32)
    from tests.gpu_util import dev
    import oracle.stack as ostack
    new_bits = ostack.to_bf16_bits(new.astype(np.float64))
    src = bf16_tensor(new_bits)
    k_new, v_new = src[:, : Hkv * D], src[:, Hkv * D: 2 * Hkv * D]
    # fused
    kc, vc = bf16_tensor(k), bf16_tensor(v)
    out = vq.multirow_attn(bf16_tensor(q), kc, vc, T, 1 / math.sqrt(D), k_new=k_new, v_new=v_new)
    # separate append then attention
    kc2, vc2 = bf16_tensor(k), bf16_tensor(v)
    vq.kv_append(src, 0, Hkv * D, kc2, vc2, T - M)
    out2 = vq.multirow_attn(bf16_tensor(q), kc2, vc2, T, 1 / math.sqrt(D))
    torch.cuda.synchronize()
    assert torch.equal(kc, kc2) and torch.equal(vc, vc2)
    assert torch.equal(out, out2)
    # oracle on the appended cache
    ka, va = k.copy(), v.copy()
    ka[:, T - M: T] = new_bits[:, : Hkv * D].reshape(M, Hkv, D).transpose(1, 0, 2)
    va[:, T - M: T] = new_bits[:, Hkv * D: 2 * Hkv * D].reshape(M, Hkv, D).transpose(1, 0, 2)
    ref = oa.multirow_attention(q, ka, va, M, Hq, Hkv, D, T, T_cap, 1 / math.sqrt(D))
    assert_close(to_f64(out), ref, "append fused vs oracle")
    # rows past T untouched
    assert torch.equal(kc[:, T:], bf16_tensor(k)[:, T:])


# ------------------------------------------------------------------ tree verify
def _tree(vq, q, k, v, T, scale, mask, k_new=None, v_new=None, kc=None, vc=None):
    from tests.gpu_util import i32_tensor
    mt = i32_tensor(np.asarray(mask, np.uint32).view(np.int32))
    kc = bf16_tensor(k) if kc is None else kc
    vc = bf16_tensor(v) if vc is None else vc
    out = vq.multirow_attn(bf16_tensor(q), kc, vc, T, scale, tree_mask=mt, k_new=k_new, v_new=v_new)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("M,Hq,Hkv,D,T,T_cap", [
    (4, 2, 2, 64, 256, 256),       # config 0 heads
    (8, 12, 2, 64, 300, 300),      # GQA, 48 rows
    (16, 8, 2, 128, 16, 16),       # T == M: only drafted keys
    (16, 24, 4, 256, 200, 208),    # 27B heads, 96 rows per KV head
    (5, 4, 4, 128, 3000, 3000),    # several key ranges, the tree in the last one
    (1, 8, 8, 64, 70, 70),         # a single node
])
def test_tree_random(vq, M, Hq, Hkv, D, T, T_cap):
    from synth import tree_masks
    q, k, v = attn_inputs(23, M, Hq, Hkv, D, T_cap, extra=T)
    mask = tree_masks(23, M, extra=T)
    scale = 1 / math.sqrt(D)
    got = to_f64(_tree(vq, q, k, v, T, scale, mask))
    ref = oa.tree_attention(q, k, v, M, Hq, Hkv, D, T, T_cap, scale, mask)
    assert_close(got, ref, f"tree M={M} Hq={Hq} Hkv={Hkv} D={D} T={T}")


def test_tree_arbitrary_masks(vq):
    """Masks that are not trees: the self bit missing, bits at or above M, all bits."""
    M, Hq, Hkv, D, T = 8, 12, 2, 64, 100
    q, k, v = attn_inputs(24, M, Hq, Hkv, D, T)
    mask = np.array([0, 0xFFFFFFFF, 0x100, 5, 0xF0, 2, 0xFF, 1 << 31], np.uint32)
    got = to_f64(_tree(vq, q, k, v, T, 0.125, mask))
    assert_close(got, oa.tree_attention(q, k, v, M, Hq, Hkv, D, T, T, 0.125, mask), "arbitrary masks")


@pytest.mark.parametrize("M,D,T", [(4, 64, 256), (8, 256, 5000), (16, 128, 16)])
def test_tree_chain_equals_causal(vq, M, D, T):
    """The chain mask gives the causal call's output bit for bit (same kernel, same
    arithmetic)."""
    from synth import chain_masks
    Hq, Hkv = 8, 2
    q, k, v = attn_inputs(25, M, Hq, Hkv, D, T, extra=T)
    scale = 1 / math.sqrt(D)
    tree = _tree(vq, q, k, v, T, scale, chain_masks(M))
    causal = vq.multirow_attn(bf16_tensor(q), bf16_tensor(k), bf16_tensor(v), T, scale)
    torch.cuda.synchronize()
    assert torch.equal(tree, causal)


def test_tree_config2_sampled(vq):
    """27B heads at 16k + 16 tree nodes: sampled (node, head) pairs against the oracle."""
    from synth import tree_masks
    M, Hq, Hkv, D, ctx = 16, 24, 4, 256, 16384
    T = ctx + M
    q, k, v = attn_inputs(26, M, Hq, Hkv, D, T)
    mask = tree_masks(26, M)
    out = to_f64(_tree(vq, q, k, v, T, 1 / 16, mask))
    rng = np.random.default_rng(26)
    pairs = [(m, int(h)) for m in range(M) for h in rng.choice(Hq, 2, replace=False)]
    ref = oa.tree_attention(q, k, v, M, Hq, Hkv, D, T, T, 1 / 16, mask, pairs=pairs)
    assert_close(np.stack([out[m, h] for m, h in pairs]), ref, "tree at 16k")


def test_tree_with_append(vq):
    """Tree verify with the append fused in: equals the tree call on a cache appended beforehand."""
    from synth import tree_masks
    import oracle.stack as ostack
    M, Hq, Hkv, D, T = 8, 12, 2, 128, 2050
    q, k, v = attn_inputs(27, M, Hq, Hkv, D, T + 4, extra=T)
    mask = tree_masks(27, M)
    new_bits = ostack.to_bf16_bits(np.random.default_rng(27).standard_normal((M, 2 * Hkv * D)))
    src = bf16_tensor(new_bits)
    k_new, v_new = src[:, : Hkv * D], src[:, Hkv * D:]
    kc, vc = bf16_tensor(k), bf16_tensor(v)
    out = _tree(vq, q, k, v, T, 0.1, mask, k_new=k_new, v_new=v_new, kc=kc, vc=vc)
    kc2, vc2 = bf16_tensor(k), bf16_tensor(v)
    vq.kv_append(src, 0, Hkv * D, kc2, vc2, T - M)
    out2 = _tree(vq, q, k, v, T, 0.1, mask, kc=kc2, vc=vc2)
    assert torch.equal(kc, kc2) and torch.equal(vc, vc2) and torch.equal(out, out2)
    ka, va = k.copy(), v.copy()
    ka[:, T - M: T] = new_bits[:, : Hkv * D].reshape(M, Hkv, D).transpose(1, 0, 2)
    va[:, T - M: T] = new_bits[:, Hkv * D:].reshape(M, Hkv, D).transpose(1, 0, 2)
    assert_close(to_f64(out), oa.tree_attention(q, ka, va, M, Hq, Hkv, D, T, T + 4, 0.1, mask), "tree + append")


# ------------------------------------------------------------- several sequences
def _batched_inputs(seed, Ms, Ts, Hq, Hkv, D, T_cap):
    B = len(Ms)
    qs, ks, vs = [], [], []
    for b in range(B):
        q, k, v = attn_inputs(seed, Ms[b], Hq, Hkv, D, T_cap, extra=100 * b + Ts[b])
        qs.append(q)
        ks.append(k)
        vs.append(v)
    return qs, np.stack(ks), np.stack(vs)


@pytest.mark.parametrize("Ms,Ts,Hq,Hkv,D", [
    ([4, 1, 7], [300, 5000, 40], 12, 2, 64),       # different rows and lengths, one long
    ([4, 4, 4, 4], [16400, 200, 9000, 4], 24, 4, 256),   # four 27B-head streams of K = 3
    ([16], [77], 8, 2, 128),                        # one sequence
    ([2, 3], [2, 3], 4, 4, 128),                    # T_b == M_b
])
@pytest.mark.parametrize("tree", [False, True])
def test_batched_sequences(vq, Ms, Ts, Hq, Hkv, D, tree):
    from synth import tree_masks
    T_cap = max(Ts) + 8
    qs, kc, vc = _batched_inputs(28, Ms, Ts, Hq, Hkv, D, T_cap)
    masks = [tree_masks(28, m, extra=b) if tree else None for b, m in enumerate(Ms)]
    qall = bf16_tensor(np.concatenate(qs))
    rs = i32_tensor(np.concatenate([[0], np.cumsum(Ms)]))
    sl = i32_tensor(np.array(Ts))
    mt = i32_tensor(np.concatenate(masks).view(np.int32)) if tree else None
    out = to_f64(vq.multirow_attn_batched(qall, rs, sl, bf16_tensor(kc), bf16_tensor(vc), max(Ms), max(Ts), 0.1,
                                          tree_mask=mt))
    torch.cuda.synchronize()
    r0 = 0
    for b, (m, T) in enumerate(zip(Ms, Ts)):
        if T > 4096:   # long sequences: sampled (row, head) pairs
            pairs = [(i, h) for i in range(m) for h in (0, Hq - 1)]
        else:
            pairs = None
        args = (qs[b], kc[b], vc[b], m, Hq, Hkv, D, T, T_cap, 0.1)
        if tree:
            ref = oa.tree_attention(*args, masks[b], pairs=pairs)
        else:
            ref = oa.multirow_attention(*args, pairs=pairs)
        got = out[r0: r0 + m] if pairs is None else np.stack([out[r0 + i, h] for i, h in pairs])
        assert_close(got, ref, f"sequence {b} (M={m}, T={T}, tree={tree})")
        r0 += m


def test_batched_append_and_empty_sequence(vq):
    """Fused append per sequence, and a sequence with no rows (row_start[b] ==
    row_start[b+1]) that leaves its cache and the others' results untouched."""
    import oracle.stack as ostack
    Ms, Ts, Hq, Hkv, D = [3, 0, 5], [1030, 50, 70], 8, 2, 128
    T_cap = 1040
    qs, kc, vc = _batched_inputs(29, [3, 1, 5], Ts, Hq, Hkv, D, T_cap)
    qs[1] = qs[1][:0]
    R = sum(Ms)
    new_bits = ostack.to_bf16_bits(np.random.default_rng(29).standard_normal((R, 2 * Hkv * D)))
    src = bf16_tensor(new_bits)
    kd, vd = bf16_tensor(kc), bf16_tensor(vc)
    rs = i32_tensor(np.array([0, 3, 3, 8]))
    sl = i32_tensor(np.array(Ts))
    out = to_f64(vq.multirow_attn_batched(bf16_tensor(np.concatenate(qs)), rs, sl, kd, vd, 5, max(Ts), 0.09,
                                          k_new=src[:, : Hkv * D], v_new=src[:, Hkv * D:]))
    torch.cuda.synchronize()
    assert torch.equal(kd[1], bf16_tensor(kc[1])) and torch.equal(vd[1], bf16_tensor(vc[1]))
    r0 = 0
    for b, (m, T) in enumerate(zip(Ms, Ts)):
        if m == 0:
            continue
        ka, va = kc[b].copy(), vc[b].copy()
        ka[:, T - m: T] = new_bits[r0: r0 + m, : Hkv * D].reshape(m, Hkv, D).transpose(1, 0, 2)
        va[:, T - m: T] = new_bits[r0: r0 + m, Hkv * D:].reshape(m, Hkv, D).transpose(1, 0, 2)
        assert np.array_equal(to_f64(kd[b]), to_f64(bf16_tensor(ka)))
        ref = oa.multirow_attention(qs[b], ka, va, m, Hq, Hkv, D, T, T_cap, 0.09)
        assert_close(out[r0: r0 + m], ref, f"sequence {b} with append")
        r0 += m


# Long key ranges (16 KV heads, ten tiles per range: the unconditional main
# loop and the tested tail both run) at every row-tile count, for the head
# sizes the 27B shape does not use. Every row of the last KV head is compared
# (every row position of every row tile).
LONG_RANGES = [
    (4, 32, 64), (8, 96, 64), (16, 80, 64), (16, 128, 64),     # 8 / 48 / 80 / 128 rows per KV head
    (4, 32, 128), (8, 96, 128), (16, 80, 128), (16, 128, 128),
]
LONG_HKV, LONG_CTX = 16, 5000


@pytest.mark.parametrize("M,Hq,D", LONG_RANGES)
@pytest.mark.parametrize("tree", [False, True])
def test_long_ranges_every_row_tile(vq, M, Hq, D, tree):
    from synth import tree_masks
    Hkv, T = LONG_HKV, LONG_CTX + M
    G = Hq // Hkv
    q, k, v = attn_inputs(60 + M, M, Hq, Hkv, D, T, extra=D)
    scale = 1 / math.sqrt(D)
    mask = tree_masks(60, M, extra=D) if tree else None
    got = to_f64(_tree(vq, q, k, v, T, scale, mask)) if tree else _run(vq, q, k, v, T, scale)
    # The oracle on the last KV head alone (heads are independent): its G query
    # heads against that head's cache.
    qs, ks, vs = np.ascontiguousarray(q[:, Hq - G:]), k[Hkv - 1:], v[Hkv - 1:]
    if tree:
        ref = oa.tree_attention(qs, ks, vs, M, G, 1, D, T, T, scale, mask)
    else:
        ref = oa.multirow_attention(qs, ks, vs, M, G, 1, D, T, T, scale)
    assert_close(got[:, Hq - G:], ref, f"long ranges M={M} Hq={Hq} D={D} tree={tree}")
