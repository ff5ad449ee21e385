"""GPU parity of the 8-bit KV cache: the quantizing append against the oracle's
codes and (scale, bias) words bit for bit, attention over the cache against the
float64 oracle (causal and tree), and bit-equality with the bf16 path on a cache
whose values lie on the quantization grid."""
import math

import numpy as np
import pytest
import torch

import oracle.kv8 as okv
from synth import attn_inputs, tree_masks
from tests.gpu_util import assert_close, bf16_tensor, dev, i32_tensor, to_f64
from tests.pins_kv8 import _grid_rows

pytestmark = pytest.mark.gpu


def _words(sb: np.ndarray) -> np.ndarray:
    """[..., G, 2] uint16 (scale, bias) -> [..., G] uint32 words (scale in the low half)."""
    return np.ascontiguousarray(sb, np.uint16).view(np.uint32)[..., 0] if sb.shape[-1] == 2 else sb


def _dev_cache(codes, sb):
    c = torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).to(dev())
    w = torch.from_numpy(np.ascontiguousarray(sb, np.uint16).view(np.int32).reshape(sb.shape[:-1])).to(dev())
    return c, w


def _oracle_cache(seed, M, Hq, Hkv, D, T_cap):
    q, k, v = attn_inputs(seed, M, Hq, Hkv, D, T_cap)
    kc, ks = okv.quantize_rows(k)
    vc, vs = okv.quantize_rows(v)
    return q, kc, ks, vc, vs


def _mask_tensor(mask):
    return i32_tensor(np.asarray(mask, np.uint32).view(np.int32))


@pytest.mark.parametrize("M,Hkv,D,pos,T_cap", [(4, 2, 64, 252, 256), (8, 4, 256, 100, 120), (16, 2, 128, 0, 16),
                                               (1, 8, 64, 7, 9)])
def test_append_codes_exact(vq, M, Hkv, D, pos, T_cap):
    """Codes and words of the appended rows equal the oracle's, bit for bit; every
    other position is untouched. Rows include a constant group and evenly spaced
    values (many exact halves after the division)."""
    rng = np.random.default_rng(M * 1000 + D)
    width = 2 * Hkv * D + 8
    from synth import f32_to_bf16_bits
    rows = f32_to_bf16_bits(rng.standard_normal((M, width)).astype(np.float32) * 3)
    rows[0, :64] = rows[0, 0]                                          # constant key group
    rows[-1, Hkv * D: Hkv * D + 64] = f32_to_bf16_bits(np.linspace(-2, 2, 64).astype(np.float32))
    src = bf16_tensor(rows)
    kq = torch.full((Hkv, T_cap, D), 7, dtype=torch.uint8, device=dev())
    vq8 = torch.full((Hkv, T_cap, D), 7, dtype=torch.uint8, device=dev())
    ks = torch.full((Hkv, T_cap, D // 64), 123, dtype=torch.int32, device=dev())
    vs = torch.full((Hkv, T_cap, D // 64), 123, dtype=torch.int32, device=dev())
    vq.kv8_append(src, 0, Hkv * D, kq, ks, vq8, vs, pos)
    torch.cuda.synchronize()
    knew = rows[:, : Hkv * D].reshape(M, Hkv, D).transpose(1, 0, 2)
    vnew = rows[:, Hkv * D: 2 * Hkv * D].reshape(M, Hkv, D).transpose(1, 0, 2)
    for got_c, got_w, x in ((kq, ks, knew), (vq8, vs, vnew)):
        c, sb = okv.quantize_rows(x)
        gc, gw = got_c.cpu().numpy(), got_w.cpu().numpy().view(np.uint32)
        assert np.array_equal(gc[:, pos: pos + M], c), "codes"
        assert np.array_equal(gw[:, pos: pos + M], _words(sb)), "scale|bias words"
        assert np.all(np.delete(gc, np.s_[pos: pos + M], axis=1) == 7)
        assert np.all(np.delete(gw, np.s_[pos: pos + M], axis=1) == 123)


@pytest.mark.parametrize("M,Hq,Hkv,D,T,T_cap", [
    (4, 2, 2, 64, 256, 256),       # config 0 heads
    (5, 12, 2, 64, 300, 320),      # GQA 6:1
    (16, 8, 2, 128, 16, 16),       # T == M
    (8, 24, 4, 256, 200, 200),     # 27B heads, two row tiles
    (3, 8, 8, 128, 5000, 5000),    # several key ranges
    (16, 24, 4, 256, 90, 96),      # 96 rows per KV head
])
@pytest.mark.parametrize("tree", [False, True])
def test_int8_attention(vq, M, Hq, Hkv, D, T, T_cap, tree):
    q, kc, ks, vc, vs = _oracle_cache(40 + M, M, Hq, Hkv, D, T_cap)
    mask = tree_masks(40, M, extra=T) if tree else None
    scale = 1 / math.sqrt(D)
    k8, kw = _dev_cache(kc, ks)
    v8, vw = _dev_cache(vc, vs)
    out = vq.multirow_attn_int8(bf16_tensor(q), k8, kw, v8, vw, T, scale,
                                tree_mask=None if mask is None else _mask_tensor(mask))
    torch.cuda.synchronize()
    ref = okv.int8_attention(q, kc, ks, vc, vs, M, Hq, Hkv, D, T, T_cap, scale, mask=mask)
    assert_close(to_f64(out), ref, f"int8 M={M} Hq={Hq} Hkv={Hkv} D={D} T={T} tree={tree}")


def test_int8_grid_equals_bf16(vq):
    """On a cache whose values are exact on the quantization grid, the dequantized
    tiles equal the bf16 tiles, so the int8 call returns the bf16 call's output bit
    for bit (causal and tree)."""
    M, Hq, Hkv, D, T = 8, 24, 4, 256, 3000
    q = attn_inputs(41, M, Hq, Hkv, D, T)[0]
    kb, _, _ = _grid_rows(4, (Hkv, T, D), step_exp=-7)
    vb, _, _ = _grid_rows(5, (Hkv, T, D), step_exp=-6)
    kc, ks = okv.quantize_rows(kb)
    vc, vs = okv.quantize_rows(vb)
    k8, kw = _dev_cache(kc, ks)
    v8, vw = _dev_cache(vc, vs)
    for mask in (None, tree_masks(41, M)):
        mt = None if mask is None else _mask_tensor(mask)
        a = vq.multirow_attn_int8(bf16_tensor(q), k8, kw, v8, vw, T, 0.0625, tree_mask=mt)
        b = vq.multirow_attn(bf16_tensor(q), bf16_tensor(kb), bf16_tensor(vb), T, 0.0625, tree_mask=mt)
        torch.cuda.synchronize()
        assert torch.equal(a, b)


def test_int8_append_then_attention(vq):
    """The verify step's order on an 8-bit cache: quantize the M new rows in, then attend over T keys."""
    M, Hq, Hkv, D, ctx = 4, 24, 4, 256, 2048
    T = ctx + M
    q, kc, ks, vc, vs = _oracle_cache(42, M, Hq, Hkv, D, T)
    from synth import f32_to_bf16_bits
    rows = f32_to_bf16_bits(np.random.default_rng(42).standard_normal((M, 2 * Hkv * D)).astype(np.float32))
    k8, kw = _dev_cache(kc, ks)
    v8, vw = _dev_cache(vc, vs)
    vq.kv8_append(bf16_tensor(rows), 0, Hkv * D, k8, kw, v8, vw, ctx)
    out = vq.multirow_attn_int8(bf16_tensor(q), k8, kw, v8, vw, T, 1 / 16)
    torch.cuda.synchronize()
    nk = okv.quantize_rows(rows[:, : Hkv * D].reshape(M, Hkv, D).transpose(1, 0, 2))
    nv = okv.quantize_rows(rows[:, Hkv * D:].reshape(M, Hkv, D).transpose(1, 0, 2))
    kc[:, ctx:], ks[:, ctx:] = nk
    vc[:, ctx:], vs[:, ctx:] = nv
    ref = okv.int8_attention(q, kc, ks, vc, vs, M, Hq, Hkv, D, T, T, 1 / 16)
    assert_close(to_f64(out), ref, "append then attention")


def test_int8_config_sampled(vq):
    """27B heads, 16k committed positions + 8 drafted rows: sampled pairs against the oracle."""
    M, Hq, Hkv, D, ctx = 8, 24, 4, 256, 16384
    T = ctx + M
    q, kc, ks, vc, vs = _oracle_cache(43, M, Hq, Hkv, D, T)
    k8, kw = _dev_cache(kc, ks)
    v8, vw = _dev_cache(vc, vs)
    out = to_f64(vq.multirow_attn_int8(bf16_tensor(q), k8, kw, v8, vw, T, 1 / 16))
    rng = np.random.default_rng(43)
    pairs = [(m, int(h)) for m in range(M) for h in rng.choice(Hq, 2, replace=False)]
    ref = okv.int8_attention(q, kc, ks, vc, vs, M, Hq, Hkv, D, T, T, 1 / 16, pairs=pairs)
    assert_close(np.stack([out[m, h] for m, h in pairs]), ref, "int8 at 16k")


@pytest.mark.parametrize("M,Hq,D", [(4, 32, 64), (16, 128, 64), (4, 32, 128), (8, 96, 128), (16, 80, 128),
                                    (16, 128, 128)])
def test_int8_long_ranges(vq, M, Hq, D):
    """Ten tiles per key range (16 KV heads): the unconditional main loop and
    the tested tail both run; every row of the last KV head compared."""
    Hkv, T = 16, 5000 + M
    q, kc, ks, vc, vs = _oracle_cache(70 + M, M, Hq, Hkv, D, T)
    scale = 1 / math.sqrt(D)
    k8, kw = _dev_cache(kc, ks)
    v8, vw = _dev_cache(vc, vs)
    out = to_f64(vq.multirow_attn_int8(bf16_tensor(q), k8, kw, v8, vw, T, scale))
    torch.cuda.synchronize()
    G = Hq // Hkv
    # The oracle on the last KV head alone (heads are independent).
    ref = okv.int8_attention(np.ascontiguousarray(q[:, Hq - G:]), kc[Hkv - 1:], ks[Hkv - 1:], vc[Hkv - 1:],
                             vs[Hkv - 1:], M, G, 1, D, T, T, scale)
    assert_close(out[:, Hq - G:], ref, f"int8 long ranges M={M} Hq={Hq} D={D}")
