"""GPU parity of the tiled pack and of vq_qmm_packed (store, residual and SwiGLU
epilogues, RMSNorm prologue) against the float64 oracle, and bit-level
agreement with the row-major path where the arithmetic order is the same."""
import numpy as np
import pytest
import torch

import oracle.qmm as oq
import oracle.stack as ostack
from synth import qmm_activations, qmm_weights
from tests.gpu_util import assert_close, bf16_tensor, dev, interleave_gate_up, to_f64, words_tensor

pytestmark = pytest.mark.gpu


def _dev_w(w):
    return words_tensor(w["wq"]), bf16_tensor(w["scales"]), bf16_tensor(w["biases"])


def _pack(vq, w):
    wq, s, b = _dev_w(w)
    p = vq.qmm_pack(wq, s, b, w["bits"], w["N"], w["K"])
    torch.cuda.synchronize()
    return p


def _expected_pack(w) -> np.ndarray:
    """The tiled layout built from its definition: per 32-row tile and per block of
    128 code bytes per row, the 32 x 128 code bytes as 256 units of 16 bytes, unit
    64j + l holding bytes 16(2j + l // 32) .. +16 of row l % 32 (the order in which
    lane l of a wave receives them from its j-th 16-byte load), then per row the
    block's scales and then its biases (4 + 4 bf16 for 4-bit, 2 + 2 for 8-bit)."""
    N, K, bits = w["N"], w["K"], w["bits"]
    G = K // 64
    GB = 4 if bits == 4 else 2
    KB = -(-G // GB)
    tiles = -(-N // 32)
    row_bytes = K * bits // 8
    codes = np.zeros((tiles * 32, KB * 128), dtype=np.uint8)
    codes[:N, :row_bytes] = np.asarray(w["wq"], dtype=np.uint32).view(np.uint8).reshape(N, row_bytes)
    s = np.zeros((tiles * 32, KB * GB), dtype=np.uint16)
    b = np.zeros((tiles * 32, KB * GB), dtype=np.uint16)
    s[:N, :G] = np.asarray(w["scales"]).reshape(N, G)
    b[:N, :G] = np.asarray(w["biases"]).reshape(N, G)
    out = []
    for t in range(tiles):
        rows = slice(32 * t, 32 * t + 32)
        for kb in range(KB):
            blk = codes[rows, 128 * kb: 128 * kb + 128].reshape(32, 8, 16)   # [row, 16-byte chunk, byte]
            units = [blk[l % 32, 2 * j + l // 32] for j in range(4) for l in range(64)]
            out.append(np.concatenate(units))
            sb = np.concatenate([s[rows, GB * kb: GB * kb + GB], b[rows, GB * kb: GB * kb + GB]], axis=1)
            out.append(np.ascontiguousarray(sb).view(np.uint8).reshape(-1))
    return np.concatenate(out)


@pytest.mark.parametrize("bits,N,K", [(4, 500, 1088), (8, 70, 320), (4, 64, 64), (8, 33, 1024)])
def test_pack_layout_exact(vq, bits, N, K):
    w = qmm_weights(21, N, K, bits, layer=K)
    got = _pack(vq, w).cpu().numpy()
    exp = _expected_pack(w)
    assert got.shape == exp.shape == (vq.qmm_pack_bytes(bits, N, K),)
    assert np.array_equal(got, exp)


def _packed(vq, w, x_bits, **kw):
    x = bf16_tensor(x_bits)
    y = vq.qmm_packed(x, _pack(vq, w), w["bits"], w["N"], w["K"], **kw)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("M", [1, 2, 4, 7, 8, 9, 12, 16])
def test_packed_store_config0(vq, bits, M):
    w = qmm_weights(0, 512, 1024, bits)
    x = qmm_activations(0, M, 1024)
    ref = oq.skinny_qmm(x, w["wq"], w["scales"], w["biases"], bits, 64, M, 512, 1024)
    assert_close(to_f64(_packed(vq, w, x)), ref, f"packed bits={bits} M={M}")


@pytest.mark.parametrize("bits,M,N,K", [
    (4, 3, 200, 64 * 3),        # ragged N, G not a multiple of the block (zero-padded groups)
    (4, 5, 33, 64 * 17),
    (8, 7, 130, 64 * 21),       # odd G for 8-bit blocks of two groups
    (4, 16, 256, 8192),         # many K splits
    (8, 9, 96, 8192),
    (4, 1, 4000, 64),
    (8, 12, 1000, 1088),
    (4, 4, 65536, 512),         # one K split (no cross-workgroup reduction)
    # plan rules for long K: narrow outputs take full 16-group ranges (ragged last
    # range), wider ones at least three blocks per range
    (4, 4, 300, 64 * 97),
    (8, 8, 5120, 64 * 75),
    (4, 4, 8256, 64 * 70),
])
def test_packed_store_ragged(vq, bits, M, N, K):
    w = qmm_weights(11, N, K, bits, layer=N)
    x = qmm_activations(11, M, K, extra=K)
    ref = oq.skinny_qmm(x, w["wq"], w["scales"], w["biases"], bits, 64, M, N, K)
    assert_close(to_f64(_packed(vq, w, x)), ref, f"{bits}-bit M={M} N={N} K={K}")
    assert_close(to_f64(_packed(vq, w, x, out_dtype=torch.float32)), ref, "f32 out")


@pytest.mark.parametrize("bits,M,N,K", [(4, 4, 512, 8192), (8, 8, 384, 4096), (4, 16, 8192, 1024)])
def test_packed_matches_row_major_bits(vq, bits, M, N, K):
    """Same split plan and arithmetic order as the row-major path when K / 64 is a
    multiple of 4: identical float32 results."""
    w = qmm_weights(13, N, K, bits)
    x = qmm_activations(13, M, K)
    a = _packed(vq, w, x, out_dtype=torch.float32)
    wq, s, b = _dev_w(w)
    r = vq.skinny_qmm(bf16_tensor(x), wq, s, b, bits, N, K, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(a, r)


@pytest.mark.parametrize("bits,M,N,K", [(4, 4, 5120, 6144), (8, 3, 200, 192), (4, 12, 65536, 512),
                                        (4, 16, 640, 17408),
                                        # 512 column blocks: the unsplit chunked path at 4 and 8 rows
                                        (4, 4, 65536, 512), (8, 8, 65536, 1024)])
@pytest.mark.parametrize("inplace", [False, True])
def test_residual_epilogue(vq, bits, M, N, K, inplace):
    w = qmm_weights(14, N, K, bits)
    x = qmm_activations(14, M, K)
    r_bits = qmm_activations(15, M, N)
    # the unfused composition on the device: bf16 product, then a float32 add rounded to bf16
    wq, s, b = _dev_w(w)
    p = vq.skinny_qmm(bf16_tensor(x), wq, s, b, bits, N, K)
    torch.cuda.synchronize()
    r = to_f64(bf16_tensor(r_bits))
    expect = ostack.round_bf16((r.astype(np.float32) + to_f64(p).astype(np.float32)).astype(np.float64))
    res = bf16_tensor(r_bits)
    out = res if inplace else None
    parts = vq.sumsq_parts(N)
    ss = torch.full((M, parts), float("nan"), dtype=torch.float32, device=dev())
    y = _packed(vq, w, x, epilogue=vq.VQ_EPI_RESIDUAL, residual=res, out=out, y_sumsq=ss)
    got = to_f64(y)
    assert np.array_equal(got, expect), f"max diff {np.abs(got - expect).max()}"
    # against the oracle: residual + rounded product
    ref = ostack.round_bf16(r + ostack.round_bf16(oq.skinny_qmm(x, w["wq"], w["scales"], w["biases"], bits, 64,
                                                                 M, N, K)))
    assert_close(got, ref, "residual vs oracle")
    # sums of squares of the stored rows per 128 columns
    pad = np.zeros((M, parts * 128))
    pad[:, :N] = got
    ss_ref = (pad.reshape(M, parts, 128) ** 2).sum(axis=2)
    np.testing.assert_allclose(ss.cpu().numpy(), ss_ref, rtol=1e-5, atol=1e-30)


@pytest.mark.parametrize("bits,M,I,K", [(4, 4, 1024, 1024), (8, 8, 320, 2048), (4, 16, 32768, 512),
                                        (4, 1, 64, 5120),
                                        # 512 column blocks: the unsplit chunked path at 4 and 8 rows
                                        (4, 4, 32768, 512), (8, 8, 32768, 1024)])
def test_swiglu_epilogue(vq, bits, M, I, K):
    wg = qmm_weights(16, I, K, bits, layer=0)
    wu = qmm_weights(16, I, K, bits, layer=1)
    w = interleave_gate_up(wg, wu)
    x = qmm_activations(16, M, K)
    y = to_f64(_packed(vq, w, x, epilogue=vq.VQ_EPI_SWIGLU))
    assert y.shape == (M, I)
    g = ostack.round_bf16(oq.skinny_qmm(x, wg["wq"], wg["scales"], wg["biases"], bits, 64, M, I, K))
    u = ostack.round_bf16(oq.skinny_qmm(x, wu["wq"], wu["scales"], wu["biases"], bits, 64, M, I, K))
    ref = ostack.round_bf16(ostack.silu_mul(g, u))
    assert_close(y, ref, "swiglu vs oracle")
    # and against the unfused device path on the same interleaved rows
    wq, s, b = _dev_w(w)
    gu = vq.skinny_qmm(bf16_tensor(x), wq, s, b, bits, 2 * I, K)
    gu = gu.view(M, I // 64, 2, 64)
    gate = gu[:, :, 0, :].reshape(M, I)
    up = gu[:, :, 1, :].reshape(M, I)
    unf = vq.silu_mul(torch.cat([gate, up], dim=1).contiguous())
    torch.cuda.synchronize()
    d = np.abs(y - to_f64(unf))
    assert float(d.max()) <= 2.0 ** -7 * float(np.abs(to_f64(unf)).max()), "fused vs unfused SwiGLU"


def test_row_sumsq(vq):
    xb = qmm_activations(17, 5, 1000)
    got = vq.row_sumsq(bf16_tensor(xb)).cpu().numpy()
    x = to_f64(bf16_tensor(xb))
    pad = np.zeros((5, 8 * 128))
    pad[:, :1000] = x
    np.testing.assert_allclose(got, (pad.reshape(5, 8, 128) ** 2).sum(axis=2), rtol=1e-5)


@pytest.mark.parametrize("bits,M,N,K", [(4, 4, 2048, 5120), (8, 16, 512, 1024), (4, 1, 300, 256)])
def test_rmsnorm_prologue(vq, bits, M, N, K):
    w = qmm_weights(18, N, K, bits)
    hb = qmm_activations(18, M, K)
    h = bf16_tensor(hb)
    ss = vq.row_sumsq(h)
    y = to_f64(_packed(vq, w, hb, x_sumsq=ss, eps=1e-6))
    a = ostack.to_bf16_bits(ostack.rmsnorm(to_f64(h)))
    ref = oq.skinny_qmm(a, w["wq"], w["scales"], w["biases"], bits, 64, M, N, K)
    assert_close(y, ref, "rmsnorm prologue vs oracle")


def test_residual_then_norm_chain(vq):
    """h1 = h0 + W1 x (sums of squares written by the epilogue), then W2 rms(h1)."""
    M, H, K1 = 4, 1024, 2048
    w1 = qmm_weights(19, H, K1, 4, layer=0)
    w2 = qmm_weights(19, 512, H, 4, layer=1)
    xb = qmm_activations(19, M, K1)
    h0b = qmm_activations(20, M, H)
    h = bf16_tensor(h0b)
    ss = torch.empty((M, vq.sumsq_parts(H)), dtype=torch.float32, device=dev())
    _packed(vq, w1, xb, epilogue=vq.VQ_EPI_RESIDUAL, residual=h, out=h, y_sumsq=ss)
    y = to_f64(vq.qmm_packed(h, _pack(vq, w2), 4, 512, H, x_sumsq=ss, eps=1e-6))
    h1 = ostack.round_bf16(to_f64(bf16_tensor(h0b)) + ostack.round_bf16(
        oq.skinny_qmm(xb, w1["wq"], w1["scales"], w1["biases"], 4, 64, M, H, K1)))
    a = ostack.to_bf16_bits(ostack.rmsnorm(h1))
    ref = oq.skinny_qmm(a, w2["wq"], w2["scales"], w2["biases"], 4, 64, M, 512, H)
    assert_close(y, ref, "residual -> rmsnorm chain")


@pytest.mark.parametrize("bits,M", [(4, 4), (8, 8), (4, 16), (8, 13)])
def test_wide_norm_residual(vq, bits, M):
    """RMSNorm prologue and residual epilogue together on an output wide enough for
    the unsplit chunked path (N = 65536: 512 column blocks), against the oracle."""
    N, K = 65536, 1024
    w = qmm_weights(17, N, K, bits, layer=M)
    xb = qmm_activations(17, M, K, extra=M)
    rb = qmm_activations(18, M, N, extra=M)
    x = bf16_tensor(xb)
    ss = vq.row_sumsq(x)
    a = ostack.to_bf16_bits(ostack.rmsnorm(to_f64(x)))
    y = to_f64(vq.qmm_packed(x, _pack(vq, w), bits, N, K, x_sumsq=ss, eps=1e-6, epilogue=vq.VQ_EPI_RESIDUAL,
                             residual=bf16_tensor(rb)))
    ref = ostack.round_bf16(to_f64(bf16_tensor(rb)) + ostack.round_bf16(
        oq.skinny_qmm(a, w["wq"], w["scales"], w["biases"], bits, 64, M, N, K)))
    assert_close(y, ref, f"{bits}-bit M={M} norm + residual")


@pytest.mark.parametrize("bits,M", [(4, 3), (8, 8), (4, 13), (8, 16)])
def test_chunked_walk_ragged(vq, bits, M):
    """The unsplit path (N = 65536: 512 column blocks) over K = 37 groups: the
    workgroup walks several chunks of x, the last one shorter than a chunk (and,
    at 4 bits, ending in zero-padded groups), with the RMSNorm prologue and
    float32 output, on sampled columns."""
    N, K = 65536, 64 * 37
    w = qmm_weights(19, N, K, bits, layer=M)
    xb = qmm_activations(19, M, K, extra=M)
    x = bf16_tensor(xb)
    ss = vq.row_sumsq(x)
    a = ostack.to_bf16_bits(ostack.rmsnorm(to_f64(x)))
    y = to_f64(vq.qmm_packed(x, _pack(vq, w), bits, N, K, x_sumsq=ss, eps=1e-6, out_dtype=torch.float32))
    c = np.unique(np.concatenate([np.random.default_rng(19 + M).choice(N, size=48, replace=False), [0, N - 1]]))
    ref = oq.skinny_qmm(a, w["wq"], w["scales"], w["biases"], bits, 64, M, N, K, cols=c)
    assert_close(y[:, c], ref, f"{bits}-bit M={M} chunked walk, K = 37 groups")


def test_packed_deterministic(vq):
    w = qmm_weights(22, 1024, 8192, 4)
    x = qmm_activations(22, 8, 8192)
    p = _pack(vq, w)
    xt = bf16_tensor(x)
    a = vq.qmm_packed(xt, p, 4, 1024, 8192, out_dtype=torch.float32)
    for _ in range(3):
        b = vq.qmm_packed(xt, p, 4, 1024, 8192, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(a, b)


@pytest.mark.parametrize("bits,M", [(4, 4), (8, 8), (4, 16), (8, 16)])
def test_step_projections_full_shape_sampled(vq, bits, M):
    """The five projections of the verify step at 27B shapes on the tiled pack, in
    the launch configuration of the step (RMSNorm prologue on q|k|v, gate|up and
    lm_head; residual epilogue on o and down; SwiGLU on gate|up; float32 lm_head
    logits, whose 1940 column blocks take the unsplit path), on sampled output
    columns that the oracle computes one by one."""
    H, I, V = 5120, 17408, 248320
    cfg = 3 if bits == 4 else 4
    rng = np.random.default_rng(100 + bits)

    def sample(n, k=40):
        return np.unique(np.concatenate([rng.choice(n, size=k, replace=False), [0, n - 1]]))

    def normed(seed):
        hb = qmm_activations(cfg, M, H, extra=seed)
        h = bf16_tensor(hb)
        return hb, h, vq.row_sumsq(h), ostack.to_bf16_bits(ostack.rmsnorm(to_f64(h)))

    # q|k|v with the RMSNorm prologue
    w = qmm_weights(cfg, 8192, H, bits, layer=0)
    hb, h, ss, a = normed(1)
    y = to_f64(vq.qmm_packed(h, _pack(vq, w), bits, 8192, H, x_sumsq=ss, eps=1e-6))
    c = sample(8192)
    assert_close(y[:, c], oq.skinny_qmm(a, w["wq"], w["scales"], w["biases"], bits, 64, M, 8192, H, cols=c), "qkv")
    del w

    # o and down with the residual epilogue (o: K = 6144; down: K = 17408)
    for name, K, layer in (("o", 6144, 1), ("down", I, 3)):
        w = qmm_weights(cfg, H, K, bits, layer=layer)
        xb = qmm_activations(cfg, M, K, extra=10 + layer)
        rb = qmm_activations(cfg, M, H, extra=20 + layer)
        res = bf16_tensor(rb)
        ss = torch.empty((M, vq.sumsq_parts(H)), dtype=torch.float32, device=dev())
        y = to_f64(vq.qmm_packed(bf16_tensor(xb), _pack(vq, w), bits, H, K, epilogue=vq.VQ_EPI_RESIDUAL,
                                 residual=res, y_sumsq=ss))
        c = sample(H)
        p = oq.skinny_qmm(xb, w["wq"], w["scales"], w["biases"], bits, 64, M, H, K, cols=c)
        ref = ostack.round_bf16(to_f64(bf16_tensor(rb))[:, c] + ostack.round_bf16(p))
        assert_close(y[:, c], ref, name)
        del w

    # gate|up with the RMSNorm prologue and the SwiGLU epilogue
    wg = qmm_weights(cfg, I, H, bits, layer=4)
    wu = qmm_weights(cfg, I, H, bits, layer=5)
    wi = interleave_gate_up(wg, wu)
    hb, h, ss, a = normed(2)
    y = to_f64(vq.qmm_packed(h, _pack(vq, wi), bits, 2 * I, H, x_sumsq=ss, eps=1e-6,
                             epilogue=vq.VQ_EPI_SWIGLU))
    del wi
    c = sample(I)
    g = ostack.round_bf16(oq.skinny_qmm(a, wg["wq"], wg["scales"], wg["biases"], bits, 64, M, I, H, cols=c))
    u = ostack.round_bf16(oq.skinny_qmm(a, wu["wq"], wu["scales"], wu["biases"], bits, 64, M, I, H, cols=c))
    assert_close(y[:, c], ostack.round_bf16(ostack.silu_mul(g, u)), "gate_up")
    del wg, wu

    # lm_head: RMSNorm prologue, float32 logits
    w = qmm_weights(cfg, V, H, bits, layer=999)
    hb, h, ss, a = normed(3)
    y = to_f64(vq.qmm_packed(h, _pack(vq, w), bits, V, H, x_sumsq=ss, eps=1e-6, out_dtype=torch.float32))
    c = sample(V, 64)
    assert_close(y[:, c], oq.skinny_qmm(a, w["wq"], w["scales"], w["biases"], bits, 64, M, V, H, cols=c), "lm_head")
