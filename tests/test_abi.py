"""The C-ABI library without a GPU: it loads, exports every declared symbol, and
rejects invalid arguments on the host before any HIP call."""
import ctypes
import glob
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def vqmod():
    from speculative_decoding_verify_vq_amd import vq
    return vq


def _declared():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        src = open(h).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        names |= set(re.findall(r"\b(vq_\w+)\s*\(", src))
    return sorted(names)


def test_every_declared_symbol_exported(vqmod):
    names = _declared()
    assert len(names) >= 13
    for n in names:
        assert hasattr(vqmod.lib, n), n


def test_status_strings(vqmod):
    assert vqmod.status_string(0) == "ok"
    assert vqmod.status_string(1) == "invalid argument"
    assert vqmod.version() == "0.1.0"


A16 = 1 << 20  # a fake, 256-byte-aligned "device address": never dereferenced (validation fails first)


def _qmm(vq, **kw):
    a = dict(x=A16, ldx=1024, wq=A16, s=A16, b=A16, bits=4, gs=64, M=4, N=512, K=1024, y=A16, ldy=512,
             yd=0, ws=A16, wsz=1 << 30, stream=None)
    a.update(kw)
    return vq.lib.vq_skinny_qmm(a["x"], a["ldx"], a["wq"], a["s"], a["b"], a["bits"], a["gs"], a["M"], a["N"],
                                a["K"], a["y"], a["ldy"], a["yd"], a["ws"], a["wsz"], a["stream"])


@pytest.mark.parametrize("bad", [
    dict(x=None), dict(wq=None), dict(y=None), dict(bits=3), dict(bits=16), dict(gs=32), dict(M=0), dict(M=17),
    dict(N=0), dict(K=96), dict(K=0), dict(ldx=1000), dict(ldx=1028), dict(ldy=100), dict(yd=7),
    dict(x=A16 + 8), dict(wq=A16 + 4), dict(y=A16 + 1), dict(ws=None, N=64, K=8192), dict(wsz=16, N=64, K=8192),
    dict(ws=A16 + 64, N=64, K=8192),
])
def test_qmm_rejects(vqmod, bad):
    assert _qmm(vqmod, **bad) == vqmod.VQ_ERR_INVALID_ARG
    assert vqmod.last_error()


def _qmm_noalloc(vq, **kw):
    a = dict(x=A16, ldx=1024, wq=A16, s=A16, b=A16, bits=4, gs=64, M=4, N=512, K=1024, y=A16, ldy=512, yd=0,
             stream=None)
    a.update(kw)
    return vq.lib.vq_skinny_qmm_noalloc(a["x"], a["ldx"], a["wq"], a["s"], a["b"], a["bits"], a["gs"], a["M"],
                                        a["N"], a["K"], a["y"], a["ldy"], a["yd"], a["stream"])


@pytest.mark.parametrize("bad", [
    dict(x=None), dict(wq=None), dict(y=None), dict(bits=3), dict(gs=32), dict(M=0), dict(M=17), dict(N=0),
    dict(K=96), dict(ldx=1000), dict(ldy=100), dict(yd=7), dict(x=A16 + 8), dict(y=A16 + 1),
    dict(M=16, N=248320, K=5120, ldx=5120, ldy=248320), dict(M=4, N=248320, K=5120, ldx=5120, ldy=248320),
])
def test_qmm_noalloc_rejects(vqmod, bad):
    """Invalid arguments, and shapes whose scratch exceeds the library's 16 MiB
    array, are rejected on the host before anything is launched."""
    assert _qmm_noalloc(vqmod, **bad) == vqmod.VQ_ERR_INVALID_ARG
    assert vqmod.last_error()
    if "N" in bad and bad["N"] == 248320:
        assert "scratch" in vqmod.last_error()
        assert vqmod.lib.vq_skinny_qmm_workspace(4, 64, bad["M"], bad["N"], bad["K"]) > (16 << 20)


def test_qmm_noalloc_limit_covers_layer_projections(vqmod):
    """Every projection of a 27B-shaped layer (fused q|k|v and gate|up included)
    fits the no-allocation scratch at every verify width up to 16."""
    for N, K in ((8192, 5120), (5120, 6144), (34816, 5120), (5120, 17408)):
        for M in (1, 4, 8, 16):
            for bits in (4, 8):
                assert vqmod.lib.vq_skinny_qmm_workspace(bits, 64, M, N, K) <= (16 << 20)


def _attn(vq, **kw):
    a = dict(q=A16, qrs=128, k=A16, v=A16, hs=256 * 64, M=4, Hq=2, Hkv=2, D=64, T=256, scale=0.125, out=A16,
             ors=128, ws=A16, wsz=1 << 30)
    a.update(kw)
    return vq.lib.vq_multirow_attn(a["q"], a["qrs"], a["k"], a["v"], a["hs"], a["M"], a["Hq"], a["Hkv"], a["D"],
                                   a["T"], a["scale"], a["out"], a["ors"], a["ws"], a["wsz"], None)


@pytest.mark.parametrize("bad", [
    dict(q=None), dict(out=None), dict(M=0), dict(M=17), dict(Hq=3), dict(Hkv=0), dict(D=96), dict(T=3),
    dict(hs=256 * 64 - 8), dict(hs=256 * 64 + 4), dict(scale=float("inf")), dict(scale=float("nan")),
    dict(q=A16 + 2), dict(Hq=48, Hkv=1, M=4), dict(T=100000, ws=None), dict(qrs=120), dict(qrs=132),
    dict(ors=64),
])
def test_attn_rejects(vqmod, bad):
    assert _attn(vqmod, **bad) == vqmod.VQ_ERR_INVALID_ARG


def _acc(vq, **kw):
    a = dict(p=A16, q=A16, kind=0, ps=0, qs=0, d=A16, u=A16, B=4, K=3, V=1000, T=1.0, tk=0, tp=1.0, ot=A16,
             on=A16, po=None, ws=A16, wsz=1 << 30)
    a.update(kw)
    return vq.lib.vq_spec_accept(a["p"], a["q"], a["kind"], a["ps"], a["qs"], a["d"], a["u"], a["B"], a["K"],
                                 a["V"], a["T"], a["tk"], a["tp"], a["ot"], a["on"], a["po"], a["ws"], a["wsz"], None)


@pytest.mark.parametrize("bad", [
    dict(p=None), dict(u=None), dict(ot=None), dict(on=None), dict(q=None), dict(d=None), dict(B=0), dict(K=-1),
    dict(K=16), dict(V=1), dict(V=(1 << 20) + 1), dict(kind=2), dict(tk=-1), dict(tp=0.0), dict(tp=1.5),
    dict(tp=float("nan")), dict(kind=1, T=0.0), dict(kind=1, T=float("inf")), dict(ps=3999), dict(qs=10),
    dict(ps=-1), dict(ps=4000, qs=3000, B=70000), dict(p=A16 + 2), dict(ws=None),
])
def test_accept_rejects(vqmod, bad):
    assert _acc(vqmod, **bad) == vqmod.VQ_ERR_INVALID_ARG


def test_valid_call_without_gpu_is_a_clean_error(vqmod):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    rc = _qmm(vqmod)
    assert rc in (vqmod.VQ_ERR_HIP, vqmod.VQ_ERR_UNSUPPORTED_DEVICE) and vqmod.last_error()


def test_workspace_queries_are_pure(vqmod):
    vq = vqmod
    assert vq.qmm_workspace_bytes(4, 4, 8192, 5120) == vq.qmm_workspace_bytes(4, 4, 8192, 5120) > 0
    assert vq.qmm_workspace_bytes(4, 4, 8192, 96) == 0          # invalid shape -> 0
    assert vq.attn_workspace_bytes(4, 2, 2, 64, 256) >= 0
    assert vq.accept_workspace_bytes(1, 3, 1000, 0, 0, 0) > 0
    assert vq.accept_workspace_bytes(1, 3, 1000, 1, 0, 0) > vq.accept_workspace_bytes(1, 3, 1000, 0, 0, 0)


def _packed(vq, **kw):
    a = dict(x=A16, ldx=1024, ss=None, parts=0, eps=1e-6, pk=A16, bits=4, gs=64, M=4, N=512, K=1024, epi=0,
             r=None, ldr=0, y=A16, ldy=512, yd=0, yss=None, ws=A16, wsz=1 << 30)
    a.update(kw)
    return vq.lib.vq_qmm_packed(a["x"], a["ldx"], a["ss"], a["parts"], a["eps"], a["pk"], a["bits"], a["gs"],
                                a["M"], a["N"], a["K"], a["epi"], a["r"], a["ldr"], a["y"], a["ldy"], a["yd"],
                                a["yss"], a["ws"], a["wsz"], None)


@pytest.mark.parametrize("bad", [
    dict(x=None), dict(pk=None), dict(y=None), dict(bits=2), dict(gs=128), dict(M=0), dict(M=17), dict(K=100),
    dict(ldx=1020), dict(x=A16 + 8), dict(pk=A16 + 8), dict(ss=A16, parts=0), dict(ss=A16, parts=257),
    dict(ss=A16, parts=4, eps=-1.0), dict(ss=A16, parts=4, eps=float("nan")), dict(ss=A16 + 2, parts=4),
    dict(epi=3), dict(epi=-1), dict(yd=5), dict(ldy=100), dict(yss=A16),
    dict(epi=1), dict(epi=1, r=A16, ldr=100), dict(epi=1, r=A16, ldr=512, yd=1), dict(epi=1, r=A16, ldr=1024),
    dict(epi=1, r=A16 + 1, ldr=512), dict(epi=1, r=A16, ldr=512, yss=A16 + 2),
    dict(epi=2, N=500), dict(epi=2, ldy=100), dict(epi=2, yd=1), dict(epi=2, yss=A16),
    dict(ws=None, N=64, K=8192), dict(wsz=16, N=64, K=8192),
])
def test_packed_rejects(vqmod, bad):
    assert _packed(vqmod, **bad) == vqmod.VQ_ERR_INVALID_ARG
    assert vqmod.last_error()


@pytest.mark.parametrize("bad", [
    dict(wq=None), dict(out=None), dict(bits=5), dict(gs=32), dict(K=70), dict(N=0), dict(nbytes=16),
    dict(wq=A16 + 4), dict(out=A16 + 8),
])
def test_pack_rejects(vqmod, bad):
    a = dict(wq=A16, s=A16, b=A16, bits=4, gs=64, N=512, K=1024, out=A16, nbytes=1 << 30)
    a.update(bad)
    rc = vqmod.lib.vq_qmm_pack(a["wq"], a["s"], a["b"], a["bits"], a["gs"], a["N"], a["K"], a["out"], a["nbytes"],
                               None)
    assert rc == vqmod.VQ_ERR_INVALID_ARG


def test_pack_sizes(vqmod):
    vq = vqmod
    # 4-bit: 32-row tiles x 256-input blocks of 4608 bytes; 8-bit: 128-input blocks of 4352 bytes
    assert vq.qmm_pack_bytes(4, 512, 1024) == 16 * 4 * 4608
    assert vq.qmm_pack_bytes(4, 500, 1088) == 16 * 5 * 4608      # ragged N and K are zero-padded
    assert vq.qmm_pack_bytes(8, 512, 1024) == 16 * 8 * 4352
    assert vq.qmm_pack_bytes(4, 512, 100) == 0
    assert vq.sumsq_parts(5120) == 40 and vq.sumsq_parts(129) == 2
    assert vq.qmm_packed_workspace_bytes(4, 4, 8192, 5120) > 0


@pytest.mark.parametrize("bad", [
    dict(kn=None), dict(vn=None), dict(nrs=100), dict(nrs=132), dict(kn=A16 + 8), dict(q=None), dict(T=3),
    dict(hs=256 * 64 - 8), dict(scale=float("nan")), dict(ws=None, T=100000),
])
def test_attn_append_rejects(vqmod, bad):
    a = dict(q=A16, qrs=128, kn=A16, vn=A16, nrs=128, k=A16, v=A16, hs=256 * 64, M=4, Hq=2, Hkv=2, D=64, T=256,
             scale=0.125, out=A16, ors=128, ws=A16, wsz=1 << 30)
    a.update(bad)
    rc = vqmod.lib.vq_multirow_attn_append(a["q"], a["qrs"], a["kn"], a["vn"], a["nrs"], a["k"], a["v"], a["hs"],
                                           a["M"], a["Hq"], a["Hkv"], a["D"], a["T"], a["scale"], a["out"],
                                           a["ors"], a["ws"], a["wsz"], None)
    assert rc == vqmod.VQ_ERR_INVALID_ARG


@pytest.mark.parametrize("bad", [
    dict(mask=None), dict(mask=A16 + 2), dict(kn=None), dict(vn=None), dict(nrs=100), dict(q=None), dict(T=3),
    dict(scale=float("inf")), dict(ws=None, T=100000), dict(M=17),
])
def test_attn_tree_rejects(vqmod, bad):
    a = dict(q=A16, qrs=128, kn=A16, vn=A16, nrs=128, k=A16, v=A16, hs=256 * 64, M=4, Hq=2, Hkv=2, D=64, T=256,
             scale=0.125, mask=A16, out=A16, ors=128, ws=A16, wsz=1 << 30)
    a.update(bad)
    rc = vqmod.lib.vq_multirow_attn_tree(a["q"], a["qrs"], a["kn"], a["vn"], a["nrs"], a["k"], a["v"], a["hs"],
                                         a["M"], a["Hq"], a["Hkv"], a["D"], a["T"], a["scale"], a["mask"], a["out"],
                                         a["ors"], a["ws"], a["wsz"], None)
    assert rc == vqmod.VQ_ERR_INVALID_ARG
    assert "vq_multirow_attn_tree" in vqmod.last_error()


@pytest.mark.parametrize("bad", [
    dict(ks=None), dict(vs=None), dict(ks=A16 + 2), dict(mask=A16 + 2), dict(kc=None), dict(kc=A16 + 8),
    dict(hs=256 * 64 + 8), dict(hs=100 * 64), dict(M=0), dict(D=96), dict(ws=None, T=100000),
])
def test_attn_int8_rejects(vqmod, bad):
    a = dict(q=A16, qrs=128, kc=A16, ks=A16, vc=A16, vs=A16, hs=256 * 64, M=4, Hq=2, Hkv=2, D=64, T=256,
             scale=0.125, mask=None, out=A16, ors=128, ws=A16, wsz=1 << 30)
    a.update(bad)
    rc = vqmod.lib.vq_multirow_attn_int8(a["q"], a["qrs"], a["kc"], a["ks"], a["vc"], a["vs"], a["hs"], a["M"],
                                         a["Hq"], a["Hkv"], a["D"], a["T"], a["scale"], a["mask"], a["out"],
                                         a["ors"], a["ws"], a["wsz"], None)
    assert rc == vqmod.VQ_ERR_INVALID_ARG
    assert "vq_multirow_attn_int8" in vqmod.last_error()


@pytest.mark.parametrize("bad", [
    dict(src=None), dict(kc=None), dict(vs=None), dict(M=0), dict(M=17), dict(D=96), dict(pos=-1),
    dict(ld=100), dict(hs=256 * 64 + 8), dict(hs=64 * 3), dict(ks=A16 + 2),
])
def test_kv8_append_rejects(vqmod, bad):
    a = dict(src=A16, ld=512, ko=0, vo=128, kc=A16, ks=A16, vc=A16, vs=A16, hs=256 * 64, M=4, Hkv=2, D=64, pos=10)
    a.update(bad)
    rc = vqmod.lib.vq_kv8_append(a["src"], a["ld"], a["ko"], a["vo"], a["kc"], a["ks"], a["vc"], a["vs"], a["hs"],
                                 a["M"], a["Hkv"], a["D"], a["pos"], None)
    assert rc == vqmod.VQ_ERR_INVALID_ARG


@pytest.mark.parametrize("bad", [
    dict(rs=None), dict(sl=None), dict(rs=A16 + 2), dict(B=0), dict(B=4097), dict(R=0), dict(mr=17), dict(mr=0),
    dict(bs=256 * 64), dict(bs=2 * 256 * 64 + 4), dict(kn=None), dict(mask=A16 + 1), dict(T=3), dict(ws=None, T=100000),
])
def test_attn_batched_rejects(vqmod, bad):
    a = dict(q=A16, qrs=128, rs=A16, sl=A16, B=3, R=12, mr=4, T=256, kn=A16, vn=A16, nrs=128, k=A16, v=A16,
             bs=2 * 256 * 64, hs=256 * 64, Hq=2, Hkv=2, D=64, scale=0.125, mask=None, out=A16, ors=128, ws=A16,
             wsz=1 << 30)
    a.update(bad)
    rc = vqmod.lib.vq_multirow_attn_batched(a["q"], a["qrs"], a["rs"], a["sl"], a["B"], a["R"], a["mr"], a["T"],
                                            a["kn"], a["vn"], a["nrs"], a["k"], a["v"], a["bs"], a["hs"], a["Hq"],
                                            a["Hkv"], a["D"], a["scale"], a["mask"], a["out"], a["ors"], a["ws"],
                                            a["wsz"], None)
    assert rc == vqmod.VQ_ERR_INVALID_ARG
    assert "vq_multirow_attn_batched" in vqmod.last_error()


def test_batched_workspace_grows_with_sequences(vqmod):
    one = vqmod.lib.vq_multirow_attn_batched_workspace(1, 4, 24, 4, 256, 16388)
    assert one == vqmod.attn_workspace_bytes(4, 24, 4, 256, 16388)
    assert vqmod.lib.vq_multirow_attn_batched_workspace(4, 4, 24, 4, 256, 16388) > 0
    assert vqmod.lib.vq_multirow_attn_batched_workspace(0, 4, 24, 4, 256, 16388) == 0
