"""Python binding of the C ABI in include/vq.h and include/vq_glue.h.

Argument marshalling only: every computation runs in the HIP library
``libvq.so`` (built in-tree by ``python -m speculative_decoding_verify_vq_amd.build``).
PyTorch provides device memory and the current stream. Importing this module
fails loudly if the library has not been built; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# VQ_LIBRARY names another build of the same library (e.g. one with host-side
# sanitizers); by default the in-tree libvq.so.
LIB_PATH = os.environ.get("VQ_LIBRARY") or os.path.join(_HERE, "libvq.so")
if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m speculative_decoding_verify_vq_amd.build`")
lib = ctypes.CDLL(LIB_PATH)

VQ_OK, VQ_ERR_INVALID_ARG, VQ_ERR_HIP, VQ_ERR_UNSUPPORTED_DEVICE = 0, 1, 2, 3
VQ_BF16, VQ_F32 = 0, 1
VQ_PROBS, VQ_LOGITS = 0, 1
VQ_EPI_STORE, VQ_EPI_RESIDUAL, VQ_EPI_SWIGLU = 0, 1, 2

_c = ctypes
_P, _I, _I64, _F, _SZ = _c.c_void_p, _c.c_int, _c.c_int64, _c.c_float, _c.c_size_t


def _proto(name, res, args):
    fn = getattr(lib, name)
    fn.restype, fn.argtypes = res, args
    return fn


_proto("vq_status_string", _c.c_char_p, [_I])
_proto("vq_last_error", _c.c_char_p, [])
_proto("vq_version", _c.c_char_p, [])
_proto("vq_skinny_qmm_workspace", _SZ, [_I, _I, _I, _I, _I])
_proto("vq_skinny_qmm", _I, [_P, _I64, _P, _P, _P, _I, _I, _I, _I, _I, _P, _I64, _I, _P, _SZ, _P])
_proto("vq_skinny_qmm_noalloc", _I, [_P, _I64, _P, _P, _P, _I, _I, _I, _I, _I, _P, _I64, _I, _P])
_proto("vq_stream_read", _I, [_P, _SZ, _I, _I, _P, _P])
_proto("vq_qmm_pack_bytes", _SZ, [_I, _I, _I, _I])
_proto("vq_qmm_pack", _I, [_P, _P, _P, _I, _I, _I, _I, _P, _SZ, _P])
_proto("vq_sumsq_parts", _I, [_I])
_proto("vq_qmm_packed_workspace", _SZ, [_I, _I, _I, _I, _I])
_proto("vq_qmm_packed", _I, [_P, _I64, _P, _I, _F, _P, _I, _I, _I, _I, _I, _I, _P, _I64, _P, _I64, _I, _P, _P, _SZ,
                             _P])
_proto("vq_row_sumsq_bf16", _I, [_P, _I64, _I, _I, _P, _P])
_proto("vq_multirow_attn_workspace", _SZ, [_I, _I, _I, _I, _I])
_proto("vq_multirow_attn", _I, [_P, _I64, _P, _P, _I64, _I, _I, _I, _I, _I, _F, _P, _I64, _P, _SZ, _P])
_proto("vq_multirow_attn_append", _I, [_P, _I64, _P, _P, _I64, _P, _P, _I64, _I, _I, _I, _I, _I, _F, _P, _I64, _P,
                                       _SZ, _P])
_proto("vq_multirow_attn_tree", _I, [_P, _I64, _P, _P, _I64, _P, _P, _I64, _I, _I, _I, _I, _I, _F, _P, _P, _I64, _P,
                                     _SZ, _P])
_proto("vq_multirow_attn_int8", _I, [_P, _I64, _P, _P, _P, _P, _I64, _I, _I, _I, _I, _I, _F, _P, _P, _I64, _P, _SZ,
                                     _P])
_proto("vq_multirow_attn_batched_workspace", _SZ, [_I, _I, _I, _I, _I, _I])
_proto("vq_multirow_attn_batched", _I, [_P, _I64, _P, _P, _I, _I, _I, _I, _P, _P, _I64, _P, _P, _I64, _I64, _I, _I, _I,
                                        _F, _P, _P, _I64, _P, _SZ, _P])
_proto("vq_kv8_append", _I, [_P, _I64, _I, _I, _P, _P, _P, _P, _I64, _I, _I, _I, _I, _P])
_proto("vq_spec_accept_workspace", _SZ, [_I, _I, _I, _I, _I64, _I64])
_proto("vq_spec_accept", _I, [_P, _P, _I, _I64, _I64, _P, _P, _I, _I, _I, _F, _I, _F, _P, _P, _P, _P, _SZ, _P])
_proto("vq_rmsnorm_bf16", _I, [_P, _I64, _P, _I64, _I, _I, _F, _P])
_proto("vq_add_bf16", _I, [_P, _P, _P, _I64, _P])
_proto("vq_silu_mul_bf16", _I, [_P, _I64, _P, _I64, _I, _I, _P])
_proto("vq_kv_append_bf16", _I, [_P, _I64, _I, _I, _P, _P, _I64, _I, _I, _I, _I, _P])


class VQError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {status_string(status)}: {last_error()}")


def status_string(status: int) -> str:
    return lib.vq_status_string(status).decode()


def last_error() -> str:
    return lib.vq_last_error().decode()


def version() -> str:
    return lib.vq_version().decode()


def _check(fn: str, rc: int) -> None:
    if rc != VQ_OK:
        raise VQError(fn, rc)


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


# ------------------------------------------------------------------- workspace
class Workspace:
    """Zero-initialised scratch memory per device, grown on demand.

    The library leaves the completion counters of a workspace zero after every
    call, so one workspace serves any number of calls issued in stream order.
    Calls that may run concurrently need workspaces of their own.
    """

    def __init__(self):
        self._buf: dict[tuple, torch.Tensor] = {}
        self._lock = threading.Lock()

    def get(self, nbytes: int, device, kind: str) -> torch.Tensor | None:
        """A workspace of at least ``nbytes`` for operation ``kind`` on ``device``.

        Each operation kind keeps its own buffer: only calls of the same kind
        share the layout of counters and partial sums.
        """
        if nbytes == 0:
            return None
        dev = torch.device(device).index or 0
        key = (dev, kind)
        with self._lock:
            buf = self._buf.get(key)
            if buf is None or buf.numel() < nbytes + 256:
                size = max(nbytes, 2 * buf.numel() if buf is not None else 0)
                buf = torch.zeros(size + 256, dtype=torch.uint8, device=torch.device("cuda", dev))
                self._buf[key] = buf
            off = (-buf.data_ptr()) % 256
            return buf[off: off + nbytes]


_default_ws = Workspace()


def _ws(nbytes: int, device, workspace, kind: str):
    if workspace is not None:
        return workspace
    return _default_ws.get(nbytes, device, kind)


# ------------------------------------------------------------------------- QMM
def qmm_workspace_bytes(bits: int, M: int, N: int, K: int, group_size: int = 64) -> int:
    return int(lib.vq_skinny_qmm_workspace(bits, group_size, M, N, K))


def skinny_qmm(x: torch.Tensor, wq: torch.Tensor, scales: torch.Tensor, biases: torch.Tensor, bits: int,
               N: int, K: int, group_size: int = 64, out: torch.Tensor | None = None,
               out_dtype: torch.dtype = torch.bfloat16, workspace: torch.Tensor | None = None,
               stream=None) -> torch.Tensor:
    """y[M, N] = x[M, K] @ dequant(wq, scales, biases)^T (see include/vq.h)."""
    M = x.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=x.device)
    y_dtype = VQ_F32 if out.dtype == torch.float32 else VQ_BF16
    need = qmm_workspace_bytes(bits, M, N, K, group_size)
    ws = _ws(need, x.device, workspace, "qmm")
    wsz = 0 if ws is None else ws.numel() * ws.element_size()
    rc = lib.vq_skinny_qmm(x.data_ptr(), x.stride(0), wq.data_ptr(), scales.data_ptr(), biases.data_ptr(), bits,
                           group_size, M, N, K, out.data_ptr(), out.stride(0), y_dtype, _ptr(ws), wsz,
                           _stream(stream))
    _check("vq_skinny_qmm", rc)
    return out


def skinny_qmm_noalloc(x: torch.Tensor, wq: torch.Tensor, scales: torch.Tensor, biases: torch.Tensor, bits: int,
                       N: int, K: int, out: torch.Tensor, group_size: int = 64, stream=None) -> torch.Tensor:
    """skinny_qmm into a caller-given ``out`` with the library's own scratch
    (vq_skinny_qmm_noalloc: no workspace, nothing allocated in the call)."""
    M = x.shape[0]
    y_dtype = VQ_F32 if out.dtype == torch.float32 else VQ_BF16
    rc = lib.vq_skinny_qmm_noalloc(x.data_ptr(), x.stride(0), wq.data_ptr(), scales.data_ptr(), biases.data_ptr(),
                                   bits, group_size, M, N, K, out.data_ptr(), out.stride(0), y_dtype,
                                   _stream(stream))
    _check("vq_skinny_qmm_noalloc", rc)
    return out


def stream_read(src: torch.Tensor, sink: torch.Tensor, workgroups: int, nontemporal: bool = False,
                stream=None) -> None:
    """Reads every byte of ``src`` (vq_stream_read in include/vq_bench.h: the
    streaming-read ceiling); ``sink`` holds at least 4 * workgroups int32."""
    rc = lib.vq_stream_read(src.data_ptr(), src.numel() * src.element_size(), int(nontemporal), workgroups,
                            sink.data_ptr(), _stream(stream))
    _check("vq_stream_read", rc)


def qmm_pack_bytes(bits: int, N: int, K: int, group_size: int = 64) -> int:
    return int(lib.vq_qmm_pack_bytes(bits, group_size, N, K))


def qmm_pack(wq: torch.Tensor, scales: torch.Tensor, biases: torch.Tensor, bits: int, N: int, K: int,
             group_size: int = 64, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """The tiled pack of a row-major weight (uint8 device tensor; see vq_qmm_pack in include/vq.h)."""
    nbytes = qmm_pack_bytes(bits, N, K, group_size)
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=wq.device)
    rc = lib.vq_qmm_pack(wq.data_ptr(), scales.data_ptr(), biases.data_ptr(), bits, group_size, N, K,
                         out.data_ptr(), out.numel() * out.element_size(), _stream(stream))
    _check("vq_qmm_pack", rc)
    return out


def sumsq_parts(N: int) -> int:
    return int(lib.vq_sumsq_parts(N))


def qmm_packed_workspace_bytes(bits: int, M: int, N: int, K: int, group_size: int = 64) -> int:
    return int(lib.vq_qmm_packed_workspace(bits, group_size, M, N, K))


def qmm_packed(x: torch.Tensor, packed: torch.Tensor, bits: int, N: int, K: int, *, group_size: int = 64,
               x_sumsq: torch.Tensor | None = None, eps: float = 1e-6, epilogue: int = VQ_EPI_STORE,
               residual: torch.Tensor | None = None, out: torch.Tensor | None = None,
               out_dtype: torch.dtype = torch.bfloat16, y_sumsq: torch.Tensor | None = None,
               workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """QMM on a tiled pack with the fused RMSNorm prologue and store / residual /
    SwiGLU epilogues (see vq_qmm_packed in include/vq.h). x_sumsq, y_sumsq are
    float32 [M, sumsq_parts(.)] tensors."""
    M = x.shape[0]
    n_out = N // 2 if epilogue == VQ_EPI_SWIGLU else N
    if out is None:
        out = torch.empty((M, n_out), dtype=out_dtype, device=x.device)
    y_dtype = VQ_F32 if out.dtype == torch.float32 else VQ_BF16
    need = qmm_packed_workspace_bytes(bits, M, N, K, group_size)
    ws = _ws(need, x.device, workspace, "qmm_packed")
    wsz = 0 if ws is None else ws.numel() * ws.element_size()
    parts = 0 if x_sumsq is None else x_sumsq.shape[-1]
    rc = lib.vq_qmm_packed(x.data_ptr(), x.stride(0), _ptr(x_sumsq), parts, eps, packed.data_ptr(), bits,
                           group_size, M, N, K, epilogue, _ptr(residual),
                           0 if residual is None else residual.stride(0), out.data_ptr(), out.stride(0), y_dtype,
                           _ptr(y_sumsq), _ptr(ws), wsz, _stream(stream))
    _check("vq_qmm_packed", rc)
    return out


def row_sumsq(x: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """float32 [M, ceil(N / 128)] sums of squares of x [M, N] per 128 columns (see include/vq_glue.h)."""
    M, N = x.shape
    if out is None:
        out = torch.empty((M, sumsq_parts(N)), dtype=torch.float32, device=x.device)
    rc = lib.vq_row_sumsq_bf16(x.data_ptr(), x.stride(0), M, N, out.data_ptr(), _stream(stream))
    _check("vq_row_sumsq_bf16", rc)
    return out


# ------------------------------------------------------------------- attention
def attn_workspace_bytes(M: int, Hq: int, Hkv: int, D: int, T: int) -> int:
    return int(lib.vq_multirow_attn_workspace(M, Hq, Hkv, D, T))


def multirow_attn(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, T: int,
                  scale: float | None = None, out: torch.Tensor | None = None,
                  workspace: torch.Tensor | None = None, stream=None, k_new: torch.Tensor | None = None,
                  v_new: torch.Tensor | None = None, tree_mask: torch.Tensor | None = None) -> torch.Tensor:
    """q [M, Hq, D] bf16 (heads of a row contiguous; any row stride); caches
    [Hkv, T_cap, D] bf16 (row-contiguous); returns out [M, Hq, D]. With k_new and
    v_new ([M, >= Hkv*D] rows, same row stride) the M rows are appended at cache
    positions T-M .. T-1 inside the call (vq_multirow_attn_append). With
    tree_mask (int32/uint32 device tensor [M] of ancestor bits) the rows are the
    nodes of a draft tree (vq_multirow_attn_tree)."""
    M, Hq, D = q.shape
    Hkv = k_cache.shape[0]
    if scale is None:
        scale = D ** -0.5
    if out is None:
        out = torch.empty_like(q)
    need = attn_workspace_bytes(M, Hq, Hkv, D, T)
    ws = _ws(need, q.device, workspace, "attn")
    wsz = 0 if ws is None else ws.numel() * ws.element_size()
    if tree_mask is not None:
        if (k_new is None) != (v_new is None) or (k_new is not None and k_new.stride(0) != v_new.stride(0)):
            raise ValueError("k_new and v_new go together, with the same row stride")
        rc = lib.vq_multirow_attn_tree(q.data_ptr(), q.stride(0), _ptr(k_new), _ptr(v_new),
                                       0 if k_new is None else k_new.stride(0), k_cache.data_ptr(),
                                       v_cache.data_ptr(), k_cache.stride(0), M, Hq, Hkv, D, T, float(scale),
                                       tree_mask.data_ptr(), out.data_ptr(), out.stride(0), _ptr(ws), wsz,
                                       _stream(stream))
        _check("vq_multirow_attn_tree", rc)
    elif k_new is None:
        rc = lib.vq_multirow_attn(q.data_ptr(), q.stride(0), k_cache.data_ptr(), v_cache.data_ptr(),
                                  k_cache.stride(0), M, Hq, Hkv, D, T, float(scale), out.data_ptr(), out.stride(0),
                                  _ptr(ws), wsz, _stream(stream))
        _check("vq_multirow_attn", rc)
    else:
        if k_new.stride(0) != v_new.stride(0):
            raise ValueError("k_new and v_new must have the same row stride")
        rc = lib.vq_multirow_attn_append(q.data_ptr(), q.stride(0), k_new.data_ptr(), v_new.data_ptr(),
                                         k_new.stride(0), k_cache.data_ptr(), v_cache.data_ptr(), k_cache.stride(0),
                                         M, Hq, Hkv, D, T, float(scale), out.data_ptr(), out.stride(0), _ptr(ws),
                                         wsz, _stream(stream))
        _check("vq_multirow_attn_append", rc)
    return out


def multirow_attn_batched(q: torch.Tensor, row_start: torch.Tensor, seq_len: torch.Tensor, k_cache: torch.Tensor,
                          v_cache: torch.Tensor, max_rows: int, max_T: int, scale: float | None = None,
                          out: torch.Tensor | None = None, k_new: torch.Tensor | None = None,
                          v_new: torch.Tensor | None = None, tree_mask: torch.Tensor | None = None,
                          workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Several sequences in one call (vq_multirow_attn_batched): q [R, Hq, D] stacked
    rows; row_start int32 [B+1], seq_len int32 [B] (device); caches [B, Hkv, T_cap, D]."""
    R, Hq, D = q.shape
    B, Hkv = k_cache.shape[0], k_cache.shape[1]
    if scale is None:
        scale = D ** -0.5
    if out is None:
        out = torch.empty_like(q)
    need = int(lib.vq_multirow_attn_batched_workspace(B, max_rows, Hq, Hkv, D, max_T))
    ws = _ws(need, q.device, workspace, "attn")
    wsz = 0 if ws is None else ws.numel() * ws.element_size()
    rc = lib.vq_multirow_attn_batched(q.data_ptr(), q.stride(0), row_start.data_ptr(), seq_len.data_ptr(), B, R,
                                      max_rows, max_T, _ptr(k_new), _ptr(v_new),
                                      0 if k_new is None else k_new.stride(0), k_cache.data_ptr(), v_cache.data_ptr(),
                                      k_cache.stride(0), k_cache.stride(1), Hq, Hkv, D, float(scale),
                                      _ptr(tree_mask), out.data_ptr(), out.stride(0), _ptr(ws), wsz, _stream(stream))
    _check("vq_multirow_attn_batched", rc)
    return out


def multirow_attn_int8(q: torch.Tensor, k_codes: torch.Tensor, k_sb: torch.Tensor, v_codes: torch.Tensor,
                       v_sb: torch.Tensor, T: int, scale: float | None = None, out: torch.Tensor | None = None,
                       tree_mask: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                       stream=None) -> torch.Tensor:
    """Attention over an 8-bit KV cache (vq_multirow_attn_int8): codes uint8
    [Hkv, T_cap, D]; k_sb, v_sb [Hkv, T_cap, D/64] 32-bit words (bf16 scale low,
    bias high); q [M, Hq, D] bf16; optional tree_mask [M] (32-bit)."""
    M, Hq, D = q.shape
    Hkv = k_codes.shape[0]
    if scale is None:
        scale = D ** -0.5
    if out is None:
        out = torch.empty_like(q)
    ws = _ws(attn_workspace_bytes(M, Hq, Hkv, D, T), q.device, workspace, "attn")
    wsz = 0 if ws is None else ws.numel() * ws.element_size()
    rc = lib.vq_multirow_attn_int8(q.data_ptr(), q.stride(0), k_codes.data_ptr(), k_sb.data_ptr(),
                                   v_codes.data_ptr(), v_sb.data_ptr(), k_codes.stride(0), M, Hq, Hkv, D, T,
                                   float(scale), _ptr(tree_mask), out.data_ptr(), out.stride(0), _ptr(ws), wsz,
                                   _stream(stream))
    _check("vq_multirow_attn_int8", rc)
    return out


def kv8_append(src: torch.Tensor, k_off: int, v_off: int, k_codes: torch.Tensor, k_sb: torch.Tensor,
               v_codes: torch.Tensor, v_sb: torch.Tensor, pos: int, stream=None) -> None:
    """Quantize the M rows of src (bf16 [M, >= ...]) into an 8-bit cache at pos (vq_kv8_append)."""
    Hkv, _, D = k_codes.shape
    _check("vq_kv8_append", lib.vq_kv8_append(src.data_ptr(), src.stride(0), k_off, v_off, k_codes.data_ptr(),
                                              k_sb.data_ptr(), v_codes.data_ptr(), v_sb.data_ptr(),
                                              k_codes.stride(0), src.shape[0], Hkv, D, pos, _stream(stream)))


# ------------------------------------------------------------------ acceptance
def accept_workspace_bytes(B: int, K: int, V: int, input_kind: int, p_stride: int, q_stride: int) -> int:
    return int(lib.vq_spec_accept_workspace(B, K, V, input_kind, p_stride, q_stride))


def spec_accept(p: torch.Tensor, q: torch.Tensor | None, draft: torch.Tensor | None, uniforms: torch.Tensor, *,
                logits: bool = False, temperature: float = 1.0, top_k: int = 0, top_p: float = 1.0,
                probs_out: torch.Tensor | None = None, out_tokens: torch.Tensor | None = None,
                out_n: torch.Tensor | None = None, workspace: torch.Tensor | None = None, stream=None):
    """Exact acceptance for B verifies.

    p: float32 [B, K+1, V] or [K+1, V] (shared by every entry); q: [B, K, V] or
    [K, V]; draft: int32 [B, K]; uniforms: float32 [B, K+1]. Returns
    (tokens int32 [B, K+1], n_accepted int32 [B]).
    """
    B, K1 = uniforms.shape
    K = K1 - 1
    V = p.shape[-1]
    ps = p.stride(0) if p.dim() == 3 else 0
    qs = (q.stride(0) if q.dim() == 3 else 0) if q is not None else 0
    kind = VQ_LOGITS if logits else VQ_PROBS
    if out_tokens is None:
        out_tokens = torch.empty((B, K + 1), dtype=torch.int32, device=p.device)
    if out_n is None:
        out_n = torch.empty((B,), dtype=torch.int32, device=p.device)
    need = accept_workspace_bytes(B, K, V, kind, ps, qs)
    ws = _ws(need, p.device, workspace, "accept")
    wsz = 0 if ws is None else ws.numel() * ws.element_size()
    rc = lib.vq_spec_accept(p.data_ptr(), _ptr(q) if K > 0 else None, kind, ps, qs,
                            _ptr(draft) if K > 0 else None, uniforms.data_ptr(), B, K, V, float(temperature),
                            int(top_k), float(top_p), out_tokens.data_ptr(), out_n.data_ptr(), _ptr(probs_out),
                            _ptr(ws), wsz, _stream(stream))
    _check("vq_spec_accept", rc)
    return out_tokens, out_n


# ------------------------------------------------------------------------ glue
def rmsnorm(x: torch.Tensor, out: torch.Tensor | None = None, eps: float = 1e-6, stream=None) -> torch.Tensor:
    out = torch.empty_like(x) if out is None else out
    _check("vq_rmsnorm_bf16", lib.vq_rmsnorm_bf16(x.data_ptr(), x.stride(0), out.data_ptr(), out.stride(0),
                                                  x.shape[0], x.shape[1], float(eps), _stream(stream)))
    return out


def add_(a: torch.Tensor, b: torch.Tensor, stream=None) -> torch.Tensor:
    """a += b (bf16, contiguous)."""
    _check("vq_add_bf16", lib.vq_add_bf16(a.data_ptr(), b.data_ptr(), a.data_ptr(), a.numel(), _stream(stream)))
    return a


def silu_mul(gu: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    M, I2 = gu.shape
    out = torch.empty((M, I2 // 2), dtype=gu.dtype, device=gu.device) if out is None else out
    _check("vq_silu_mul_bf16", lib.vq_silu_mul_bf16(gu.data_ptr(), gu.stride(0), out.data_ptr(), out.stride(0), M,
                                                    I2 // 2, _stream(stream)))
    return out


def kv_append(src: torch.Tensor, k_off: int, v_off: int, k_cache: torch.Tensor, v_cache: torch.Tensor, pos: int,
              stream=None) -> None:
    Hkv, _, D = k_cache.shape
    _check("vq_kv_append_bf16", lib.vq_kv_append_bf16(src.data_ptr(), src.stride(0), k_off, v_off,
                                                      k_cache.data_ptr(), v_cache.data_ptr(), k_cache.stride(0),
                                                      src.shape[0], Hkv, D, pos, _stream(stream)))
