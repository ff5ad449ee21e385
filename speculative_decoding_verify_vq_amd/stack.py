"""One verify step of a dense pre-norm stack, composed from the library's kernels.

The verify pass of MTP speculative decoding runs the last committed token and
the K drafted tokens (M = K + 1 rows) through one forward pass, then accepts or
rejects the drafts exactly (page "The fastest way to run local LLMs on a Mac",
sections "Why native MTP doubles decode" and "Why exact acceptance matters").
Per layer, with h the bf16 residual stream and S its per-row sums of squares
(per 128 columns):

    qkv = qmm(rms(h), W_qkv)                         RMSNorm fused into the staging of x
    attention layers: c = multirow_attn(q, K cache, V cache, T = ctx + M), which
          appends k, v at positions ctx .. ctx+M-1 itself
    other layers (their recurrent state is out of scope): c = q
    h, S = h + qmm(c, W_o)                           residual epilogue, writes S
    act  = swiglu(qmm(rms(h), W_gate_up))            gate|up rows interleaved per 64 outputs
    h, S = h + qmm(act, W_down)

then float32 logits = qmm(rms(h), W_lm) feed spec_accept in logits mode together
with the draft logits. With B > 1 sequences (each with its own caches and
context length) the B*M rows are stacked and share every weight pass; the
attention layers run vq_multirow_attn_batched and acceptance has B entries. Weights are held in the tiled pack of vq_qmm_pack. Every
launch goes to one stream, so the whole step can be captured once into a HIP
graph and replayed.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

from . import vq


def qmm_algorithmic_bytes(M: int, N: int, K: int, bits: int, group_size: int = 64, out_bytes: int = 2) -> int:
    """Minimum HBM bytes of one skinny-QMM call: packed codes + bf16 scale and bias
    per group + bf16 activations in + outputs."""
    return N * K * bits // 8 + 4 * N * (K // group_size) + 2 * M * K + out_bytes * M * N


@dataclass
class StackConfig:
    layers: int = 64
    hidden: int = 5120
    inter: int = 17408
    Hq: int = 24
    Hkv: int = 4
    D: int = 256
    vocab: int = 248320
    bits: int = 4
    lm_bits: int = 4
    attn_every: int = 4          # attention on layers attn_every-1, 2*attn_every-1, ...
    ctx: int = 16384             # committed positions in every KV cache
    M: int = 4                   # verify rows = K + 1 (per sequence)
    B: int = 1                   # sequences verified together (their B * M rows share the weight pass)
    temperature: float = 0.7
    top_k: int = 0
    top_p: float = 0.95
    group_size: int = 64
    eps: float = 1e-6

    @property
    def rows(self) -> int:
        return self.B * self.M

    def is_attn(self, layer: int) -> bool:
        return layer % self.attn_every == self.attn_every - 1

    @property
    def q_width(self) -> int:
        return self.Hq * self.D

    @property
    def qkv_width(self) -> int:
        return (self.Hq + 2 * self.Hkv) * self.D

    @property
    def n_attn(self) -> int:
        return sum(self.is_attn(i) for i in range(self.layers))

    def shapes(self) -> dict:
        """Output/input sizes (N, K) of each projection of a layer, and of the lm_head."""
        return {"qkv": (self.qkv_width, self.hidden), "o": (self.hidden, self.q_width),
                "gate_up": (2 * self.inter, self.hidden), "down": (self.hidden, self.inter),
                "lm_head": (self.vocab, self.hidden)}


@dataclass
class QPack:
    """One quantized weight matrix W[N, K] in the tiled pack of vq_qmm_pack."""
    packed: torch.Tensor   # uint8, vq.qmm_pack_bytes(bits, N, K) bytes
    N: int
    K: int
    bits: int
    group_size: int = 64

    def nbytes(self) -> int:
        """Algorithmic bytes of the weight: codes + one bf16 scale and bias per group."""
        return self.N * self.K * self.bits // 8 + 4 * self.N * (self.K // self.group_size)

    @staticmethod
    def from_rows(wq: torch.Tensor, scales: torch.Tensor, biases: torch.Tensor, bits: int, N: int, K: int,
                  group_size: int = 64) -> "QPack":
        """Packs a row-major weight (int32 code words, bf16 scales and biases [N, K / gs])."""
        return QPack(vq.qmm_pack(wq, scales, biases, bits, N, K, group_size), N, K, bits, group_size)


@dataclass
class StackWeights:
    layers: list = field(default_factory=list)   # per layer: dict name -> QPack ("gate_up" rows interleaved)
    lm_head: QPack | None = None
    k_cache: list = field(default_factory=list)  # per attention layer: bf16 [Hkv, T_cap, D] ([B, Hkv, T_cap, D] for B > 1)
    v_cache: list = field(default_factory=list)

    def weight_bytes(self) -> int:
        return sum(p.nbytes() for lay in self.layers for p in lay.values()) + self.lm_head.nbytes()


class DenseVerifyStack:
    """Preallocated buffers and workspaces for one verify step (M rows)."""

    def __init__(self, cfg: StackConfig, weights: StackWeights, device="cuda", ctx_per_seq=None):
        """ctx_per_seq (B > 1 only): committed positions of each sequence (default cfg.ctx each)."""
        self.cfg = cfg
        self.w = weights
        dev = torch.device(device)
        M = cfg.rows
        bf = torch.bfloat16
        self.h = torch.empty((M, cfg.hidden), dtype=bf, device=dev)
        self.ss = torch.empty((M, vq.sumsq_parts(cfg.hidden)), dtype=torch.float32, device=dev)
        self.qkv = torch.empty((M, cfg.qkv_width), dtype=bf, device=dev)
        self.ctx_out = torch.empty((M, cfg.q_width), dtype=bf, device=dev)
        self.act = torch.empty((M, cfg.inter), dtype=bf, device=dev)
        B, Mb = cfg.B, cfg.M
        self.logits = torch.empty((B, Mb, cfg.vocab), dtype=torch.float32, device=dev)
        self.probs = torch.empty((B, 2 * Mb - 1, cfg.vocab), dtype=torch.float32, device=dev)
        self.tokens = torch.empty((B, Mb), dtype=torch.int32, device=dev)
        self.n_acc = torch.empty((B,), dtype=torch.int32, device=dev)
        ctxs = [cfg.ctx] * B if ctx_per_seq is None else list(ctx_per_seq)
        assert len(ctxs) == B
        self.ctxs = ctxs
        self.row_start = torch.tensor([b * Mb for b in range(B + 1)], dtype=torch.int32, device=dev)
        self.seq_len = torch.tensor([c + Mb for c in ctxs], dtype=torch.int32, device=dev)
        sh = cfg.shapes()
        qmm_ws = max(vq.qmm_packed_workspace_bytes(b, M, N, K)
                     for name, (N, K) in sh.items()
                     for b in ([cfg.lm_bits] if name == "lm_head" else [cfg.bits]))
        T = max(ctxs) + Mb
        if B == 1:
            attn_ws = vq.attn_workspace_bytes(Mb, cfg.Hq, cfg.Hkv, cfg.D, T)
        else:
            attn_ws = int(vq.lib.vq_multirow_attn_batched_workspace(B, Mb, cfg.Hq, cfg.Hkv, cfg.D, T))
        acc_ws = vq.accept_workspace_bytes(B, Mb - 1, cfg.vocab, vq.VQ_LOGITS, Mb * cfg.vocab, (Mb - 1) * cfg.vocab)
        z = lambda n: torch.zeros(n + 256, dtype=torch.uint8, device=dev) if n else None
        self._ws = {"qmm": z(qmm_ws), "attn": z(attn_ws), "accept": z(acc_ws)}

    def _wsv(self, kind):
        buf = self._ws[kind]
        if buf is None:
            return None
        off = (-buf.data_ptr()) % 256
        return buf[off:]

    def _qmm(self, x, pack: QPack, out, *, norm: bool = False, epilogue: int = vq.VQ_EPI_STORE, y_sumsq=None,
             residual=None):
        if epilogue == vq.VQ_EPI_RESIDUAL and residual is None:
            residual = self.h
        vq.qmm_packed(x, pack.packed, pack.bits, pack.N, pack.K, group_size=pack.group_size,
                      x_sumsq=self.ss if norm else None, eps=self.cfg.eps, epilogue=epilogue,
                      residual=residual, out=out, y_sumsq=y_sumsq, workspace=self._wsv("qmm"))

    def forward_hidden(self, h_in: torch.Tensor, after_layer=None) -> torch.Tensor:
        """Runs the layers on h_in [M, hidden] (bf16); returns the final hidden rows
        (their sums of squares are left in self.ss for the final RMSNorm).
        ``after_layer(layer, h)``, if given, is called after each layer with the
        hidden rows (on the stream, before the next layer's launches)."""
        cfg = self.cfg
        # Layer 0 reads h_in directly (its residual epilogue writes the first
        # hidden rows into self.h), so no copy of h_in is launched.
        vq.row_sumsq(h_in, out=self.ss)
        if not self.w.layers:
            self.h.copy_(h_in)
        ai = 0
        for li, lay in enumerate(self.w.layers):
            src = h_in if li == 0 else self.h
            self._qmm(src, lay["qkv"], self.qkv, norm=True)
            q = self.qkv[:, : cfg.q_width]
            if cfg.is_attn(li):
                kc, vc = self.w.k_cache[ai], self.w.v_cache[ai]
                ai += 1
                R = cfg.rows
                qv = q.as_strided((R, cfg.Hq, cfg.D), (self.qkv.stride(0), cfg.D, 1))
                ov = self.ctx_out.view(R, cfg.Hq, cfg.D)
                k_new = self.qkv[:, cfg.q_width: cfg.q_width + cfg.Hkv * cfg.D]
                v_new = self.qkv[:, cfg.q_width + cfg.Hkv * cfg.D:]
                if cfg.B == 1:
                    vq.multirow_attn(qv, kc, vc, self.ctxs[0] + cfg.M, cfg.D ** -0.5, out=ov,
                                     workspace=self._wsv("attn"), k_new=k_new, v_new=v_new)
                else:
                    vq.multirow_attn_batched(qv, self.row_start, self.seq_len, kc, vc, cfg.M, max(self.ctxs) + cfg.M,
                                             cfg.D ** -0.5, out=ov, k_new=k_new, v_new=v_new,
                                             workspace=self._wsv("attn"))
                c = self.ctx_out
            else:
                c = q
            self._qmm(c, lay["o"], self.h, epilogue=vq.VQ_EPI_RESIDUAL, y_sumsq=self.ss, residual=src)
            self._qmm(self.h, lay["gate_up"], self.act, norm=True, epilogue=vq.VQ_EPI_SWIGLU)
            self._qmm(self.act, lay["down"], self.h, epilogue=vq.VQ_EPI_RESIDUAL, y_sumsq=self.ss)
            if after_layer is not None:
                after_layer(li, self.h)
        return self.h

    def step(self, h_in, draft_logits, drafts, uniforms, after_layer=None):
        """One verify step: layers, lm_head, exact acceptance.

        h_in bf16 [B*M, hidden] (sequence b's rows at b*M); draft_logits float32
        [B, K, V]; drafts int32 [B, K]; uniforms float32 [B, K+1]. Returns
        (tokens int32 [B, K+1], n_accepted int32 [B]). ``after_layer`` as in
        forward_hidden.
        """
        cfg = self.cfg
        self.forward_hidden(h_in, after_layer)
        self._qmm(self.h, self.w.lm_head, self.logits.view(cfg.rows, cfg.vocab), norm=True)
        vq.spec_accept(self.logits, draft_logits, drafts, uniforms, logits=True, temperature=cfg.temperature,
                       top_k=cfg.top_k, top_p=cfg.top_p, probs_out=self.probs, out_tokens=self.tokens,
                       out_n=self.n_acc, workspace=self._wsv("accept"))
        return self.tokens, self.n_acc

    def bytes_per_step(self) -> dict:
        """Algorithmic HBM bytes of one step: weights once, KV (K and V) once per
        attention layer, and the logit rows of the acceptance step."""
        cfg = self.cfg
        kv = cfg.n_attn * 4 * cfg.Hkv * sum(c + cfg.M for c in self.ctxs) * cfg.D
        acc = cfg.B * (2 * cfg.M - 1) * cfg.vocab * 4
        return {"weights": self.w.weight_bytes(), "kv": kv, "accept_rows": acc,
                "total": self.w.weight_bytes() + kv + acc}
