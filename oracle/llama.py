"""Oracle composition of a Llama-shaped forward step (test infrastructure).

The same sequence of operations as the HIP engine, evaluated with the CPU
oracle's primitives in numpy float32 arrays (bf16 values widened).  Each
request is processed on its own: the oracle has no batch, so its output for
a request cannot depend on one.  KV lives in the oracle's own paged pools
(numpy), written at the same (page, slot) addresses.

The model is bf16 throughout, so attention takes the bf16-weight form
(p rounded to bf16 before the sums, as matrix cores consume it).

Layer (pre-norm, SwiGLU, RoPE on q and k):
  x = rmsnorm(h) ; qkv = x W_qkv^T ; q,k = rope(q,k) ; append k,v
  a = attention(q) ; h = h + a W_o^T ; x = rmsnorm(h)
  h = h + (silu(x W_g^T) * (x W_u^T)) W_d^T
then logits = rmsnorm(h) W_lm^T (fp32), token = argmax.
"""
from __future__ import annotations

import numpy as np

from . import add, argmax, decode_attn, gemm, prefill_attn, rmsnorm, rope, silu_mul


def _np(t):
    if hasattr(t, "detach"):
        return t.detach().float().cpu().numpy()
    return np.asarray(t, dtype=np.float32)


class OracleModel:
    """cfg: object with d, h, h_kv, d_h, ffn, vocab, eps, kv_chunk, page_size,
    scale and rope (bool); weights: object with embed, layers (attn_norm,
    wqkv, wo, ffn_norm, wgu, wdown), final_norm, lm_head (torch or numpy);
    gemm: the GEMM primitive (the oracle's serial one unless a test swaps in
    another valid order to measure how far two orders drift apart)."""

    def __init__(self, cfg, weights, num_pages: int, cos_t=None, sin_t=None, layers=None,
                 gemm=gemm):
        self.cfg = cfg
        self.gemm = gemm
        self.nl = layers if layers is not None else len(weights.layers)
        self.embed = _np(weights.embed)
        self.layers = []
        for lw in weights.layers[:self.nl]:
            self.layers.append({k: _np(getattr(lw, k)) for k in
                                ("attn_norm", "wqkv", "wo", "ffn_norm", "wgu", "wdown")})
        self.final_norm = _np(weights.final_norm)
        self.lm_head = _np(weights.lm_head)
        self.cos = _np(cos_t) if cos_t is not None else None
        self.sin = _np(sin_t) if sin_t is not None else None
        shape = (self.nl, num_pages, cfg.h_kv, cfg.page_size, cfg.d_h)
        self.k = np.zeros(shape, np.float32)
        self.v = np.zeros(shape, np.float32)

    def forward(self, pages, pos0: int, tokens, want_logits: bool = True):
        """Rows tokens[0..n) of one request at positions pos0.. ; returns the
        fp32 logits of the last row (or None) and its argmax."""
        c = self.cfg
        n = len(tokens)
        pos = np.arange(pos0, pos0 + n, dtype=np.int32)
        bt = np.asarray(pages, np.int32)[None, :]
        h = self.embed[np.asarray(tokens, np.int64)]
        hd = c.h * c.d_h
        kvd = c.h_kv * c.d_h
        for li, lw in enumerate(self.layers):
            x = rmsnorm(h, lw["attn_norm"], c.eps, True)
            qkv = self.gemm(x, lw["wqkv"], True)
            q = qkv[:, :hd].reshape(n, c.h, c.d_h)
            k = qkv[:, hd:hd + kvd].reshape(n, c.h_kv, c.d_h)
            v = qkv[:, hd + kvd:].reshape(n, c.h_kv, c.d_h)
            if c.rope:
                q = rope(q, pos, self.cos, self.sin, True)
                k = rope(k, pos, self.cos, self.sin, True)
            pg = bt[0, pos // c.page_size]
            self.k[li, pg, :, pos % c.page_size] = k
            self.v[li, pg, :, pos % c.page_size] = v
            if n == 1:
                a = decode_attn(q, self.k[li], self.v[li], bt, np.array([pos0 + 1], np.int32),
                                c.h_kv, c.page_size, c.kv_chunk, c.scale, True, p_bf16=True)
            else:
                a = prefill_attn(q, np.array([0, n], np.int32), np.array([pos0], np.int32),
                                 self.k[li], self.v[li], bt, c.h_kv, c.page_size, c.kv_chunk,
                                 c.scale, True, p_bf16=True)
            h = add(h, self.gemm(a.reshape(n, hd), lw["wo"], True), True)
            x = rmsnorm(h, lw["ffn_norm"], c.eps, True)
            act = silu_mul(self.gemm(x, lw["wgu"], True), True)
            h = add(h, self.gemm(act, lw["wdown"], True), True)
        if not want_logits:
            return None, None
        x = rmsnorm(h[-1:], self.final_norm, c.eps, True)
        logits = self.gemm(x, self.lm_head, False)
        return logits[0], int(argmax(logits)[0])
