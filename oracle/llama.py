"""Oracle composition of a Llama-shaped forward step (test infrastructure).

The same sequence of operations as the HIP engine, evaluated with the CPU
oracle's primitives in numpy float32 arrays (bf16 values widened).  Each
request is processed on its own: the oracle has no batch, so its output for
a request cannot depend on one.  KV lives in the oracle's own paged pools
(numpy), written at the same (page, slot) addresses.

The model is bf16 throughout, so attention takes the bf16-weight form
(p rounded to bf16 before the sums, as matrix cores consume it).  With
bf16=False every intermediate stays fp32 and attention keeps fp32 weights:
the same wiring without the carried rounding, which is how the composition
itself is checked against a float64 forward written from the layer
definition (tests/test_oracle_model_pin.py).

Layer (pre-norm, SwiGLU, RoPE on q and k):
  x = rmsnorm(h) ; qkv = x W_qkv^T ; q,k = rope(q,k) ; append k,v
  a = attention(q) ; h = h + a W_o^T ; x = rmsnorm(h)
  h = h + (silu(x W_g^T) * (x W_u^T)) W_d^T
then logits = rmsnorm(h) W_lm^T (fp32), token = argmax.

Weight layout: the fused gate/up weight wgu [2F, d] comes in 8-row blocks,
rows 16p .. 16p + 7 being gate rows 8p .. 8p + 7 and rows 16p + 8 .. 16p + 15
the matching up rows; the oracle takes W_g and W_u out of it at load.
"""
from __future__ import annotations

import numpy as np

from . import add, argmax, decode_attn, gemm, prefill_attn, rmsnorm, rope, silu_mul


def _np(t):
    if hasattr(t, "detach"):
        return t.detach().float().cpu().numpy()
    return np.asarray(t, dtype=np.float32)


def gate_up_halves(wgu):
    """W_g stacked over W_u ([2F, d]) from the fused weight's 8-row blocks."""
    wgu = np.asarray(wgu)
    f2, d = wgu.shape
    blocks = wgu.reshape(f2 // 16, 2, 8, d)
    return np.concatenate([blocks[:, 0].reshape(f2 // 2, d), blocks[:, 1].reshape(f2 // 2, d)])


class OracleModel:
    """cfg: object with d, h, h_kv, d_h, ffn, vocab, eps, kv_chunk, page_size,
    scale and rope (bool); weights: object with embed, layers (attn_norm,
    wqkv, wo, ffn_norm, wgu, wdown), final_norm, lm_head (torch or numpy);
    gemm: the GEMM primitive (the oracle's serial one unless a test swaps in
    another valid order to measure how far two orders drift apart); bf16:
    carry bf16 between operations (the model's precision) or fp32."""

    def __init__(self, cfg, weights, num_pages: int, cos_t=None, sin_t=None, layers=None,
                 gemm=gemm, bf16: bool = True):
        self.cfg = cfg
        self.gemm = gemm
        self.rb = bool(bf16)
        self.nl = layers if layers is not None else len(weights.layers)
        self.embed = _np(weights.embed)
        self.layers = []
        for lw in weights.layers[:self.nl]:
            lay = {k: _np(getattr(lw, k)) for k in
                   ("attn_norm", "wqkv", "wo", "ffn_norm", "wgu", "wdown")}
            lay["wgu"] = gate_up_halves(lay["wgu"])   # [W_g; W_u]
            self.layers.append(lay)
        self.final_norm = _np(weights.final_norm)
        self.lm_head = _np(weights.lm_head)
        self.cos = _np(cos_t) if cos_t is not None else None
        self.sin = _np(sin_t) if sin_t is not None else None
        shape = (self.nl, num_pages, cfg.h_kv, cfg.page_size, cfg.d_h)
        self.k = np.zeros(shape, np.float32)
        self.v = np.zeros(shape, np.float32)

    def layer(self, li: int, h, pages, pos0: int):
        """Decoder layer li on the residual rows h [n, d] of one request at
        positions pos0 .. pos0 + n - 1: appends their K and V to the layer's
        pool at the request's pages and returns the new residual rows."""
        c, rb = self.cfg, self.rb
        lw = self.layers[li]
        n = h.shape[0]
        pos = np.arange(pos0, pos0 + n, dtype=np.int32)
        bt = np.asarray(pages, np.int32)[None, :]
        hd = c.h * c.d_h
        kvd = c.h_kv * c.d_h
        x = rmsnorm(h, lw["attn_norm"], c.eps, rb)
        qkv = self.gemm(x, lw["wqkv"], rb)
        q = qkv[:, :hd].reshape(n, c.h, c.d_h)
        k = qkv[:, hd:hd + kvd].reshape(n, c.h_kv, c.d_h)
        v = qkv[:, hd + kvd:].reshape(n, c.h_kv, c.d_h)
        if c.rope:
            q = rope(q, pos, self.cos, self.sin, rb)
            k = rope(k, pos, self.cos, self.sin, rb)
        pg = bt[0, pos // c.page_size]
        self.k[li, pg, :, pos % c.page_size] = k
        self.v[li, pg, :, pos % c.page_size] = v
        if n == 1:
            a = decode_attn(q, self.k[li], self.v[li], bt, np.array([pos0 + 1], np.int32),
                            c.h_kv, c.page_size, c.kv_chunk, c.scale, rb, p_bf16=rb)
        else:
            a = prefill_attn(q, np.array([0, n], np.int32), np.array([pos0], np.int32),
                             self.k[li], self.v[li], bt, c.h_kv, c.page_size, c.kv_chunk,
                             c.scale, rb, p_bf16=rb)
        h = add(h, self.gemm(a.reshape(n, hd), lw["wo"], rb), rb)
        x = rmsnorm(h, lw["ffn_norm"], c.eps, rb)
        act = silu_mul(self.gemm(x, lw["wgu"], rb), rb)
        return add(h, self.gemm(act, lw["wdown"], rb), rb)

    def head(self, h):
        """Final norm and LM head of residual rows h [n, d]: fp32 logits [n, V]."""
        x = rmsnorm(h, self.final_norm, self.cfg.eps, self.rb)
        return self.gemm(x, self.lm_head, False)

    def forward(self, pages, pos0: int, tokens, want_logits: bool = True):
        """Rows tokens[0..n) of one request at positions pos0.. ; returns the
        fp32 logits of the last row (or None) and its argmax."""
        h = self.embed[np.asarray(tokens, np.int64)]
        for li in range(self.nl):
            h = self.layer(li, h, pages, pos0)
        if not want_logits:
            return None, None
        logits = self.head(h[-1:])
        return logits[0], int(argmax(logits)[0])
