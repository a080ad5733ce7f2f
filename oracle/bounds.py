"""Error bounds for comparing split-KV attention with the oracle (test
infrastructure, like the rest of this package).

bf16 KV runs on matrix cores: the scores come out of the hardware's
accumulation order and the softmax weights are rounded to bf16 before the
sums ("Batch invariance and reproducible inference", "Non-associativity,
concretely": any fixed order is as correct as another, so the parity with
the oracle's serial order is a bound, not bits).  The bound below is derived
in fp64 from the inputs, per output element of the merged result:

  scores:   |ds| <= 2 (d_h + 1) u sum_i |q_i k_i| scale + u |s|   (two fp32
            dot products in any order, then the scaling);
  weights:  each side rounds p = exp(s - m_chunk) to bf16, possibly against
            a different chunk maximum and with s off by ds, so
            |dP| <= P (2^-7 + 3 max|ds| + 8 u);
  sums:     l and acc in any order: 2 (n + 1) u sum P |v| and 2 (n + 1) u l;
  merge:    rescaling factors exp(m_c - M) off by (2 max|ds| + 4 u);
  output:   |d out| <= [sum_c w_c sum_k dP_k |v_k - out|
                       + 4 (n + 1) u sum_c w_c sum_k P_k |v_k|
                       + (2 max|ds| + 4 u) sum_c w_c |acc_c - out l_c|] / L
            plus, for bf16 outputs, one bf16 ulp (2^-7 |out|) for two values
            that straddle a rounding boundary.
"""
from __future__ import annotations

import numpy as np

U = 2.0 ** -24


def _np(a):
    if hasattr(a, "detach"):
        return a.detach().float().cpu().numpy()
    return np.asarray(a, np.float32)


def _rows(pool, bt_row, s, h_kv_i, page_size):
    idx = np.arange(s)
    return pool[bt_row[idx // page_size], h_kv_i, idx % page_size].astype(np.float64)


def attn_bound(q, k_pool, v_pool, block_table, kv_len, h_kv: int, page_size: int, chunk: int,
               scale: float, out_bf16: bool, positions=None, rows_bt=None):
    """Bound per element of the [rows, h, d_h] attention output.  Decode:
    row r attends to kv_len[r] keys with block-table row r.  Prefill: pass
    positions (absolute position of each row; it sees keys 0..pos) and
    rows_bt (block-table row of each row) instead of kv_len."""
    q = _np(q).astype(np.float64)
    kp, vp = _np(k_pool), _np(v_pool)
    bt = np.asarray(block_table)
    nrow, h, d_h = q.shape
    group = h // h_kv
    bound = np.zeros_like(q)
    for r in range(nrow):
        if positions is None:
            s_len, btr = int(kv_len[r]), bt[r]
        else:
            s_len, btr = int(positions[r]) + 1, bt[int(rows_bt[r])]
        nch = (s_len + chunk - 1) // chunk
        for g in range(h_kv):
            K = _rows(kp, btr, s_len, g, page_size)          # [n, d_h]
            V = _rows(vp, btr, s_len, g, page_size)
            Q = q[r, g * group:(g + 1) * group]              # [G, d_h]
            s = (Q @ K.T) * scale                            # [G, n]
            ds = 2 * (d_h + 1) * U * (np.abs(Q) @ np.abs(K).T) * scale + U * np.abs(s)
            dmax = ds.max(axis=1, keepdims=True)             # [G, 1]
            pad = nch * chunk - s_len
            sp = np.pad(s, ((0, 0), (0, pad)), constant_values=-np.inf).reshape(group, nch, chunk)
            m = sp.max(axis=2)                               # [G, nch]
            P = np.exp(sp - m[:, :, None]).reshape(group, -1)[:, :s_len]
            w = np.exp(m - m.max(axis=1, keepdims=True))     # [G, nch]
            wk = np.repeat(w, chunk, axis=1)[:, :s_len]
            WP = wk * P
            L = WP.sum(axis=1, keepdims=True)
            out = WP @ V / L                                 # [G, d_h]
            dP = P * (2.0 ** -7 + 3 * dmax + 8 * U)
            t1 = np.stack([(wk[i] * dP[i]) @ np.abs(V - out[i]) for i in range(group)])
            t2 = 4 * (s_len + 1) * U * (WP @ np.abs(V))
            Pp = np.pad(P, ((0, 0), (0, pad))).reshape(group, nch, chunk)
            Vp = np.pad(V, ((0, pad), (0, 0))).reshape(nch, chunk, d_h)
            lc = Pp.sum(axis=2)                              # [G, nch]
            ac = np.einsum("gck,ckd->gcd", Pp, Vp)           # [G, nch, d_h]
            t3 = (2 * dmax + 4 * U) * np.einsum("gc,gcd->gd", w,
                                                np.abs(ac - out[:, None, :] * lc[:, :, None]))
            b = (t1 + t2 + t3) / L
            if out_bf16:
                b = b + 2.0 ** -7 * np.abs(out)
            bound[r, g * group:(g + 1) * group] = b
    return bound
