"""Teacher-forced check of one decoder layer of the engine against the
oracle, kernel by kernel and as a whole.

Given what the engine's kernels wrote for the decode rows of layer li (the
tap buffers of Engine.forward) and the layer's KV pages after the step,
every kernel is re-run by the oracle on the engine's own input to that
kernel and compared with the engine's output:

  bitwise (the kernel mirrors the oracle's order):
      attention norm, residual adds, FFN norm, SiLU-mul;
  within the derived bound (matrix-core order differs from the oracle's
  serial one):
      QKV GEMM -- values directly, queries and keys through RoPE;
      attention over the engine's own q and KV pages (oracle/bounds.py);
      O, gate/up and down GEMMs (the bound of helpers.gemm_bf16_tol).

So every layer's output lies within the composition of the per-kernel
bounds of its inputs.  The whole layer is also run by the oracle model
(oracle/llama.py, OracleModel.layer) from the engine's input residual row,
and the relative gap of the two output rows is returned for the report.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from helpers import bits_equal, gu_halves, mismatch_report

U = 2.0 ** -24


def rope_tol(a_tol, b_tol, cos, sin, ref):
    """Bound on |engine - oracle| of a rotated bf16 pair x' = a c - b s,
    x'' = b c + a s whose inputs a, b are within a_tol, b_tol: the rotation
    moves them by at most |c| da + |s| db (one fma and one product, each
    within an ulp of fp32), and the two bf16 roundings may straddle a
    boundary (one bf16 ulp, 2^-7 |ref|)."""
    d = np.abs(cos) * a_tol + np.abs(sin) * b_tol
    return 2.0 ** -7 * np.abs(ref) + 1.01 * d + 4 * U * np.abs(ref) + 1e-30


def gemm_tol(A, W, ref):
    """The bound of helpers.gemm_bf16_tol with the magnitude sum taken in
    fp32 (a sum of non-negative terms: relative error below K u, covered by
    the extra factor 1.01), which keeps full-size weights cheap to handle."""
    K = A.shape[1]
    s = (np.abs(np.asarray(A, np.float32)) @ np.abs(np.asarray(W, np.float32)).T)
    s = s.astype(np.float64) * 1.01
    return 2.0 ** -7 * np.abs(ref) + 1.01 * 2.0 * (K + 1) * U * s + 1e-30


def _within(name, got, ref, tol):
    err = np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))
    bad = err > tol
    assert not bad.any(), (f"{name}: {int(bad.sum())} of {err.size} outside the bound; "
                           f"max excess {float(np.max(err - tol)):.3e}")
    return float(np.max(err / np.maximum(tol, 1e-30)))


def check_layer(cfg, lw, taps, li, pos, kps, vps, cos_t, sin_t):
    """Rows of several decode requests at once.  lw: the layer's weights as
    float32 numpy ({attn_norm, wqkv, wo, ffn_norm, wgu, wdown}), as the oracle
    model holds them (wgu = [W_g; W_u]); taps:
    {name: float32 numpy [rows, n]} for this layer (h_in, x_attn, q, att, o,
    h_mid, x_ffn, gu (optional), act, down, h_out); pos: each row's absolute
    position; kps, vps: per row, float32 [npg, h_kv, page, d_h], the
    request's pages (block-table order) after the step; cos_t, sin_t:
    float32 RoPE tables (None: no rotation).
    Returns {kernel: max error / bound} for the report."""
    c = cfg
    t = taps
    n = t["h_in"].shape[0]
    hd, kvd = c.h * c.d_h, c.h_kv * c.d_h
    half = c.d_h // 2
    ps = c.page_size
    pos = np.asarray(pos, np.int32)
    out = {}

    def same(name, got, ref):
        assert bits_equal(got, ref), f"layer {li} {name}: {mismatch_report(got, ref)}"

    same("attn rmsnorm", t["x_attn"], oracle.rmsnorm(t["h_in"], lw["attn_norm"], c.eps, True))
    # QKV: values straight from the product, queries and keys through RoPE
    qkv = oracle.gemm(t["x_attn"], lw["wqkv"], True)
    tol = gemm_tol(t["x_attn"], lw["wqkv"], qkv)
    k_eng = np.stack([kps[i][pos[i] // ps, :, pos[i] % ps] for i in range(n)])
    v_eng = np.stack([vps[i][pos[i] // ps, :, pos[i] % ps] for i in range(n)])
    out["qkv(v)"] = _within(f"layer {li} v", v_eng.reshape(n, kvd), qkv[:, hd + kvd:],
                            tol[:, hd + kvd:])

    def rotated(x, xt, nh):
        x3, t3 = x.reshape(n, nh, c.d_h), xt.reshape(n, nh, c.d_h)
        if cos_t is None:
            return x3, t3
        ref = oracle.rope(x3, pos, cos_t, sin_t, True)
        cs, sn = cos_t[pos][:, None, :], sin_t[pos][:, None, :]
        a_t, b_t = t3[..., :half], t3[..., half:]
        bnd = np.concatenate([rope_tol(a_t, b_t, cs, sn, ref[..., :half]),
                              rope_tol(b_t, a_t, cs, sn, ref[..., half:])], axis=-1)
        return ref, bnd

    q_ref, q_tol = rotated(qkv[:, :hd], tol[:, :hd], c.h)
    q_eng = t["q"].reshape(n, c.h, c.d_h)
    out["qkv(q)"] = _within(f"layer {li} q", q_eng, q_ref, q_tol)
    k_ref, k_tol = rotated(qkv[:, hd:hd + kvd], tol[:, hd:hd + kvd], c.h_kv)
    out["qkv(k)"] = _within(f"layer {li} k", k_eng, k_ref, k_tol)
    # attention over the engine's own query and pages, request by request
    from oracle.bounds import attn_bound
    worst = 0.0
    for i in range(n):
        npg = kps[i].shape[0]
        bt = np.arange(npg, dtype=np.int32)[None, :]
        kv_len = np.array([pos[i] + 1], np.int32)
        qi = q_eng[i:i + 1]
        a_ref = oracle.decode_attn(qi, kps[i], vps[i], bt, kv_len, c.h_kv, ps, c.kv_chunk,
                                   c.scale, round_bf16=True, p_bf16=True)
        a_tol = attn_bound(qi, kps[i], vps[i], bt, kv_len, c.h_kv, ps, c.kv_chunk, c.scale,
                           out_bf16=True)
        worst = max(worst, _within(f"layer {li} attention (row {i})",
                                   t["att"][i].reshape(1, c.h, c.d_h), a_ref, a_tol))
    out["attention"] = worst
    att = t["att"].reshape(n, hd)
    o_ref = oracle.gemm(att, lw["wo"], True)
    out["o_proj"] = _within(f"layer {li} O", t["o"], o_ref, gemm_tol(att, lw["wo"], o_ref))
    same("residual add 1", t["h_mid"], oracle.add(t["h_in"], t["o"], True))
    same("ffn rmsnorm", t["x_ffn"], oracle.rmsnorm(t["h_mid"], lw["ffn_norm"], c.eps, True))
    gu_ref = oracle.gemm(t["x_ffn"], lw["wgu"], True)
    gu_tol = gemm_tol(t["x_ffn"], lw["wgu"], gu_ref)
    if "gu" in t:
        # the engine's product comes in 8-column gate/up blocks; the oracle's
        # weights are [W_g; W_u], so its product is [gate | up]
        gh = gu_halves(t["gu"])
        out["gate_up"] = _within(f"layer {li} gate/up", gh, gu_ref, gu_tol)
        same("silu_mul", t["act"], oracle.silu_mul(gh, True))
    else:
        # fused SwiGLU: |d(silu(g) u)| <= |silu'(g)| |u| dg + |silu(g)| du,
        # |silu'| <= 1.1; plus one bf16 ulp of the result
        g, u = gu_ref[:, :c.ffn], gu_ref[:, c.ffn:]
        act_ref = oracle.silu_mul(gu_ref, True)
        sg = np.abs(g / (1.0 + np.exp(-g.astype(np.float64))))
        bnd = (2.0 ** -7 * np.abs(act_ref) + 1.01 * (1.1 * np.abs(u) * gu_tol[:, :c.ffn]
                                                      + sg * gu_tol[:, c.ffn:]) + 1e-30)
        out["gate_up+silu"] = _within(f"layer {li} swiglu", t["act"], act_ref, bnd)
    d_ref = oracle.gemm(t["act"], lw["wdown"], True)
    out["down_proj"] = _within(f"layer {li} down", t["down"], d_ref,
                               gemm_tol(t["act"], lw["wdown"], d_ref))
    same("residual add 2", t["h_out"], oracle.add(t["h_mid"], t["down"], True))
    return out


def whole_layer_gap(om, li, h_in, pos, kp, vp, h_out):
    """The oracle model's layer li from the engine's input residual row
    (one request); returns max |engine - oracle| / max |oracle| of the
    output row.  The oracle's pool for this layer gets the engine's pages
    first (the layer then writes its own K and V for the row's slot)."""
    npg = kp.shape[0]
    om.k[li, :npg], om.v[li, :npg] = kp, vp
    ref = om.layer(li, h_in, list(range(npg)), pos)
    return float(np.max(np.abs(h_out - ref)) / np.max(np.abs(ref)))


def tap_rows(rows):
    """An Engine.forward tap that keeps the given packed rows of every
    buffer it is shown, as float32 numpy, keyed (name, layer)."""
    store = {}
    idx = None

    def tap(name, li, t):
        nonlocal idx
        if idx is None or idx.device != t.device:
            idx = torch.tensor(rows, dtype=torch.long, device=t.device)
        store[(name, li)] = t.reshape(t.shape[0], -1)[idx].float().cpu().numpy()
    return tap, store


def layer_taps(store, li):
    return {name: v for (name, l_), v in store.items() if l_ == li}
