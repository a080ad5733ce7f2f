"""Pin of the oracle's model composition (oracle/llama.py) to something
other than itself.

The reference below is a float64 forward of a Llama-style decoder written
from the layer definition alone -- pre-norm RMSNorm with eps inside the root
and a learned gain, a fused QKV projection split into query, key and value
heads, rotate-half rotary embedding on queries and keys (never values) with
angle p * theta^(-2i/d_h), causal softmax attention in which query head i
reads key/value head floor(i / (h / h_kv)), an output projection added to the
residual, a second pre-norm, a SwiGLU MLP (SiLU of the gate rows times the up
rows, then the down projection; the fused gate/up weight holds 8 gate rows
then the matching 8 up rows in each block of 16) added to the residual, and
a final RMSNorm
with the LM head.  It imports nothing from oracle/ and shares no code with
it: softmax over whole rows in float64, no chunks, no pages, no bf16.

The oracle runs the same tiny model in fp32 mode (no carried bf16 rounding)
in the engine's way -- paged KV, two prefill cuts that straddle a 64-key chunk
edge, then decode steps -- and every logit row it returns must agree with
the reference row at that position within TOL_F32 (max |o - r| / max |r|).

Why TOL_F32 = 1e-4.  Every fp32 operation of the oracle is within one
rounding (u = 2^-24) of its exact value, and every reduction of length K is
within gamma_K = K u / (1 - K u) of the exact sum relative to the sum of
magnitudes (Higham, ch. 3); the longest reduction here is K = 256, so one
layer's outputs carry relative errors of order 256 u = 1.5e-5 before
amplification.  The normalised activations of this small random model
amplify such errors by a modest factor through two layers.  1e-4 leaves room
for that (the measured gap is about 3e-7), and the test below shows that every
planted wiring mistake moves the logits by more than 1000 x TOL_F32, so the
bound separates a right composition from a wrong one with a wide margin.

Planted mistakes (each made in the oracle on the CPU, each must fail):
gate and up halves swapped; a residual add dropped; RoPE applied to values;
RoPE left off the keys; the key/value heads of a GQA group swapped; the
output projection transposed; the two norm gains swapped; the final norm
left out.
"""
from __future__ import annotations

import math
from types import SimpleNamespace

import numpy as np
import pytest
import torch

import synth

TOL_F32 = 1e-4
TOL_BF16 = 2e-2     # the bf16 mode: loose sanity band only (see the test)

CFG = SimpleNamespace(d=64, h=4, h_kv=2, d_h=16, ffn=96, vocab=97, layers=2, eps=1e-5,
                      kv_chunk=64, page_size=16, rope=True, theta=500000.0)
CFG.scale = float(np.float32(1.0 / math.sqrt(CFG.d_h)))
SEQ = 96                      # positions 0..95: prefill 37 + 53 (cut at 37, chunk edge 64), 6 decodes
SCHED = [(0, 37), (37, 53)] + [(90 + i, 1) for i in range(6)]


def _weights(seed=0):
    """Random tiny model, bf16-representable values; std 1/sqrt(fan-in) so
    every sublayer contributes to the residual stream (random gains, not 1)."""
    c = CFG
    k = [seed * 100]

    def rnd(shape, std):
        k[0] += 1
        return synth.normal(shape, seed=k[0], std=std).to(torch.bfloat16).float()

    def gain(n):
        k[0] += 1
        return (1.0 + 0.25 * synth.normal((n,), seed=k[0])).to(torch.bfloat16).float()

    layers = []
    for _ in range(c.layers):
        layers.append(SimpleNamespace(
            attn_norm=gain(c.d), wqkv=rnd(((c.h + 2 * c.h_kv) * c.d_h, c.d), c.d ** -0.5),
            wo=rnd((c.d, c.h * c.d_h), (c.h * c.d_h) ** -0.5), ffn_norm=gain(c.d),
            wgu=rnd((2 * c.ffn, c.d), c.d ** -0.5), wdown=rnd((c.d, c.ffn), c.ffn ** -0.5)))
    return SimpleNamespace(embed=rnd((c.vocab, c.d), 1.0), layers=layers,
                           final_norm=gain(c.d), lm_head=rnd((c.vocab, c.d), c.d ** -0.5))


# ---------------------------------------------------------------------------
# float64 reference from the layer definition (independent of oracle/)
# ---------------------------------------------------------------------------

def _rms(x, g, eps):
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * g


def _rotate(x, pos, theta):
    """Rotary embedding, rotate-half pairing (i, i + d_h/2), x [T, heads, d_h]."""
    d_h = x.shape[-1]
    half = d_h // 2
    inv = theta ** (-2.0 * np.arange(half) / d_h)
    ang = pos[:, None].astype(np.float64) * inv[None, :]
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def reference_logits(w, tokens):
    """float64 logits of every position of the token sequence (causal)."""
    c = CFG
    f = lambda t: np.asarray(t, np.float64)  # noqa: E731
    T = len(tokens)
    pos = np.arange(T)
    h = f(w.embed)[np.asarray(tokens)]
    group = c.h // c.h_kv
    causal = np.tril(np.ones((T, T), bool))
    for lw in w.layers:
        x = _rms(h, f(lw.attn_norm), c.eps)
        qkv = x @ f(lw.wqkv).T
        q = qkv[:, :c.h * c.d_h].reshape(T, c.h, c.d_h)
        k = qkv[:, c.h * c.d_h:(c.h + c.h_kv) * c.d_h].reshape(T, c.h_kv, c.d_h)
        v = qkv[:, (c.h + c.h_kv) * c.d_h:].reshape(T, c.h_kv, c.d_h)
        q, k = _rotate(q, pos, c.theta), _rotate(k, pos, c.theta)
        att = np.empty((T, c.h, c.d_h))
        for i in range(c.h):
            g = i // group
            s = (q[:, i] @ k[:, g].T) / math.sqrt(c.d_h)
            s = np.where(causal, s, -np.inf)
            p = np.exp(s - s.max(axis=1, keepdims=True))
            att[:, i] = (p / p.sum(axis=1, keepdims=True)) @ v[:, g]
        h = h + att.reshape(T, -1) @ f(lw.wo).T
        x = _rms(h, f(lw.ffn_norm), c.eps)
        gu = (x @ f(lw.wgu).T).reshape(T, c.ffn // 8, 2, 8)   # blocks of 8 gate, 8 up
        gate, up = gu[:, :, 0].reshape(T, c.ffn), gu[:, :, 1].reshape(T, c.ffn)
        h = h + (gate / (1.0 + np.exp(-gate)) * up) @ f(lw.wdown).T
    return _rms(h, f(w.final_norm), c.eps) @ f(w.lm_head).T


# ---------------------------------------------------------------------------
# the oracle under test, driven as the engine drives a request
# ---------------------------------------------------------------------------

def _oracle_rows(w, tokens, bf16=False, model_hook=None):
    import oracle.llama as OL
    cos_t, sin_t = synth.rope_tables(128, CFG.d_h, CFG.theta)
    om = OL.OracleModel(CFG, w, num_pages=16, cos_t=cos_t, sin_t=sin_t, bf16=bf16)
    if model_hook is not None:
        model_hook(om)
    rng = np.random.default_rng(7)
    pages = [int(p) for p in rng.permutation(16)[:SEQ // CFG.page_size]]
    rows = {}
    for p0, n in SCHED:
        if model_hook is not None and hasattr(om, "_pos_hook"):
            om._pos_hook(p0, n)
        logits, _ = om.forward(pages, p0, tokens[p0:p0 + n])
        rows[p0 + n - 1] = np.asarray(logits, np.float64)
    return rows


def _rel_err(rows, ref):
    return max(float(np.max(np.abs(r - ref[p])) / np.max(np.abs(ref[p]))) for p, r in rows.items())


@pytest.fixture(scope="module")
def case():
    w = _weights(0)
    tokens = [int(t) for t in synth.token_ids(SEQ, CFG.vocab, seed=3)]
    return w, tokens, reference_logits(w, tokens)


def test_oracle_model_matches_float64_forward(case):
    w, tokens, ref = case
    err = _rel_err(_oracle_rows(w, tokens), ref)
    print(f"oracle (fp32 mode) vs float64 forward: {err:.2e}")
    assert err <= TOL_F32, err


def test_oracle_model_bf16_mode_stays_near_float64_forward(case):
    """The bf16 mode is the same wiring with bf16 carried between operations
    (each rounding within 2^-9 relative, pinned with the primitives); over two
    layers the logits stay within a few percent of the float64 forward.  This
    is a sanity band, not the pin: the pin is the fp32-mode test above."""
    w, tokens, ref = case
    err = _rel_err(_oracle_rows(w, tokens, bf16=True), ref)
    print(f"oracle (bf16 mode) vs float64 forward: {err:.2e}")
    assert err <= TOL_BF16, err


def _swap_gate_up(t):
    """Gate rows and up rows exchanged in every 16-row block of the weight."""
    return t.reshape(t.shape[0] // 16, 2, 8, t.shape[1]).flip(1).reshape(t.shape)


def _mut_weights(w, **kw):
    out = SimpleNamespace(embed=w.embed, final_norm=w.final_norm, lm_head=w.lm_head,
                          layers=[SimpleNamespace(**vars(lw)) for lw in w.layers])
    for key, fn in kw.items():
        for lw in out.layers:
            setattr(lw, key, fn(lw))
    return out


def _swap_kv_heads(lw):
    """Exchange kv heads 0 and 1 in the key and value rows of W_qkv: query
    head 0 then reads what the definition calls kv head 1."""
    c = CFG
    t = lw.wqkv.clone()
    for base in (c.h * c.d_h, (c.h + c.h_kv) * c.d_h):
        a = t[base:base + c.d_h].clone()
        t[base:base + c.d_h] = t[base + c.d_h:base + 2 * c.d_h]
        t[base + c.d_h:base + 2 * c.d_h] = a
    return t


def _rope_on_values(om):
    """The oracle's QKV product is wrapped so that the value columns also get
    the rotation of their positions."""
    c = CFG
    inner = om.gemm
    state = {}
    om._pos_hook = lambda p0, n: state.update(pos=np.arange(p0, p0 + n, dtype=np.int32))

    def g(A, W, rb):
        out = inner(A, W, rb)
        if W.shape[0] == (c.h + 2 * c.h_kv) * c.d_h:
            import oracle
            n = out.shape[0]
            v0 = (c.h + c.h_kv) * c.d_h
            v = out[:, v0:].reshape(n, c.h_kv, c.d_h)
            out = out.copy()
            out[:, v0:] = oracle.rope(v, state["pos"], om.cos, om.sin, rb).reshape(n, -1)
        return out
    om.gemm = g


def _rope_q_only(monkeypatch):
    import oracle.llama as OL
    real = OL.rope
    calls = [0]

    def r(x, *a):
        calls[0] += 1
        return real(x, *a) if calls[0] % 2 == 1 else np.asarray(x, np.float32)
    monkeypatch.setattr(OL, "rope", r)


def _drop_residual(monkeypatch):
    import oracle.llama as OL
    real = OL.add
    calls = [0]

    def a(x, y, rb):
        calls[0] += 1       # the second add of every layer loses its residual
        return real(x, y, rb) if calls[0] % 2 == 1 else np.asarray(y, np.float32)
    monkeypatch.setattr(OL, "add", a)


def _no_final_norm(monkeypatch):
    import oracle.llama as OL
    real = OL.rmsnorm

    def n(x, g, eps, rb):
        if g is n.final:
            return np.asarray(x, np.float32)
        return real(x, g, eps, rb)
    n.final = None
    monkeypatch.setattr(OL, "rmsnorm", n)
    return n


MUTATIONS = ["gate_up_swapped", "residual_dropped", "rope_on_values", "rope_q_only",
             "kv_heads_swapped", "wo_transposed", "norm_gains_swapped", "final_norm_missing"]


@pytest.mark.parametrize("mutation", MUTATIONS)
def test_planted_wiring_mistake_fails_the_pin(case, mutation, monkeypatch):
    w, tokens, ref = case
    hook = None
    if mutation == "gate_up_swapped":
        w = _mut_weights(w, wgu=lambda lw: _swap_gate_up(lw.wgu))
    elif mutation == "residual_dropped":
        _drop_residual(monkeypatch)
    elif mutation == "rope_on_values":
        hook = _rope_on_values
    elif mutation == "rope_q_only":
        _rope_q_only(monkeypatch)
    elif mutation == "kv_heads_swapped":
        w = _mut_weights(w, wqkv=_swap_kv_heads)
    elif mutation == "wo_transposed":
        w = _mut_weights(w, wo=lambda lw: lw.wo.T.contiguous())
    elif mutation == "norm_gains_swapped":
        w = _mut_weights(w, attn_norm=lambda lw: lw.ffn_norm, ffn_norm=lambda lw: lw.attn_norm)
    elif mutation == "final_norm_missing":
        n = _no_final_norm(monkeypatch)

        def hook(om):
            n.final = om.final_norm
    err = _rel_err(_oracle_rows(w, tokens, model_hook=hook), ref)
    print(f"{mutation}: {err:.2e}")
    assert err > 1000 * TOL_F32, f"{mutation} not caught: {err}"
