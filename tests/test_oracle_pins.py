"""Pins for the CPU oracle (no GPU).

Each check ties the oracle to something other than itself: values printed on
the pages (tests/golden), closed forms, library routines for the special
cases they cover (torch's bfloat16 cast, numpy's argmax and binary32 add),
exact integer arithmetic, and float64 brute force within derived error
bounds.  The cases are chosen so that a plausible mistake -- a dropped term,
a wrong sign or index, a transposed operand, a lost fma, a wrong query-group
mapping, a shifted chunk boundary -- fails at least one of them.
"""
import math
import struct
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth
from conftest import golden

U = 2.0 ** -24  # unit roundoff of binary32


def f32_from_hex(h):
    return struct.unpack("<f", struct.pack("<I", int(h, 16)))[0]


def hex_of(x):
    return struct.unpack("<I", struct.pack("<f", x))[0]


# --------------------------------------------------------------------------
# Figure 1 witness: serial and pairwise binary32 sums differ in ulps
# --------------------------------------------------------------------------

def test_figure1_witness_serial_vs_pairwise():
    g = golden("witness_fig1.txt")
    p = np.array([f32_from_hex(h) for h in g["input_hex"].split()], dtype=np.float32)
    serial = oracle.sum_serial(p)
    pairwise = oracle.sum_pairwise(p)
    assert hex_of(serial) == int(g["serial_hex"], 16)
    assert hex_of(pairwise) == int(g["pairwise_hex"], 16)
    assert hex_of(pairwise) - hex_of(serial) == int(g["ulps_apart"])
    # printed intermediates (printed to 8 significant digits)
    assert f"{oracle.sum_serial(p[:2]):.8g}" == g["p0_plus_p1"]
    assert f"{oracle.sum_serial(p[:3]):.5g}" == g["serial_after_p2"]
    assert f"{oracle.sum_serial(p[2:]):.8g}" == g["p2_plus_p3"]
    exact = sum(Fraction(float(v)) for v in p)
    assert f"{float(exact):.8g}" == g["exact_sum"]
    # both answers exceed the exact sum; their errors have the same sign
    assert Fraction(serial) > exact and Fraction(pairwise) > exact


# --------------------------------------------------------------------------
# scalar helpers
# --------------------------------------------------------------------------

def test_bf16_rne_matches_torch_cast():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2**32, size=200000, dtype=np.uint64).astype(np.uint32)
    bits[:8] = [0x3f808000, 0x3f818000, 0x3f80ffff, 0x7f7fffff, 0x00008000, 0x80018000,
                0x7f800000, 0xff800000]  # ties to even, overflow to inf, denormals, infs
    x = bits.view(np.float32)
    finite = np.isfinite(x) | np.isinf(x)
    x = x[finite]
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).float().numpy()
    got = np.array([oracle.bf16_rne(float(v)) for v in x[:20000]], dtype=np.float32)
    assert np.array_equal(got.view(np.uint32), ref[:20000].view(np.uint32))
    assert math.isnan(oracle.bf16_rne(float("nan")))


def test_exp_accuracy_and_fixed_points():
    x = np.linspace(-103.9, 88.7, 1_000_001).astype(np.float32)
    x = np.concatenate([x, np.float32([0.0, -0.0, 1e-30, -1e-30, 0.5, -0.5, 10.0, -10.0])])
    y = oracle.exp_array(x).astype(np.float64)
    ref = np.exp(x.astype(np.float64))
    ulp = np.spacing(ref.astype(np.float32)).astype(np.float64)
    normal = ref > 1.2e-38
    assert np.max(np.abs(y - ref)[normal] / ulp[normal]) <= 1.0
    assert oracle.exp(0.0) == 1.0 and oracle.exp(-0.0) == 1.0
    assert oracle.exp(-200.0) == 0.0 and math.isinf(oracle.exp(100.0))
    assert math.isnan(oracle.exp(float("nan")))
    # monotone on a fine grid
    z = oracle.exp_array(np.linspace(-5, 5, 100001).astype(np.float32))
    assert np.all(np.diff(z) >= 0)


# --------------------------------------------------------------------------
# RMSNorm
# --------------------------------------------------------------------------

def _rms64(x, g, eps):
    x = x.astype(np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * g.astype(np.float64)


@pytest.mark.parametrize("d", [1, 2, 3, 8, 13, 256, 1000, 2048, 4096, 14336])
def test_rmsnorm_vs_fp64(d):
    x = synth.normal((5, d), seed=10 + d).numpy()
    g = synth.normal((d,), seed=20 + d).numpy()
    eps = 1e-5
    y = oracle.rmsnorm(x, g, eps, round_bf16=False)
    ref = _rms64(x, g, eps)
    nv = (d + 7) // 8
    D = ((nv + 255) // 256) * 8 + 9          # longest fma chain + tree depth
    tol = (D / 2 + 6) * U * np.abs(ref) + 1e-35
    assert np.all(np.abs(y - ref) <= tol)
    # bf16 output is the binary32 result rounded once
    yb = oracle.rmsnorm(x, g, eps, round_bf16=True)
    assert np.array_equal(yb, torch.from_numpy(y).to(torch.bfloat16).float().numpy())


def test_rmsnorm_dropped_term_is_caught():
    # a single element changes the norm measurably: the fp64 check above
    # separates a complete sum from one missing its last element
    d = 4096
    x = np.ones((1, d), np.float32)
    x[0, -1] = 8.0
    g = np.ones(d, np.float32)
    y = oracle.rmsnorm(x, g, 0.0, round_bf16=False)
    ref = _rms64(x, g, 0.0)
    ref_drop = _rms64(x[:, :-1], g[:-1], 0.0)
    assert abs(y[0, 0] - ref[0, 0]) < 1e-6 * ref[0, 0]
    assert abs(y[0, 0] - ref_drop[0, 0]) > 1e-3 * ref[0, 0]


def test_rmsnorm_constant_row_closed_form():
    for c, d in [(0.5, 4096), (3.0, 256), (-2.0, 14336)]:
        x = np.full((2, d), c, np.float32)
        g = np.full(d, 1.5, np.float32)
        y = oracle.rmsnorm(x, g, 1e-5, round_bf16=False)
        ref = c / math.sqrt(c * c + 1e-5) * 1.5
        assert np.all(np.abs(y - ref) <= 4 * U * abs(ref))


def test_rmsnorm_rows_independent():
    x = synth.normal((16, 4096), seed=3).numpy()
    g = synth.normal((4096,), seed=4).numpy()
    full = oracle.rmsnorm(x, g, 1e-5, True)
    perm = np.random.default_rng(0).permutation(16)
    part = oracle.rmsnorm(x[perm], g, 1e-5, True)
    assert np.array_equal(full[perm], part)
    assert np.array_equal(full[3:4], oracle.rmsnorm(x[3:4], g, 1e-5, True))


# --------------------------------------------------------------------------
# GEMM
# --------------------------------------------------------------------------

def test_gemm_integer_exact_against_int64():
    # integer operands in [-8, 8]: every partial sum is an integer below 2^24,
    # so every summation order is exact; pins layout, transpose and indexing
    for (M, N, K) in [(1, 16, 32), (7, 33, 96), (64, 48, 4096), (5, 128, 14336 // 4)]:
        A = synth.integers((M, K), -8, 8, seed=M + N).numpy()
        W = synth.integers((N, K), -8, 8, seed=K).numpy()
        C = oracle.gemm(A, W, round_bf16=False)
        ref = A.astype(np.int64) @ W.astype(np.int64).T
        assert np.array_equal(C.astype(np.int64), ref)


def test_gemm_one_hot_rows_reproduce_weight_columns():
    K, N = 256, 40
    W = synth.normal((N, K), seed=5).numpy()
    A = np.zeros((4, K), np.float32)
    for i, k in enumerate([0, 17, 128, 255]):
        A[i, k] = 1.0
    C = oracle.gemm(A, W, round_bf16=False)
    assert np.array_equal(C, W[:, [0, 17, 128, 255]].T)


def test_gemm_chain_order_and_fma():
    # fma(a1, w1, fma(a0, w0, 0)) with a0*w0 = -1 and a1*w1 = 1 + 2^-11 + 2^-24
    # gives 2^-11 + 2^-24 exactly; a separate multiply, or the reverse order,
    # gives 2^-11.
    e = 1.0 + 2.0 ** -12
    A = np.array([[-1.0, e]], np.float32)
    W = np.array([[1.0, e]], np.float32)
    C = oracle.gemm(A, W, round_bf16=False)
    assert C[0, 0] == np.float32(2.0 ** -11 + 2.0 ** -24)
    C_rev = oracle.gemm(A[:, ::-1], W[:, ::-1], round_bf16=False)
    assert C_rev[0, 0] == np.float32(2.0 ** -11)


@pytest.mark.parametrize("M,N,K", [(3, 17, 64), (16, 64, 512), (2, 8, 4096)])
def test_gemm_vs_fp64(M, N, K):
    A = synth.normal((M, K), seed=M).numpy()
    W = synth.normal((N, K), seed=N, std=0.02).numpy()
    C = oracle.gemm(A, W, round_bf16=False)
    ref = A.astype(np.float64) @ W.astype(np.float64).T
    bound = (K + 1) * U * (np.abs(A).astype(np.float64) @ np.abs(W).astype(np.float64).T)
    assert np.all(np.abs(C - ref) <= bound)
    Cb = oracle.gemm(A, W, round_bf16=True)
    assert np.array_equal(Cb, torch.from_numpy(C).to(torch.bfloat16).float().numpy())


# --------------------------------------------------------------------------
# split-KV attention: partials and merge
# --------------------------------------------------------------------------

def test_split_count_printed_example():
    g = golden("split_count.txt")
    assert oracle.num_chunks(int(g["seq_len"]), int(g["split_tile"])) == int(g["num_splits"])
    # depends on the request's length only
    assert oracle.num_chunks(1, 256) == 1 and oracle.num_chunks(256, 256) == 1
    assert oracle.num_chunks(257, 256) == 2


def _paged_case(kv_len, h, h_kv, d_h, page_size, seed, dtype=torch.float32):
    B = len(kv_len)
    place = synth.scatter_pages(kv_len, page_size, seed=seed)
    kpool = synth.normal((place.num_pages, h_kv, page_size, d_h), seed=seed + 1).to(dtype)
    vpool = synth.normal((place.num_pages, h_kv, page_size, d_h), seed=seed + 2).to(dtype)
    q = synth.normal((B, h, d_h), seed=seed + 3).to(dtype)
    return q.float().numpy(), kpool.float().numpy(), vpool.float().numpy(), place


def _gather(pool, bt_row, n, g, page_size):
    j = np.arange(n)
    return pool[bt_row[j // page_size], g, j % page_size]   # [n, d_h]


def _attn64(q, kpool, vpool, bt, kv_len, h_kv, page_size, scale, chunk=256):
    """fp64 softmax attention over all keys, plus a first-order error budget
    for the binary32 chunked evaluation: every weight exp(S_u - m) carries a
    relative error <= |dS_u| + u|S_u - m| + 2u, where dS_u <= (d_h + 1) u
    sum_d |q_d k_ud| scale bounds the fma-chain dot and the scale multiply;
    o = sum w v / sum w then moves by <= 2 max_u eps_u max|v|, and the block
    sums and the serial merge add (64 + 16 + 4 n_chunks) u max|v|."""
    B, h, d_h = q.shape
    grp = h // h_kv
    out = np.zeros((B, h, d_h))
    tol = 0.0
    for r in range(B):
        for i in range(h):
            K = _gather(kpool, bt[r], kv_len[r], i // grp, page_size).astype(np.float64)
            V = _gather(vpool, bt[r], kv_len[r], i // grp, page_size).astype(np.float64)
            qi = q[r, i].astype(np.float64)
            s = K @ qi * scale
            w = np.exp(s - s.max())
            out[r, i] = (w / w.sum()) @ V
            eps = (d_h + 1) * U * (np.abs(K) @ np.abs(qi)) * scale + U * np.abs(s - s.max()) + 2 * U
            nch = -(-int(kv_len[r]) // chunk)
            vmax = np.abs(V).max()
            tol = max(tol, 2 * eps.max() * vmax + (64 + 16 + 4 * nch) * U * vmax)
    return out, tol


@pytest.mark.parametrize("h,h_kv,d_h,chunk", [(4, 2, 64, 64), (8, 2, 128, 256), (4, 4, 64, 128)])
def test_decode_attention_vs_fp64(h, h_kv, d_h, chunk):
    kv_len = np.array([1, 2, 63, 64, 65, 200, 300, 513], np.int32)
    q, kp, vp, place = _paged_case(kv_len, h, h_kv, d_h, 16, seed=40 + d_h)
    scale = float(np.float32(1.0 / math.sqrt(d_h)))
    out = oracle.decode_attn(q, kp, vp, place.block_table, kv_len, h_kv, 16, chunk, scale,
                             round_bf16=False)
    ref, tol = _attn64(q, kp, vp, place.block_table, kv_len, h_kv, 16, scale, chunk)
    assert np.max(np.abs(out - ref)) <= tol
    # dropping the last key of the longest request is visible at this tolerance
    kv_short = kv_len.copy()
    kv_short[-1] -= 1
    ref_drop, _ = _attn64(q, kp, vp, place.block_table, kv_short, h_kv, 16, scale, chunk)
    assert np.max(np.abs(out[-1] - ref_drop[-1])) > 3 * tol


def _sparse_int_case(kv_len, h, h_kv, d_h, ps, seed, nnz=4):
    """q with nnz entries of +-1 per head, keys in {-1, 0, 1}: every score is
    an exact small integer, so with a power-of-two scale the weights are
    known to fp64."""
    rng = np.random.default_rng(seed)
    place = synth.scatter_pages(kv_len, ps, seed=seed + 1)
    shape = (place.num_pages, h_kv, ps, d_h)
    kp = rng.integers(-1, 2, size=shape).astype(np.float32)
    vp = synth.normal(shape, seed=seed + 2).to(torch.bfloat16).float().numpy()
    q = np.zeros((len(kv_len), h, d_h), np.float32)
    for r in range(len(kv_len)):
        for i in range(h):
            idx = rng.choice(d_h, size=nnz, replace=False)
            q[r, i, idx] = rng.choice([-1.0, 1.0], size=nnz)
    return q, kp, vp, place


def test_decode_attention_bf16_weights_pin():
    # p_bf16: the softmax weights are rounded to bf16 before the sums.  With
    # exact integer scores and a power-of-two scale, P = bf16(exp(s - m_chunk))
    # is fixed by fp64 (the check below makes sure no weight sits within a few
    # fp32 ulps of a bf16 rounding boundary, where the oracle's 1-ulp exp
    # could round the other way), so the merged output is known to within
    # the fp32 sum and merge error.  Without the rounding it moves far more.
    h, h_kv, d_h, ps, chunk = 4, 2, 64, 16, 64
    kv_len = np.array([1, 17, 64, 65, 200, 300], np.int32)
    q, kp, vp, place = _sparse_int_case(kv_len, h, h_kv, d_h, ps, seed=61)
    scale = 0.25
    out = oracle.decode_attn(q, kp, vp, place.block_table, kv_len, h_kv, ps, chunk, scale,
                             round_bf16=False, p_bf16=True)
    raw = oracle.decode_attn(q, kp, vp, place.block_table, kv_len, h_kv, ps, chunk, scale,
                             round_bf16=False, p_bf16=False)
    worst_gap = 0.0
    for r, n in enumerate(kv_len):
        for i in range(h):
            g = i // (h // h_kv)
            K = _gather(kp, place.block_table[r], int(n), g, ps)
            V = _gather(vp, place.block_table[r], int(n), g, ps)
            s = K @ q[r, i].astype(np.float64) * scale
            nch = -(-int(n) // chunk)
            m = np.array([s[c * chunk:(c + 1) * chunk].max() for c in range(nch)])
            p64 = np.concatenate([np.exp(s[c * chunk:(c + 1) * chunk] - m[c])
                                  for c in range(nch)])
            p32 = torch.from_numpy(p64.astype(np.float32))
            P = p32.to(torch.bfloat16).double().numpy()
            for k in (-4, 4):  # rounding stable under a few fp32 ulps
                moved = (p32.view(torch.int32) + k).view(torch.float32)
                assert np.array_equal(moved.to(torch.bfloat16).double().numpy(), P)
            w = np.repeat(np.exp(m - m.max()), chunk)[:int(n)]
            ref = (w * P) @ V / (w * P).sum()
            tol = 16 * (int(n) + nch + 4) * U * np.abs(V).max()
            assert np.max(np.abs(out[r, i] - ref)) <= tol
            worst_gap = max(worst_gap, float(np.max(np.abs(raw[r, i] - ref))))
    assert worst_gap > 1e-4   # the rounding is really applied


def test_decode_single_token_returns_v_exactly():
    kv_len = np.array([1, 1, 1], np.int32)
    q, kp, vp, place = _paged_case(kv_len, 8, 2, 128, 16, seed=7)
    out = oracle.decode_attn(q, kp, vp, place.block_table, kv_len, 2, 16, 256, 0.0884, False)
    for r in range(3):
        for i in range(8):
            v0 = vp[place.block_table[r, 0], i // 4, 0]
            assert np.array_equal(out[r, i], v0)


def test_equal_keys_give_exact_mean_of_integer_values():
    # every score equal -> p = 1, l = n, acc = sum of integer v (exact)
    n, d_h = 200, 64
    kp = np.zeros((16, 1, 16, d_h), np.float32)
    kp[:] = synth.normal((d_h,), seed=9).numpy()
    vp = synth.integers((16, 1, 16, d_h), -4, 4, seed=11).numpy()
    bt = np.arange(16, dtype=np.int32)[None, :]
    q = synth.normal((1, 2, d_h), seed=12).numpy()
    for chunk in (64, 256):
        out = oracle.decode_attn(q, kp, vp, bt, np.array([n], np.int32), 1, 16, chunk, 0.125, False)
        V = _gather(vp, bt[0], n, 0, 16)
        ref = np.array([float(Fraction(int(s), n)) for s in V.sum(0).astype(np.int64)], np.float32)
        assert np.array_equal(out[0, 0], ref) and np.array_equal(out[0, 1], ref)


def test_query_group_mapping():
    # kv head g carries value g+1 everywhere; query head i must read i // (h/h_kv)
    h, h_kv, d_h = 8, 4, 64
    kp = np.zeros((4, h_kv, 16, d_h), np.float32)
    vp = np.zeros_like(kp)
    for g in range(h_kv):
        vp[:, g] = g + 1
    bt = np.arange(4, dtype=np.int32)[None, :]
    q = synth.normal((1, h, d_h), seed=13).numpy()
    out = oracle.decode_attn(q, kp, vp, bt, np.array([50], np.int32), h_kv, 16, 64, 0.125, False)
    for i in range(h):
        assert np.all(out[0, i] == i // 2 + 1)


def test_merge_closed_forms():
    d_h, h = 8, 1
    acc = synth.integers((2, h, d_h), -50, 50, seed=3).numpy()
    # equal maxima: a = b = 1 -> (acc0 + acc1) / (l0 + l1), all exact integers
    ml = np.array([[[2.0, 3.0]], [[2.0, 5.0]]], np.float32)
    out = oracle.merge_partials(ml, acc, np.array([0, 2], np.int32), round_bf16=False)
    ref = np.array([float(Fraction(int(a + b), 8)) for a, b in zip(acc[0, 0], acc[1, 0])],
                   np.float32)
    assert np.array_equal(out[0, 0], ref)
    # one chunk: identity
    out1 = oracle.merge_partials(ml[:1], acc[:1], np.array([0, 1], np.int32), False)
    assert np.array_equal(out1[0, 0], (acc[0, 0] / np.float32(3.0)).astype(np.float32))
    # general maxima against the fp64 formula
    rng = np.random.default_rng(5)
    n = 7
    ml = np.stack([rng.normal(0, 3, n), rng.uniform(1, 50, n)], -1).astype(np.float32)[:, None, :]
    acc = rng.normal(0, 10, (n, 1, d_h)).astype(np.float32)
    out = oracle.merge_partials(ml, acc, np.array([0, n], np.int32), False)
    m = ml[:, 0, 0].astype(np.float64)
    w = np.exp(m - m.max())
    ref = (w[:, None] * acc[:, 0].astype(np.float64)).sum(0) / (w * ml[:, 0, 1]).sum()
    assert np.max(np.abs(out[0, 0] - ref)) <= 64 * U * np.abs(acc).max()


def test_oracle_decode_is_batch_invariant_bitwise():
    kv_len = synth.uniform_lengths(12, 1, 700, seed=21)
    q, kp, vp, place = _paged_case(kv_len, 8, 2, 128, 16, seed=22)
    args = dict(h_kv=2, page_size=16, chunk=256, scale=0.08838835, round_bf16=True)
    full = oracle.decode_attn(q, kp, vp, place.block_table, kv_len, **args)
    rng = np.random.default_rng(23)
    for _ in range(4):
        idx = rng.permutation(12)[: rng.integers(1, 13)]
        sub = oracle.decode_attn(q[idx], kp, vp, place.block_table[idx], kv_len[idx], **args)
        assert np.array_equal(sub, full[idx])


def test_prefill_equals_decode_and_ignores_chunk_cuts():
    h, h_kv, d_h, ps, C = 4, 2, 64, 16, 64
    L = 300
    kv = np.array([L], np.int32)
    place = synth.scatter_pages(kv, ps, seed=31)
    kp = synth.normal((place.num_pages, h_kv, ps, d_h), seed=32).numpy()
    vp = synth.normal((place.num_pages, h_kv, ps, d_h), seed=33).numpy()
    q = synth.normal((L, h, d_h), seed=34).numpy()
    bt = place.block_table
    whole = oracle.prefill_attn(q, np.array([0, L], np.int32), np.array([0], np.int32), kp, vp,
                                bt, h_kv, ps, C, 0.125, round_bf16=True)
    # the same prompt cut into chunks of 37, 100, 1, 162 tokens, one row per request
    cuts = [0, 37, 137, 138, L]
    q_start = np.array([0, 37, 137, 138, L], np.int32)
    pos0 = np.array(cuts[:-1], np.int32)
    bts = np.repeat(bt, 4, axis=0)
    cut = oracle.prefill_attn(q, q_start, pos0, kp, vp, bts, h_kv, ps, C, 0.125, True)
    assert np.array_equal(whole, cut)
    # row t of the prefill == a decode step with kv_len = t + 1
    for t in [0, 1, 63, 64, 65, 127, 128, 299]:
        dec = oracle.decode_attn(q[t:t + 1], kp, vp, bt, np.array([t + 1], np.int32), h_kv, ps, C,
                                 0.125, True)
        assert np.array_equal(dec[0], whole[t])


# --------------------------------------------------------------------------
# glue
# --------------------------------------------------------------------------

def test_rope_identity_at_zero_and_rotation_accuracy():
    cos_t, sin_t = synth.rope_tables(4096, 128)
    x = synth.normal((6, 4, 128), seed=41).numpy()
    pos = np.array([0, 1, 7, 100, 2048, 4095], np.int32)
    y = oracle.rope(x, pos, cos_t, sin_t, round_bf16=False)
    assert np.array_equal(y[0], x[0])
    c = cos_t.numpy().astype(np.float64)[pos][:, None, :]
    s = sin_t.numpy().astype(np.float64)[pos][:, None, :]
    a, b = x[..., :64].astype(np.float64), x[..., 64:].astype(np.float64)
    ref = np.concatenate([a * c - b * s, b * c + a * s], -1)
    mag = np.abs(a * c) + np.abs(b * s) + np.abs(b * c) + np.abs(a * s)
    assert np.all(np.abs(y - ref) <= 3 * U * np.concatenate([mag, mag], -1) + 1e-30)


def test_add_matches_binary32_add():
    a = synth.normal((1000,), seed=1).to(torch.bfloat16).float().numpy()
    b = synth.normal((1000,), seed=2).to(torch.bfloat16).float().numpy()
    y = oracle.add(a, b, round_bf16=False)
    assert np.array_equal(y, (a + b).astype(np.float32))
    yb = oracle.add(a, b, round_bf16=True)
    assert np.array_equal(yb, torch.from_numpy(a + b).to(torch.bfloat16).float().numpy())


def test_silu_mul_vs_fp64():
    gu = synth.normal((4, 2 * 300), seed=51, std=4.0).numpy()
    y = oracle.silu_mul(gu, round_bf16=False)
    g, u = gu[:, :300].astype(np.float64), gu[:, 300:].astype(np.float64)
    ref = g / (1.0 + np.exp(-g)) * u
    assert np.all(np.abs(y - ref) <= 6 * U * np.abs(ref) + 1e-30)
    z = oracle.silu_mul(np.array([[0.0, -200.0, 50.0, 2.0, 3.0, 1.5]], np.float32), False)
    assert z[0, 0] == 0.0 and z[0, 1] == 0.0 and z[0, 2] == np.float32(50.0 * 1.5)


def test_argmax_lowest_index_on_ties():
    x = synth.normal((8, 1000), seed=61).numpy()
    x[0, [5, 700]] = 10.0       # tie
    x[1, :] = 0.0               # all equal
    x[2, [3, 4]] = [np.float32(-0.0), 0.0]
    idx = oracle.argmax(x)
    assert np.array_equal(idx, np.argmax(x, axis=1))
    assert idx[0] == 5 and idx[1] == 0


def test_attention_bound_covers_weight_rounding_and_catches_a_dropped_key():
    # the bound used for matrix-core attention: two valid evaluations (weights
    # in fp32 and weights rounded to bf16) stay inside it; dropping a key of a
    # short request does not
    from oracle.bounds import attn_bound
    h, h_kv, d_h, ps, chunk = 4, 2, 64, 16, 64
    kv_len = np.array([5, 17, 64, 65, 130], np.int32)
    q, kp, vp, place = _paged_case(kv_len, h, h_kv, d_h, ps, seed=71)
    scale = float(np.float32(1.0 / math.sqrt(d_h)))
    a = oracle.decode_attn(q, kp, vp, place.block_table, kv_len, h_kv, ps, chunk, scale, False,
                           p_bf16=True)
    b = oracle.decode_attn(q, kp, vp, place.block_table, kv_len, h_kv, ps, chunk, scale, False,
                           p_bf16=False)
    bound = attn_bound(q, kp, vp, place.block_table, kv_len, h_kv, ps, chunk, scale, False)
    assert np.all(np.abs(a - b) <= bound)
    short = kv_len.copy()
    short[0] -= 1
    c = oracle.decode_attn(q, kp, vp, place.block_table, short, h_kv, ps, chunk, scale, False,
                           p_bf16=True)
    assert np.any(np.abs(c[0] - a[0]) > bound[0])


# --------------------------------------------------------------------------
# log and log-softmax (logprobs)
# --------------------------------------------------------------------------

def _ulps(a, b):
    """Distance in binary32 ulps between fp32 arrays a and b (same sign)."""
    ia = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    ib = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    return np.abs(ia - ib)


def test_log_within_two_ulps_of_fp64():
    rng = np.random.default_rng(31)
    x = np.exp(rng.uniform(-87.0, 88.0, 200000)).astype(np.float32)
    x = x[(x > 0) & np.isfinite(x) & (x >= np.finfo(np.float32).tiny)]
    x = np.concatenate([x, np.float32([1.0, 2.0, 0.5, 3.0, 1.4142135, 1.4142137, 0.70710677,
                                       np.finfo(np.float32).tiny, np.finfo(np.float32).max])])
    got = oracle.log(x)
    ref = np.log(x.astype(np.float64)).astype(np.float32)
    # near log = 0 the ulp scale shrinks; compare there in absolute terms
    far = np.abs(ref) > 1e-3
    assert _ulps(got[far], ref[far]).max() <= 2
    assert np.abs(got[~far].astype(np.float64) - np.log(x[~far].astype(np.float64))).max() < 1e-9
    assert oracle.log(np.float32([1.0]))[0] == 0.0
    k = np.arange(-126, 128)
    p = np.float32(2.0) ** k.astype(np.float32)
    assert _ulps(oracle.log(p)[k != 0], (k[k != 0] * math.log(2.0)).astype(np.float32)).max() <= 1
    assert np.isnan(oracle.log(np.float32([np.nan]))[0])
    assert oracle.log(np.float32([np.inf]))[0] == np.inf


def test_log_softmax_vs_fp64_and_closed_forms():
    rng = np.random.default_rng(32)
    x = (rng.standard_normal((4, 5003)) * 4.0).astype(np.float32)
    y = oracle.log_softmax(x)
    x64 = x.astype(np.float64)
    ref = x64 - (x64.max(1, keepdims=True) +
                 np.log(np.exp(x64 - x64.max(1, keepdims=True)).sum(1, keepdims=True)))
    assert np.abs(y - ref).max() < 4e-6
    # probabilities sum to one
    assert np.abs(np.exp(y.astype(np.float64)).sum(1) - 1.0).max() < 1e-5
    # one entry: log 1 = 0 exactly; two entries: -log(1 + e^(b - a))
    assert np.all(oracle.log_softmax(np.float32([[3.5], [-7.0]])) == 0.0)
    a, b = np.float32(1.25), np.float32(-0.5)
    y2 = oracle.log_softmax(np.float32([[a, b]]))[0].astype(np.float64)
    assert abs(y2[0] + math.log1p(math.exp(float(b) - float(a)))) < 3e-7
    assert abs(y2[1] - (float(b) - float(a)) + math.log1p(math.exp(float(b) - float(a)))) < 3e-7
    # large logits: the maximum is taken out before the exp (no overflow)
    big = oracle.log_softmax(np.float32([[1000.0, 999.0, 998.0]]))[0]
    ref3 = np.array([0.0, -1.0, -2.0]) - math.log(1 + math.exp(-1) + math.exp(-2))
    assert np.all(np.isfinite(big)) and np.abs(big - ref3).max() < 1e-6
    # masked entries: -inf stays -inf, a lone finite entry gets 0; all -inf: -inf
    mm = oracle.log_softmax(np.float32([[-np.inf, 2.0, -np.inf], [-np.inf, -np.inf, -np.inf]]))
    assert mm[0, 1] == 0.0 and mm[0, 0] == -np.inf and np.all(mm[1] == -np.inf)


def test_log_softmax_sums_in_the_stated_order():
    """The sum of exp runs lane-serially over the strided elements, then an
    xor butterfly per 64 lanes, then the 16 wave sums in order: a row whose
    terms straddle several lanes and waves reproduces bit for bit from the
    oracle's own exp and log composed in that order in binary32."""
    rng = np.random.default_rng(33)
    x = (rng.standard_normal(20000) * 3.0).astype(np.float32)
    m = x.max()
    e = np.array([oracle.exp(float(np.float32(v - m))) for v in x], np.float32)
    lane = np.zeros(1024, np.float32)
    for t in range(1024):
        a = np.float32(0.0)
        for i in range(t, x.size, 1024):
            a = np.float32(a + e[i])
        lane[t] = a
    waves = []
    for w in range(16):
        v = lane[64 * w:64 * w + 64].copy()
        for msk in (32, 16, 8, 4, 2, 1):
            v = np.float32(v + v[np.arange(64) ^ msk])
        waves.append(v[0])
    s = np.float32(waves[0])
    for w in range(1, 16):
        s = np.float32(s + waves[w])
    ls = oracle.log(np.float32([s]))[0]
    y = oracle.log_softmax(x[None, :])[0]
    assert np.array_equal(y.view(np.int32), ((x - m) - ls).astype(np.float32).view(np.int32))
    # and a serial sum of the same terms is a different binary32 value here
    ser = np.float32(0.0)
    for v in e:
        ser = np.float32(ser + v)
    assert ser != s


# --------------------------------------------------------------------------
# seeded sampling
# --------------------------------------------------------------------------

def test_murmur3_matches_library_routine():
    import struct as st
    from sklearn.utils import murmurhash3_32
    rng = np.random.default_rng(41)
    for _ in range(2000):
        seed, w0, w1 = (int(v) for v in rng.integers(0, 2**32, 3, dtype=np.uint64))
        ref = murmurhash3_32(st.pack("<II", w0, w1), seed=seed, positive=True)
        assert oracle.murmur3(seed, w0, w1) == ref
    assert oracle.murmur3(0, 0, 0) == murmurhash3_32(b"\0" * 8, seed=0, positive=True)


def test_log64_within_two_ulps_of_math_log():
    rng = np.random.default_rng(42)
    x = np.exp(rng.uniform(-700.0, 700.0, 100000))
    x = np.concatenate([x, [1.0, 2.0, 0.5, 2.0 ** -32 * 0.5, 1.0 - 2.0 ** -33, 22.9]])
    got = oracle.log64(x)
    ref = np.array([math.log(v) for v in x])
    far = np.abs(ref) > 1e-3
    ulp = np.abs(got[far].view(np.int64) - ref[far].view(np.int64))
    assert ulp.max() <= 2 and np.mean(ulp > 0) < 1e-3
    assert np.abs(got[~far] - ref[~far]).max() < 1e-18
    assert oracle.log64(np.array([1.0]))[0] == 0.0


def test_sample_distribution_and_limits():
    """Draws over many positions follow softmax(x / T) (a sign or temperature
    slip fails the chi-square bound), T -> 0+ and T <= 0 give the argmax, and a
    draw depends on (seed, position) only."""
    logits = np.float32([[1.0, 0.0, -1.0, 2.0, 0.5]])
    T = 0.7
    n = 20000
    x = np.repeat(logits, n, axis=0)
    toks = oracle.sample(x, np.full(n, 1234, np.uint32), np.arange(n), np.full(n, T, np.float32))
    p = np.exp(logits[0] / T)
    p /= p.sum()
    cnt = np.bincount(toks, minlength=5)
    chi2 = float(((cnt - n * p) ** 2 / (n * p)).sum())
    assert chi2 < 20.5           # 4 degrees of freedom, p ~ 4e-4
    am = int(np.argmax(logits[0]))
    assert np.all(oracle.sample(x[:50], np.arange(50), np.arange(50),
                                np.full(50, 1e-6, np.float32)) == am)
    assert np.all(oracle.sample(x[:5], np.arange(5), np.arange(5), np.zeros(5, np.float32)) == am)
    # same seed and position, same token; other seeds scatter
    a = oracle.sample(x[:1], [7], [9], [1.0])
    assert np.all(oracle.sample(np.repeat(logits, 8, 0), np.full(8, 7), np.full(8, 9),
                                np.ones(8, np.float32)) == a[0])
    assert len(set(oracle.sample(np.repeat(logits, 64, 0), np.arange(64), np.full(64, 9),
                                 np.ones(64, np.float32)).tolist())) > 1
    # masked entries are never drawn
    xm = np.repeat(np.float32([[0.0, -np.inf, 0.0]]), 500, 0)
    assert not np.any(oracle.sample(xm, np.arange(500), np.arange(500),
                                    np.ones(500, np.float32)) == 1)
