"""GPU tests of the batch-adaptive twins (bi_*_free) through the C ABI.

The twins compute the same mathematics as the invariant kernels but take
their split points from the batch (split-K and split-row partials merged by
fp32 atomics, decode split length from the occupancy policy, prefill chunk
boundaries counted from the prompt cut, chunks merged last to first).  So:
  - each twin matches the oracle within the bound of a reordered fp32
    reduction, and bit for bit where every order gives the exact result
    (integer-valued GEMM inputs);
  - negative control: a request's result moves with the batch (or the cut)
    under the twin, on the same inputs where the invariant kernel is
    bit-stable.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import PagedKV, bits_equal, dev, gemm_bf16_tol, gemm_f32_tol, scale_for, to_np

pytestmark = pytest.mark.gpu
L = pytest.importorskip("invariant_bi_rmsnorm_amd._lib")
DT = {"bf16": torch.bfloat16, "f32": torch.float32}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load()


def _close(g, o, rtol, atol_frac):
    """|g - o| <= rtol |o| + atol_frac max|o| elementwise."""
    g, o = np.asarray(g, np.float64), np.asarray(o, np.float64)
    bound = rtol * np.abs(o) + atol_frac * np.max(np.abs(o)) + 1e-30
    bad = np.abs(g - o) > bound
    return not bad.any(), f"{bad.sum()} of {bad.size} outside; worst {np.max(np.abs(g - o) / bound):.3g}x"


# ---------------------------------------------------------------------------
# RMSNorm twin
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("M,d", [(1, 4096), (7, 4096), (300, 4096), (5, 264)])
def test_rmsnorm_free_matches_oracle(dt, M, d):
    x = synth.normal((M, d), seed=M + d).to(DT[dt])
    g = synth.normal((d,), seed=3).to(DT[dt])
    y = torch.empty((M, d), dtype=DT[dt], device=dev())
    L.bi_rmsnorm_free(x.to(dev()), g.to(dev()), y, 1e-5)
    ref = oracle.rmsnorm(x, g, 1e-5, round_bf16=(dt == "bf16"))
    # r = 1/sqrt(ss/d + eps) moves by a few fp32 ulps under reordering;
    # bf16 outputs may then sit one bf16 ulp apart
    ok, msg = _close(to_np(y), ref, 2.0 ** -7 if dt == "bf16" else 1e-5, 0.0)
    assert ok, msg


def test_rmsnorm_free_moves_with_batch():
    d = 4096
    x = synth.normal((300, d), seed=21)
    g = synth.normal((d,), seed=22)
    xd, gd = x.to(dev()), g.to(dev())
    big = torch.empty_like(xd)
    L.bi_rmsnorm_free(xd, gd, big, 1e-5)
    alone_free, alone_inv, big_inv = [], [], torch.empty_like(xd)
    L.bi_rmsnorm(xd, gd, big_inv, 1e-5)
    # one row at a time: the twin splits each row over 16 workgroups that meet
    # through atomics; a different order of the sum of squares often still
    # rounds to the same 1/rms, so the negative control looks at all 300 rows
    for r in range(300):
        y = torch.empty((1, d), device=dev())
        L.bi_rmsnorm_free(xd[r:r + 1].contiguous(), gd, y, 1e-5)
        alone_free.append(y)
        y2 = torch.empty((1, d), device=dev())
        L.bi_rmsnorm(xd[r:r + 1].contiguous(), gd, y2, 1e-5)
        alone_inv.append(y2)
    alone_free = to_np(torch.cat(alone_free))
    alone_inv = to_np(torch.cat(alone_inv))
    assert bits_equal(alone_inv, to_np(big_inv))
    assert not bits_equal(alone_free, to_np(big))


# ---------------------------------------------------------------------------
# GEMM twin
# ---------------------------------------------------------------------------

GEMM_FREE = [(1, 4096, 4096), (7, 6144, 4096), (33, 4096, 4096), (64, 28672, 4096),
             (16, 4096, 14336), (3, 1000, 1024), (128, 4096, 4096), (200, 6144, 4104)]


@pytest.mark.parametrize("M,N,K", GEMM_FREE)
def test_gemm_free_integer_exact(M, N, K):
    # integers in [-8, 8]: every partial sum is exact in fp32, so any split
    # and any order of adding the slices must give the oracle's value bit
    # for bit
    A = synth.integers((M, K), -8, 8, seed=M + 1).to(torch.bfloat16)
    W = synth.integers((N, K), -8, 8, seed=N + 2).to(torch.bfloat16)
    C = torch.empty((M, N), dtype=torch.float32, device=dev())
    L.bi_gemm_free(A.to(dev()), W.to(dev()), C)
    ref = oracle.gemm(A, W, round_bf16=False)
    assert bits_equal(to_np(C), ref)


@pytest.mark.parametrize("M,N,K", GEMM_FREE[:4])
def test_gemm_free_tolerance(M, N, K):
    A = synth.normal((M, K), seed=M + 5).to(torch.bfloat16)
    W = synth.normal((N, K), seed=N + 6, std=0.02).to(torch.bfloat16)
    C = torch.empty((M, N), dtype=torch.bfloat16, device=dev())
    L.bi_gemm_free(A.to(dev()), W.to(dev()), C)
    ref = oracle.gemm(A, W, round_bf16=True)
    a, w = A.float().numpy(), W.float().numpy()
    assert np.all(np.abs(to_np(C) - ref) <= gemm_bf16_tol(a, w, ref))
    C32 = torch.empty((M, N), dtype=torch.float32, device=dev())
    L.bi_gemm_free(A.to(dev()), W.to(dev()), C32)
    ref32 = oracle.gemm(A, W, round_bf16=False)
    assert np.all(np.abs(to_np(C32) - ref32) <= gemm_f32_tol(a, w))


def test_gemm_free_moves_with_batch():
    # the twin's split count follows the rows (eight K slices for one row,
    # four for 128 at N = K = 4096), so a row's bits move with the batch
    M, N, K = 128, 4096, 4096
    A = synth.normal((M, K), seed=31).to(torch.bfloat16).to(dev())
    W = synth.normal((N, K), seed=32, std=0.02).to(torch.bfloat16).to(dev())
    big = torch.empty((M, N), dtype=torch.float32, device=dev())
    L.bi_gemm_free(A, W, big)
    one = torch.empty((1, N), dtype=torch.float32, device=dev())
    differs = 0
    for r in range(8):
        L.bi_gemm_free(A[r:r + 1].contiguous(), W, one)
        differs += not bits_equal(to_np(one), to_np(big)[r:r + 1])
    assert differs > 0


# ---------------------------------------------------------------------------
# decode attention twin
# ---------------------------------------------------------------------------

def _decode_free(q, kv, kv_len, scale, max_kv=None):
    k, v, bt = kv.to(dev())
    out = torch.empty(q.shape, dtype=q.dtype, device=dev())
    kvl = torch.as_tensor(kv_len, dtype=torch.int32).to(dev())
    L.bi_decode_attn_free(q.to(dev()), k, v, bt, kvl, int(max_kv or max(kv_len)), scale, out)
    return out


@pytest.mark.parametrize("dt,h,h_kv,d_h", [("f32", 32, 8, 128), ("bf16", 32, 8, 128),
                                           ("f32", 4, 2, 64)])
@pytest.mark.parametrize("B", [1, 5, 64])
def test_decode_attn_free_matches_oracle(dt, h, h_kv, d_h, B):
    kv_len = synth.log_uniform_lengths(B, 16, 3000, seed=B + d_h)
    kv = PagedKV(kv_len, h_kv, d_h, 16, seed=600 + B, dtype=DT[dt])
    q = synth.normal((B, h, d_h), seed=13).to(DT[dt])
    scale = scale_for(d_h)
    out = _decode_free(q, kv, kv_len, scale)
    bf = dt == "bf16"
    ref = oracle.decode_attn(q, kv.k, kv.v, kv.bt, kv_len, h_kv, 16, 256, scale,
                             round_bf16=bf, p_bf16=bf)
    if bf:
        # matrix-core chunks of the twin's own lengths: the derived bound
        from oracle.bounds import attn_bound
        bound = attn_bound(q, kv.k, kv.v, kv.bt, kv_len, h_kv, 16, 256, scale, True)
        err = np.abs(to_np(out) - ref)
        assert np.all(err <= bound), f"worst {np.max(err / (bound + 1e-30)):.3g}x of the bound"
    else:
        # other split points: fp32 reordering of sums over <= 3000 keys
        ok, msg = _close(to_np(out), ref, 0.0, 5e-5)
        assert ok, msg


def test_decode_attn_free_moves_with_batch():
    B, h, h_kv, d_h = 64, 32, 8, 128
    kv_len = synth.log_uniform_lengths(B, 128, 4000, seed=41)
    kv = PagedKV(kv_len, h_kv, d_h, 16, seed=42, dtype=torch.float32)
    q = synth.normal((B, h, d_h), seed=43)
    scale = scale_for(d_h)
    big = to_np(_decode_free(q, kv, kv_len, scale))
    differs = 0
    for r in range(8):
        sub = PagedKV.__new__(PagedKV)
        sub.k, sub.v, sub.page_size = kv.k, kv.v, 16
        sub.bt = kv.bt[r:r + 1].contiguous()
        one = to_np(_decode_free(q[r:r + 1].contiguous(), sub, kv_len[r:r + 1], scale))
        differs += not bits_equal(one, big[r:r + 1])
    assert differs > 0


def test_merge_partials_free_matches_oracle_and_differs_from_serial():
    B, h, h_kv, d_h, C = 12, 8, 2, 128, 256
    kv_len = synth.uniform_lengths(B, 600, 3000, seed=51)
    kv = PagedKV(kv_len, h_kv, d_h, 16, seed=52, dtype=torch.float32)
    q = synth.normal((B, h, d_h), seed=53)
    scale = scale_for(d_h)
    off = L.bi_chunk_offsets(kv_len, C)
    rml, racc = oracle.decode_partials(q, kv.k, kv.v, kv.bt, kv_len, off, h_kv, 16, C, scale)
    ref = oracle.merge_partials(rml, racc, off, round_bf16=False)
    ml, acc, offd = (torch.from_numpy(rml).to(dev()), torch.from_numpy(racc).to(dev()),
                     off.to(dev()))
    out = torch.empty((B, h, d_h), device=dev())
    L.bi_merge_partials_free(ml, acc, offd, out)
    ok, msg = _close(to_np(out), ref, 0.0, 1e-5)
    assert ok, msg
    ser = torch.empty_like(out)
    L.bi_merge_partials(ml, acc, offd, ser)
    assert bits_equal(to_np(ser), ref)
    assert not bits_equal(to_np(out), ref)


# ---------------------------------------------------------------------------
# prefill attention twin
# ---------------------------------------------------------------------------

def _prefill_free(q, kv_k, kv_v, bt, cuts, scale):
    qs = torch.tensor(cuts, dtype=torch.int32, device=dev())
    p0 = torch.tensor(cuts[:-1], dtype=torch.int32, device=dev())
    btr = bt.repeat(len(cuts) - 1, 1).contiguous()
    out = torch.empty_like(q)
    L.bi_prefill_attn_free(q, qs, p0, kv_k, kv_v, btr, scale, out)
    return out


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_prefill_free_matches_oracle_and_moves_with_cuts(dt):
    Lq, h, h_kv, d_h = 900, 32, 8, 128
    kv = PagedKV(np.array([Lq], np.int32), h_kv, d_h, 16, seed=61, dtype=DT[dt])
    q = synth.normal((Lq, h, d_h), seed=62).to(DT[dt])
    k, v, bt = kv.to(dev())
    qd = q.to(dev())
    scale = scale_for(d_h)
    bf = dt == "bf16"
    ref = oracle.prefill_attn(q, np.array([0, Lq], np.int32), np.array([0], np.int32), kv.k,
                              kv.v, kv.bt, h_kv, 16, 256, scale, round_bf16=bf, p_bf16=bf)
    if bf:
        # the bound on a sample of rows (every 7th, plus the cut points' neighbours)
        from oracle.bounds import attn_bound
        rows = np.unique(np.r_[0:Lq:7, 99, 100, 101, 332, 333, 334, 699, 700, 701, Lq - 1])
        bound = attn_bound(q[rows], kv.k, kv.v, kv.bt, None, h_kv, 16, 256, scale, True,
                           positions=rows, rows_bt=np.zeros(len(rows), np.int64))
    outs = []
    for cuts in ([0, Lq], [0, 100, Lq], [0, 333, 334, 700, Lq], [0, 40, 80, Lq]):
        out = to_np(_prefill_free(qd, k, v, bt, cuts, scale))
        if bf:
            err = np.abs(out[rows] - ref[rows])
            assert np.all(err <= bound), f"{cuts}: worst {np.max(err / (bound + 1e-30)):.3g}x"
        else:
            ok, msg = _close(out, ref, 0.0, 5e-5)
            assert ok, f"{cuts}: {msg}"
        outs.append(out)
    if dt == "f32":
        assert any(not bits_equal(o, outs[0]) for o in outs[1:])
