"""The products with the residual add + RMSNorm in their prologue
(bi_norm_gemm, bi_norm_gemm_swiglu, bi_norm_gemm_qkv_rope) against the two
launches they replace, bit for bit: bi_add_rmsnorm (or bi_rmsnorm) and then
bi_gemm / bi_gemm_swiglu / bi_gemm_qkv_rope.  Those are themselves held to
the oracle by test_gpu_kernels.py; the new residual and the normalised rows
are also compared with the oracle here."""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import bits_equal, dev, mismatch_report, to_np

pytestmark = pytest.mark.gpu

L = pytest.importorskip("invariant_bi_rmsnorm_amd._lib")

EPS = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load()
    yield
    torch.cuda.synchronize()


def _rows(M, K, seed):
    h = synth.normal((M, K), seed=seed).to(torch.bfloat16)
    o = synth.normal((M, K), seed=seed + 1, std=0.5).to(torch.bfloat16)
    g = synth.normal((K,), seed=seed + 2).to(torch.bfloat16)
    return h, o, g


def _two_launch_norm(h, o, g):
    """(h after the add or None, x) by the standalone norm kernels."""
    hd = h.to(dev())
    x = torch.empty_like(hd)
    if o is None:
        L.bi_rmsnorm(hd, g.to(dev()), x, EPS)
        return None, x
    L.bi_add_rmsnorm(hd, o.to(dev()), g.to(dev()), x, EPS)
    return hd, x


def _fused_bufs(h, o):
    hd = h.to(dev())
    od = o.to(dev()) if o is not None else None
    h_out = torch.full_like(hd, 7.0) if o is not None else None
    x_out = torch.full_like(hd, 7.0)
    return hd, od, h_out, x_out


def _check_norm_side(h, o, g, hd, h_out, x_out, h_ref, x_ref):
    # the inputs are untouched, the outputs are the norm kernels' and the oracle's
    assert bits_equal(to_np(hd), to_np(h))
    assert bits_equal(to_np(x_out), to_np(x_ref)), mismatch_report(to_np(x_out), to_np(x_ref))
    rh = oracle.add(h, o, round_bf16=True) if o is not None else to_np(h)
    if o is not None:
        assert bits_equal(to_np(h_out), to_np(h_ref))
        assert bits_equal(to_np(h_out), rh)
    assert bits_equal(to_np(x_out), oracle.rmsnorm(rh, g, EPS, round_bf16=True))


# (M, N, K): the decode batch sizes up to the limit at the Llama-3-8B widths,
# K not a multiple of 64 (a partial last line), K past 2048 by one vector
# (lane 0 alone holds a second vector), tiny K, N not a multiple of 16
NORM_SHAPES = [(1, 4096, 4096), (2, 6144, 4096), (3, 1000, 4096), (4, 4096, 4096),
               (1, 128256, 4096), (4, 100, 520), (3, 40, 2056), (2, 33, 8), (1, 16, 40)]


@pytest.mark.parametrize("M,N,K", NORM_SHAPES)
@pytest.mark.parametrize("add", [True, False])
@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_norm_gemm_equals_norm_then_gemm(M, N, K, add, out):
    h, o, g = _rows(M, K, seed=M * 31 + K + N)
    o = o if add else None
    W = synth.normal((N, K), seed=N + K, std=0.05).to(torch.bfloat16).to(dev())
    odt = torch.bfloat16 if out == "bf16" else torch.float32
    h_ref, x_ref = _two_launch_norm(h, o, g)
    C_ref = torch.empty((M, N), dtype=odt, device=dev())
    L.bi_gemm(x_ref, W, C_ref)
    hd, od, h_out, x_out = _fused_bufs(h, o)
    C = torch.full((M, N), 7.0, dtype=odt, device=dev())
    L.bi_norm_gemm(hd, od, g.to(dev()), EPS, h_out, x_out, W, C)
    assert bits_equal(to_np(C), to_np(C_ref)), mismatch_report(to_np(C), to_np(C_ref))
    _check_norm_side(h, o, g, hd, h_out, x_out, h_ref, x_ref)


def test_norm_gemm_without_x_out_and_repeated_calls():
    """x_out may be NULL; calls of different M on the same buffers in a row
    each give the two launches' bits."""
    K, N = 4096, 4096
    W = synth.normal((N, K), seed=3, std=0.05).to(torch.bfloat16).to(dev())
    for M in (4, 1, 3, 2):
        h, o, g = _rows(M, K, seed=100 + M)
        h_ref, x_ref = _two_launch_norm(h, o, g)
        C_ref = torch.empty((M, N), dtype=torch.bfloat16, device=dev())
        L.bi_gemm(x_ref, W, C_ref)
        hd, od, h_out, _ = _fused_bufs(h, o)
        C = torch.empty_like(C_ref)
        L.bi_norm_gemm(hd, od, g.to(dev()), EPS, h_out, None, W, C)
        assert bits_equal(to_np(C), to_np(C_ref)), f"M={M}"
        assert bits_equal(to_np(h_out), to_np(h_ref)), f"M={M}"


@pytest.mark.parametrize("M,I,K", [(1, 14336, 4096), (4, 14336, 4096), (3, 1000, 520),
                                   (2, 8, 40)])
@pytest.mark.parametrize("add", [True, False])
def test_norm_gemm_swiglu_equals_norm_then_swiglu(M, I, K, add):
    h, o, g = _rows(M, K, seed=M * 7 + I + K)
    o = o if add else None
    W = synth.normal((2 * I, K), seed=I + K, std=0.05).to(torch.bfloat16).to(dev())
    h_ref, x_ref = _two_launch_norm(h, o, g)
    act_ref = torch.empty((M, I), dtype=torch.bfloat16, device=dev())
    L.bi_gemm_swiglu(x_ref, W, act_ref)
    hd, od, h_out, x_out = _fused_bufs(h, o)
    act = torch.full_like(act_ref, 7.0)
    L.bi_norm_gemm_swiglu(hd, od, g.to(dev()), EPS, h_out, x_out, W, act)
    assert bits_equal(to_np(act), to_np(act_ref)), mismatch_report(to_np(act), to_np(act_ref))
    _check_norm_side(h, o, g, hd, h_out, x_out, h_ref, x_ref)


@pytest.mark.parametrize("M,h_q,h_kv,d_h,K", [(1, 32, 8, 128, 4096), (4, 32, 8, 128, 4096),
                                              (3, 4, 2, 64, 520), (2, 3, 1, 16, 40)])
@pytest.mark.parametrize("add", [True, False])
@pytest.mark.parametrize("tables", [True, False])
def test_norm_gemm_qkv_rope_equals_norm_then_qkv_rope(M, h_q, h_kv, d_h, K, add, tables):
    ps, seed = 16, M + K + d_h
    h, o, g = _rows(M, K, seed=seed)
    o = o if add else None
    W = synth.normal(((h_q + 2 * h_kv) * d_h, K), seed=seed + 1, std=0.05)
    W = W.to(torch.bfloat16).to(dev())
    rng = np.random.default_rng(seed)
    pages = M + 3
    slots = torch.from_numpy(rng.choice(pages * ps, size=M, replace=False).astype(np.int32))
    pos = torch.from_numpy(rng.integers(0, 4096, size=M).astype(np.int32))
    slots, pos = slots.to(dev()), pos.to(dev())
    cos_t, sin_t = synth.rope_tables(4096, d_h)
    cos_t, sin_t = (cos_t.to(dev()), sin_t.to(dev())) if tables else (None, None)
    kp = synth.normal((pages, h_kv, ps, d_h), seed=seed + 2).to(torch.bfloat16).to(dev())
    vp = synth.normal((pages, h_kv, ps, d_h), seed=seed + 3).to(torch.bfloat16).to(dev())
    kp2, vp2 = kp.clone(), vp.clone()
    h_ref, x_ref = _two_launch_norm(h, o, g)
    q_ref = torch.empty((M, h_q, d_h), dtype=torch.bfloat16, device=dev())
    L.bi_gemm_qkv_rope(x_ref, W, h_q, h_kv, d_h, pos, cos_t, sin_t, slots, q_ref, kp2, vp2)
    hd, od, h_out, x_out = _fused_bufs(h, o)
    q = torch.full_like(q_ref, 7.0)
    L.bi_norm_gemm_qkv_rope(hd, od, g.to(dev()), EPS, h_out, x_out, W, h_q, h_kv, d_h, pos,
                            cos_t, sin_t, slots, q, kp, vp)
    assert bits_equal(to_np(q), to_np(q_ref)), mismatch_report(to_np(q), to_np(q_ref))
    assert bits_equal(to_np(kp), to_np(kp2)) and bits_equal(to_np(vp), to_np(vp2))
    _check_norm_side(h, o, g, hd, h_out, x_out, h_ref, x_ref)


def test_norm_gemm_rejects_what_it_does_not_cover():
    K, N = 4096, 64
    W = torch.zeros((N, K), dtype=torch.bfloat16, device=dev())
    g = torch.ones(K, dtype=torch.bfloat16, device=dev())
    h5 = torch.zeros((5, K), dtype=torch.bfloat16, device=dev())
    with pytest.raises(L.BiError) as e:            # more rows than the prologue holds
        L.bi_norm_gemm(h5, h5.clone(), g, EPS, torch.empty_like(h5), None, W,
                       torch.empty((5, N), dtype=torch.bfloat16, device=dev()))
    assert e.value.status == L.BI_ERR_UNSUPPORTED
    Kb = 4104
    hb = torch.zeros((1, Kb), dtype=torch.bfloat16, device=dev())
    with pytest.raises(L.BiError) as e:            # K past the LDS rows
        L.bi_norm_gemm(hb, None, torch.ones(Kb, dtype=torch.bfloat16, device=dev()), EPS, None,
                       None, torch.zeros((N, Kb), dtype=torch.bfloat16, device=dev()),
                       torch.empty((1, N), dtype=torch.bfloat16, device=dev()))
    assert e.value.status == L.BI_ERR_UNSUPPORTED
    h1 = torch.zeros((1, K), dtype=torch.bfloat16, device=dev())
    with pytest.raises(L.BiError) as e:            # the new residual over the old one
        L.bi_norm_gemm(h1, h1.clone(), g, EPS, h1, None, W,
                       torch.empty((1, N), dtype=torch.bfloat16, device=dev()))
    assert e.value.status == L.BI_ERR_INVALID
