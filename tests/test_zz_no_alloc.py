"""bi_decode_attn_noalloc (partials in the library's static device buffer)
against bi_decode_attn + bi_merge_partials with caller workspace: bit for
bit, on two calls in a row, the second smaller than the first (so the
buffer holds the first call's partials when the second reads it), in bf16
(matrix-core path, d_h 128, 256-key chunks, batch 64) and fp32 (d_h 64,
64-key chunks); and a request that would overflow the buffer is refused
before any launch."""
import numpy as np
import pytest
import torch

import synth
from helpers import PagedKV, dev, scale_for

pytestmark = pytest.mark.gpu
L = pytest.importorskip("invariant_bi_rmsnorm_amd._lib")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load()


def _both(B, h, h_kv, d_h, C, dtype, seed, lo, hi):
    kv_len = synth.uniform_lengths(B, lo, hi, seed=seed)
    kv = PagedKV(kv_len, h_kv, d_h, 16, seed=seed + 1, dtype=dtype)
    kp, vp, bt = kv.to(dev())
    q = synth.normal((B, h, d_h), seed=seed + 2).to(dtype).to(dev())
    off = L.bi_chunk_offsets(kv_len, C)
    tot = int(off[-1])
    offd, kvd = off.to(dev()), torch.from_numpy(kv_len).to(dev())
    ml = torch.empty((tot, h, 2), device=dev())
    acc = torch.empty((tot, h, d_h), device=dev())
    ref = torch.empty((B, h, d_h), dtype=dtype, device=dev())
    L.bi_decode_attn(q, kp, vp, bt, kvd, offd, tot, C, scale_for(d_h), ml, acc)
    L.bi_merge_partials(ml, acc, offd, ref)
    got = torch.full((B, h, d_h), float("nan"), dtype=dtype, device=dev())
    L.bi_decode_attn_noalloc(q, kp, vp, bt, kvd, offd, tot, C, scale_for(d_h), got)
    torch.cuda.synchronize()
    return got, ref, tot


@pytest.mark.parametrize("dtype,h,h_kv,d_h,C", [(torch.bfloat16, 32, 8, 128, 256),
                                                 (torch.float32, 8, 2, 64, 64)])
def test_noalloc_decode_equals_decode_plus_merge_twice(dtype, h, h_kv, d_h, C):
    view = torch.int16 if dtype == torch.bfloat16 else torch.int32
    for call, (B, lo, hi) in enumerate([(64, 32, 4096), (7, 1, 600)]):
        got, ref, tot = _both(B, h, h_kv, d_h, C, dtype, seed=10 * call + 1, lo=lo, hi=hi)
        assert tot * h * (d_h + 2) * 4 <= L.NOALLOC_SCRATCH_BYTES
        assert torch.equal(got.view(view), ref.view(view)), f"call {call} (B={B})"


def test_noalloc_refuses_partials_beyond_the_buffer():
    h, h_kv, d_h, C = 32, 8, 128, 256
    B = 2
    q = torch.zeros((B, h, d_h), dtype=torch.bfloat16, device=dev())
    kp = torch.zeros((4, h_kv, 16, d_h), dtype=torch.bfloat16, device=dev())
    bt = torch.zeros((B, 4), dtype=torch.int32, device=dev())
    kvl = torch.ones(B, dtype=torch.int32, device=dev())
    off = torch.tensor([0, 1, 2], dtype=torch.int32, device=dev())
    out = torch.zeros((B, h, d_h), dtype=torch.bfloat16, device=dev())
    too_many = L.NOALLOC_SCRATCH_BYTES // (h * (d_h + 2) * 4) + 1
    with pytest.raises(L.BiError) as e:
        L.bi_decode_attn_noalloc(q, kp, kp, bt, kvl, off, too_many, C, 0.1, out)
    assert e.value.status == L.BI_ERR_WORKSPACE
    assert torch.count_nonzero(out) == 0
