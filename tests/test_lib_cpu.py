"""Host-side checks of the C-ABI library that need no GPU: it loads, exports
every function include/bi.h declares, and its host helpers compute what the
header says."""
import ctypes
import os
import re

import pytest

from conftest import ROOT, golden

L = pytest.importorskip("invariant_bi_rmsnorm_amd._lib")


def declared_functions():
    names = []
    for f in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if f.endswith(".h"):
            src = open(os.path.join(ROOT, "include", f)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names += re.findall(r"^\s*[A-Za-z_][\w \*]*?\b(bi_\w+)\s*\(", src, re.M)
    return sorted(set(names))


def test_library_exports_every_declared_symbol():
    lib = L.load()
    decl = declared_functions()
    assert len(decl) >= 15
    missing = [n for n in decl if not hasattr(lib, n)]
    assert not missing, missing
    # the binding wraps exactly the declared functions
    assert sorted(L.SIGNATURES) == decl


def test_status_strings_and_version():
    lib = L.load()
    assert lib.bi_abi_version() == 3
    assert lib.bi_status_string(0) == b"ok"
    assert lib.bi_status_string(2) == b"unsupported configuration"
    assert lib.bi_status_string(99) == b"unknown status"


def test_chunk_offsets_printed_example():
    g = golden("split_count.txt")
    off = L.bi_chunk_offsets([int(g["seq_len"])], int(g["split_tile"]))
    assert off.tolist() == [0, int(g["num_splits"])]
    assert L.bi_chunk_offsets([1, 256, 257, 0], 256).tolist() == [0, 1, 2, 4, 4]
    assert L.bi_attn_partials_bytes(10, 32, 128) == 10 * 32 * 130 * 4


def test_invalid_arguments_rejected_before_launch():
    lib = L.load()
    # M < 0 is rejected on the host; nothing touches a GPU
    st = lib.bi_rmsnorm(None, None, None, -1, 16, ctypes.c_float(1e-5), 1, None)
    assert st == L.BI_ERR_INVALID
    assert b"bad shape" in lib.bi_last_error()
    st = lib.bi_gemm(None, None, None, 4, 4, 4, 1, 1, None)   # null pointers
    assert st == L.BI_ERR_INVALID
    st = lib.bi_gemm(None, None, None, 4, 4, 4, 0, 1, None)   # f32 in, bf16 out
    assert st == L.BI_ERR_UNSUPPORTED
    assert lib.bi_rmsnorm(None, None, None, 0, 16, ctypes.c_float(1e-5), 1, None) == L.BI_OK
    # the norm-prologue products: more than 4 rows or K past 4096 are not
    # covered (the caller runs the two calls); o without h_out is invalid
    eps = ctypes.c_float(1e-5)
    st = lib.bi_norm_gemm(None, None, None, eps, None, None, None, None, 5, 64, 4096, 1, None)
    assert st == L.BI_ERR_UNSUPPORTED and b"at most 4 rows" in lib.bi_last_error()
    st = lib.bi_norm_gemm_swiglu(None, None, None, eps, None, None, None, None, 1, 64, 4104,
                                 None)
    assert st == L.BI_ERR_UNSUPPORTED
    fake = ctypes.c_void_p(256)
    st = lib.bi_norm_gemm(fake, fake, fake, eps, None, None, fake, fake, 1, 64, 4096, 1, None)
    assert st == L.BI_ERR_INVALID and b"h_out" in lib.bi_last_error()
    st = lib.bi_norm_gemm_qkv_rope(None, None, None, eps, None, None, None, 1, 4096, 32, 8, 120,
                                   None, None, None, None, 16, None, None, None, None)
    assert st == L.BI_ERR_INVALID                      # d_h % 16 != 0


def test_binding_argument_counts_match_header():
    src = open(os.path.join(ROOT, "include", "bi.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    for m in re.finditer(r"\b(bi_\w+)\s*\(([^)]*)\)\s*;", src):
        name, params = m.group(1), m.group(2).strip()
        n = 0 if params in ("", "void") else params.count(",") + 1
        assert len(L.SIGNATURES[name][1]) == n, name


def test_binding_rejects_mismatched_buffers_before_launch():
    """The binding's host checks raise before any pointer is taken: CPU
    tensors reach them, so no GPU is needed.  Each case would otherwise let a
    kernel read or write past a buffer (a bf16 W read with fp32 A's element
    size; partials or offsets shorter than the chunk rows)."""
    import torch
    bf, f32, i32 = torch.bfloat16, torch.float32, torch.int32
    A = torch.zeros((4, 16), dtype=f32)
    with pytest.raises(ValueError, match="W is"):
        L.bi_gemm(A, torch.zeros((8, 16), dtype=bf), torch.zeros((4, 8), dtype=f32))
    with pytest.raises(ValueError, match="W is"):
        L.bi_gemm_free(A, torch.zeros((8, 16), dtype=bf), torch.zeros((4, 8), dtype=f32))
    with pytest.raises(ValueError, match="shape mismatch"):
        L.bi_gemm(A, torch.zeros((8, 12), dtype=f32), torch.zeros((4, 8), dtype=f32))

    B, h, h_kv, d_h, tot = 2, 4, 2, 64, 5
    q = torch.zeros((B, h, d_h), dtype=bf)
    kp = torch.zeros((8, h_kv, 16, d_h), dtype=bf)
    bt = torch.zeros((B, 4), dtype=i32)
    kvl = torch.ones(B, dtype=i32)
    off = torch.zeros(B + 1, dtype=i32)
    ml = torch.zeros((tot, h, 2), dtype=f32)
    acc = torch.zeros((tot, h, d_h), dtype=f32)
    with pytest.raises(ValueError, match="part_acc"):
        L.bi_decode_attn(q, kp, kp, bt, kvl, off, tot, 64, 0.1, ml, acc[:tot - 1])
    with pytest.raises(ValueError, match="part_ml"):
        L.bi_decode_attn(q, kp, kp, bt, kvl, off, tot, 64, 0.1, ml[:2], acc)
    with pytest.raises(ValueError, match="chunk_off"):
        L.bi_decode_attn(q, kp, kp, bt, kvl, off[:B], tot, 64, 0.1, ml, acc)
    with pytest.raises(ValueError, match="kv_len"):
        L.bi_decode_attn(q, kp, kp, bt, kvl[:1], off, tot, 64, 0.1, ml, acc)
    with pytest.raises(ValueError, match="pools"):
        L.bi_decode_attn(q, kp, kp.float(), bt, kvl, off, tot, 64, 0.1, ml, acc)
    with pytest.raises(ValueError, match="block_table"):
        L.bi_decode_attn(q, kp, kp, bt[:1], kvl, off, tot, 64, 0.1, ml, acc)
    with pytest.raises(ValueError, match="fp32"):
        L.bi_decode_attn(q, kp, kp, bt, kvl, off, tot, 64, 0.1, ml.to(bf), acc)
    out = torch.zeros((B, h, d_h), dtype=bf)
    with pytest.raises(ValueError, match="chunk_off"):
        L.bi_merge_partials(ml, acc, off[:B], out)
    with pytest.raises(ValueError, match="partials"):
        L.bi_merge_partials(ml, acc[:, :, :32], off, out)
    with pytest.raises(ValueError, match="o and h_out"):
        L.bi_norm_gemm(A.to(bf), A.to(bf), torch.zeros(16, dtype=bf), 1e-5, None, None,
                       torch.zeros((8, 16), dtype=bf), torch.zeros((4, 8), dtype=bf))
    with pytest.raises(ValueError, match="gamma"):
        L.bi_norm_gemm(A.to(bf), None, torch.zeros(12, dtype=bf), 1e-5, None, None,
                       torch.zeros((8, 16), dtype=bf), torch.zeros((4, 8), dtype=bf))
    with pytest.raises(ValueError, match="bf16"):
        L.bi_norm_gemm(A, None, torch.zeros(16, dtype=bf), 1e-5, None, None,
                       torch.zeros((8, 16), dtype=bf), torch.zeros((4, 8), dtype=bf))
    with pytest.raises(ValueError, match="q_start"):
        L.bi_prefill_attn(q, torch.zeros(1, dtype=i32), torch.zeros(2, dtype=i32), kp, kp,
                          bt, 64, 0.1, q.clone())


def test_k_page_layout_helpers():
    """k_pool_from_rows puts unit u of token t of a (page, head) block at byte
    (u * page_size + t) * 16 of the block (the layout bi.h states), and
    k_pool_to_rows undoes it; V needs no conversion."""
    import torch
    for dt, it, per in ((torch.bfloat16, torch.int16, 8), (torch.float32, torch.int32, 4)):
        P, H, S, D = 3, 2, 16, 64
        # every element a distinct bit pattern
        k = torch.arange(P * H * S * D, dtype=it).reshape(P, H, S, D).view(dt)
        dev = L.k_pool_from_rows(k)
        assert dev.shape == k.shape and dev.dtype == dt
        flat = dev.view(it).reshape(-1)
        kb = k.view(it)
        for p in range(P):
            for g in range(H):
                for t in range(S):
                    for e in range(D):
                        off = (p * H + g) * S * D + ((e // per) * S + t) * per + e % per
                        assert flat[off] == kb[p, g, t, e]
        assert torch.equal(L.k_pool_to_rows(dev).view(it), kb)


def test_packed_weight_sizes_and_checks():
    """bi_packed_weight_bytes counts whole 256-row x 64-k panels steps of
    32 KiB; bi_pack_weight refuses bad shapes before any launch."""
    lib = L.load()
    assert lib.bi_packed_weight_bytes(256, 64) == 32768
    assert lib.bi_packed_weight_bytes(300, 72) == 2 * 2 * 32768
    assert lib.bi_packed_weight_bytes(1, 8) == 32768
    assert lib.bi_packed_weight_bytes(128256, 4096) == 501 * 64 * 32768
    assert lib.bi_packed_weight_bytes(0, 64) == 0 and lib.bi_packed_weight_bytes(64, 0) == 0
    fake = ctypes.c_void_p(256)
    assert lib.bi_pack_weight(fake, fake, 0, 64, None) == L.BI_ERR_INVALID
    assert lib.bi_pack_weight(fake, fake, 16, 12, None) == L.BI_ERR_UNSUPPORTED
    assert lib.bi_pack_weight(None, fake, 16, 64, None) == L.BI_ERR_INVALID
    assert lib.bi_pack_weight(ctypes.c_void_p(258), fake, 16, 64, None) == L.BI_ERR_INVALID
    assert b"misaligned" in lib.bi_last_error()
    import torch
    with pytest.raises(ValueError, match="bf16"):
        L.pack_weight(torch.zeros((4, 8), dtype=torch.float32))
