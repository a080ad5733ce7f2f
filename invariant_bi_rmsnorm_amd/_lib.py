"""Thin ctypes binding of libbi.so (include/bi.h).

Argument marshalling only: each function takes torch tensors, checks dtype,
device and contiguity, and passes raw device pointers, sizes and the current
HIP stream to the C function of the same name.  Every computation happens in
the library's HIP kernels.  There is no fallback: if libbi.so is missing or a
call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libbi.so")

BI_OK, BI_ERR_INVALID, BI_ERR_UNSUPPORTED, BI_ERR_WORKSPACE, BI_ERR_HIP = 0, 1, 2, 3, 4
BI_F32, BI_BF16 = 0, 1

_c_int, _c_long, _c_float, _c_size, _vp = (ctypes.c_int, ctypes.c_long, ctypes.c_float,
                                          ctypes.c_size_t, ctypes.c_void_p)
_i32p = ctypes.POINTER(ctypes.c_int32)

# name -> (restype, argtypes); mirrors include/bi.h
SIGNATURES = {
    "bi_abi_version": (_c_int, []),
    "bi_status_string": (ctypes.c_char_p, [_c_int]),
    "bi_last_error": (ctypes.c_char_p, []),
    "bi_chunk_offsets": (_c_int, [_i32p, _c_int, _c_int, _i32p]),
    "bi_attn_partials_bytes": (_c_size, [_c_int, _c_int, _c_int]),
    "bi_rmsnorm": (_c_int, [_vp, _vp, _vp, _c_int, _c_int, _c_float, _c_int, _vp]),
    "bi_add_rmsnorm": (_c_int, [_vp, _vp, _vp, _vp, _c_int, _c_int, _c_float, _c_int, _vp]),
    "bi_packed_weight_bytes": (_c_size, [_c_int, _c_int]),
    "bi_pack_weight": (_c_int, [_vp, _vp, _c_int, _c_int, _vp]),
    "bi_gemm": (_c_int, [_vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _vp]),
    "bi_gemm_swiglu": (_c_int, [_vp, _vp, _vp, _c_int, _c_int, _c_int, _vp]),
    "bi_gemm_qkv_rope": (_c_int, [_vp, _vp] + [_c_int] * 5 + [_vp] * 4 + [_c_int]
                         + [_vp] * 4),
    "bi_norm_gemm": (_c_int, [_vp, _vp, _vp, _c_float, _vp, _vp, _vp, _vp] + [_c_int] * 4
                     + [_vp]),
    "bi_norm_gemm_swiglu": (_c_int, [_vp, _vp, _vp, _c_float, _vp, _vp, _vp, _vp]
                            + [_c_int] * 3 + [_vp]),
    "bi_norm_gemm_qkv_rope": (_c_int, [_vp, _vp, _vp, _c_float, _vp, _vp, _vp] + [_c_int] * 5
                              + [_vp] * 4 + [_c_int] + [_vp] * 4),
    "bi_decode_attn": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp] + [_c_int] * 8
                       + [_c_float, _c_int, _vp, _vp, _vp]),
    "bi_decode_attn_noalloc": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp] + [_c_int] * 8
                               + [_c_float, _c_int, _vp, _c_int, _vp]),
    "bi_merge_partials": (_c_int, [_vp, _vp, _vp, _c_int, _c_int, _c_int, _vp, _c_int, _vp]),
    "bi_softmax_weights": (_c_int, [_vp, _vp, _vp, _c_int, _vp]),
    "bi_prefill_attn": (_c_int, [_vp, _vp, _vp, _c_int, _c_int, _vp, _vp, _vp] + [_c_int] * 6
                        + [_c_float, _c_int, _vp, _vp]),
    "bi_embed": (_c_int, [_vp, _vp, _vp, _c_int, _c_int, _c_int, _vp]),
    "bi_rope_kv_append": (_c_int, [_vp, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp, _vp,
                                   _c_int, _vp, _vp, _vp, _c_int, _vp]),
    "bi_add": (_c_int, [_vp, _vp, _vp, _c_long, _c_int, _vp]),
    "bi_silu_mul": (_c_int, [_vp, _vp, _c_int, _c_int, _c_int, _vp]),
    "bi_argmax": (_c_int, [_vp, _vp, _c_int, _c_int, _vp]),
    "bi_log_softmax": (_c_int, [_vp, _vp, _c_int, _c_int, _vp]),
    "bi_sample": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _vp]),
    # batch-adaptive twins
    "bi_rmsnorm_free_workspace_bytes": (_c_size, [_c_int, _c_int]),
    "bi_rmsnorm_free": (_c_int, [_vp, _vp, _vp, _c_int, _c_int, _c_float, _c_int, _vp, _c_size,
                                 _vp]),
    "bi_gemm_free_workspace_bytes": (_c_size, [_c_int, _c_int, _c_int]),
    "bi_gemm_free": (_c_int, [_vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _vp, _c_size,
                              _vp]),
    "bi_decode_attn_free_workspace_bytes": (_c_size, [_c_int, _c_int, _c_int, _c_int]),
    "bi_decode_attn_free": (_c_int, [_vp, _vp, _vp, _vp, _vp] + [_c_int] * 7
                            + [_c_float, _c_int, _vp, _c_size, _vp, _vp]),
    "bi_merge_partials_free": (_c_int, [_vp, _vp, _vp, _c_int, _c_int, _c_int, _vp, _c_int,
                                        _vp]),
    "bi_prefill_attn_free": (_c_int, [_vp, _vp, _vp, _c_int, _c_int, _vp, _vp, _vp]
                             + [_c_int] * 5 + [_c_float, _c_int, _vp, _vp]),
}

_lib = None


class BiError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: {status} ({msg})")
        self.status = status


def load() -> ctypes.CDLL:
    """Load libbi.so (built in-tree by invariant_bi_rmsnorm_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run invariant_bi_rmsnorm_amd/build.py "
                               "(or __graft_entry__.build()) first; there is no fallback")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _check(fn: str, status: int) -> None:
    if status != BI_OK:
        msg = load().bi_last_error().decode()
        raise BiError(fn, status, msg)


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BI_BF16
    if t.dtype == torch.float32:
        return BI_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t: torch.Tensor | None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _i32(t: torch.Tensor):
    if t.dtype != torch.int32:
        raise TypeError(f"expected int32, got {t.dtype}")
    return _ptr(t)


def _need(ok: bool, fn: str, msg: str) -> None:
    """Host-side argument check of the binding: raise before any pointer is
    taken or any kernel is launched."""
    if not ok:
        raise ValueError(f"{fn}: {msg}")


class PackedWeight:
    """A bf16 weight [N][K] in the library's packed layout (bi.h, "Packed
    weights"), made by pack_weight.  `shape` and `dtype` are the matrix's;
    `data` is the packed device buffer the bf16 products read."""

    def __init__(self, data: torch.Tensor, N: int, K: int):
        self.data, self.shape, self.dtype = data, torch.Size((N, K)), torch.bfloat16

    @property
    def device(self):
        return self.data.device

    def dim(self) -> int:
        return 2


def pack_weight(W, stream=None) -> PackedWeight:
    """The packed layout of a row-major bf16 weight [N][K] (bi_pack_weight)."""
    if isinstance(W, PackedWeight):
        return W
    _need(W.dim() == 2 and W.dtype == torch.bfloat16, "bi_pack_weight",
          f"expected a bf16 [N][K] matrix, got {W.dtype} {tuple(W.shape)}")
    N, K = W.shape
    buf = torch.empty(load().bi_packed_weight_bytes(N, K) // 2, dtype=torch.bfloat16,
                      device=W.device)
    _check("bi_pack_weight", load().bi_pack_weight(_ptr(W), _ptr(buf), N, K, _stream(stream)))
    return PackedWeight(buf, N, K)


def _wptr(W, stream):
    """The pointer the products take for W: a packed bf16 weight's buffer (a
    row-major bf16 matrix is packed first, on the call's stream -- a
    convenience of the binding; the engine packs its weights once), or a
    row-major fp32 matrix."""
    if isinstance(W, PackedWeight):
        return _ptr(W.data), W
    if W.dtype == torch.bfloat16:
        _need(stream is None, "bi_gemm", "with an explicit stream, pass a PackedWeight")
        P = pack_weight(W)
        return _ptr(P.data), P
    return _ptr(W), W


def _check_gemm_args(fn: str, A, W, C) -> tuple:
    M, K = A.shape
    N = W.shape[0]
    _need(W.dim() == 2 and W.shape[1] == K and tuple(C.shape) == (M, N), fn,
          f"shape mismatch A{tuple(A.shape)} W{tuple(W.shape)} C{tuple(C.shape)}")
    # the kernel reads W with A's element size: a mixed pair would read past W
    _need(W.dtype == A.dtype, fn, f"W is {W.dtype} but A is {A.dtype}")
    return M, N, K


def _check_attn_args(fn: str, q, k_pool, v_pool, block_table, B: int) -> None:
    _need(k_pool.dim() == 4 and tuple(v_pool.shape) == tuple(k_pool.shape), fn,
          f"pools must be [pages][h_kv][page][d_h] of one shape, got {tuple(k_pool.shape)} "
          f"and {tuple(v_pool.shape)}")
    _need(k_pool.dtype == q.dtype and v_pool.dtype == q.dtype, fn,
          f"q is {q.dtype} but the pools are {k_pool.dtype} / {v_pool.dtype}")
    _need(k_pool.shape[3] == q.shape[2], fn, f"d_h of q ({q.shape[2]}) and pools "
          f"({k_pool.shape[3]}) differ")
    _need(block_table.dim() == 2 and block_table.shape[0] >= B, fn,
          f"block_table {tuple(block_table.shape)} has fewer than {B} rows")


def _check_partials(fn: str, part_ml, part_acc, rows: int, h: int, d_h: int) -> None:
    _need(part_ml.dtype == torch.float32 and part_acc.dtype == torch.float32, fn,
          "partials must be fp32")
    _need(part_ml.numel() >= rows * h * 2, fn,
          f"part_ml holds {part_ml.numel()} floats, needs {rows} x {h} x 2")
    _need(part_acc.numel() >= rows * h * d_h, fn,
          f"part_acc holds {part_acc.numel()} floats, needs {rows} x {h} x {d_h}")


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def k_pool_from_rows(k: torch.Tensor) -> torch.Tensor:
    """A K cache given as token-major rows, [..., page_size, d_h] per (page,
    kv head) block, rearranged into the library's K page layout (bi.h, "KV
    cache layout": 16-byte units stored unit-major within each block).  Same
    shape, dtype and device; only the order of the bytes changes.  V keeps
    token-major rows and needs no conversion."""
    *lead, S, D = k.shape
    e = 16 // k.element_size()
    return k.reshape(*lead, S, D // e, e).transpose(-3, -2).contiguous().reshape(k.shape)


def k_pool_to_rows(k: torch.Tensor) -> torch.Tensor:
    """The inverse of k_pool_from_rows: token-major rows of a K cache."""
    *lead, S, D = k.shape
    e = 16 // k.element_size()
    return k.reshape(*lead, D // e, S, e).transpose(-3, -2).contiguous().reshape(k.shape)


# ---------------------------------------------------------------------------

def bi_abi_version() -> int:
    return load().bi_abi_version()


def bi_chunk_offsets(kv_len_host, kv_chunk: int) -> torch.Tensor:
    """Host helper: int32 [B+1] prefix sum of ceil(kv_len / kv_chunk)."""
    kv = torch.as_tensor(kv_len_host, dtype=torch.int32).contiguous().cpu()
    out = torch.zeros(kv.numel() + 1, dtype=torch.int32)
    n = load().bi_chunk_offsets(ctypes.cast(kv.data_ptr(), _i32p), kv.numel(), kv_chunk,
                                ctypes.cast(out.data_ptr(), _i32p))
    if n < 0:
        raise BiError("bi_chunk_offsets", BI_ERR_INVALID, "bad arguments")
    return out


def bi_attn_partials_bytes(total_chunks: int, h: int, d_h: int) -> int:
    return load().bi_attn_partials_bytes(total_chunks, h, d_h)


def bi_rmsnorm(x, gamma, y, eps: float, stream=None):
    M, d = (x.shape[0], x.shape[-1]) if x.dim() == 2 else (x.numel() // x.shape[-1], x.shape[-1])
    _check("bi_rmsnorm", load().bi_rmsnorm(_ptr(x), _ptr(gamma), _ptr(y), M, d, eps, _dt(x),
                                           _stream(stream)))
    return y


def bi_add_rmsnorm(h, o, gamma, y, eps: float, stream=None):
    """h += o (rounded to h's dtype), then y = RMSNorm(h) * gamma."""
    M, d = (h.shape[0], h.shape[-1]) if h.dim() == 2 else (h.numel() // h.shape[-1], h.shape[-1])
    if tuple(o.shape) != tuple(h.shape) or tuple(y.shape) != tuple(h.shape):
        raise ValueError(f"shape mismatch h{tuple(h.shape)} o{tuple(o.shape)} y{tuple(y.shape)}")
    _check("bi_add_rmsnorm", load().bi_add_rmsnorm(_ptr(h), _ptr(o), _ptr(gamma), _ptr(y), M, d,
                                                   eps, _dt(h), _stream(stream)))
    return y


def bi_gemm(A, W, C, stream=None):
    M, N, K = _check_gemm_args("bi_gemm", A, W, C)
    wp, _keep = _wptr(W, stream)
    _check("bi_gemm", load().bi_gemm(_ptr(A), wp, _ptr(C), M, N, K, _dt(A), _dt(C),
                                     _stream(stream)))
    return C


def bi_gemm_swiglu(A, W, act, stream=None):
    """act = silu(g) * u of A W^T, W the gate/up weight in 8-row blocks (bi.h)."""
    M, K = A.shape
    I = act.shape[1]
    if tuple(W.shape) != (2 * I, K) or act.shape[0] != M:
        raise ValueError(f"shape mismatch A{tuple(A.shape)} W{tuple(W.shape)} act{tuple(act.shape)}")
    wp, _keep = _wptr(W, stream)
    _check("bi_gemm_swiglu", load().bi_gemm_swiglu(_ptr(A), wp, _ptr(act), M, I, K,
                                                   _stream(stream)))
    return act


def bi_gemm_qkv_rope(A, W, h: int, h_kv: int, d_h: int, pos, cos_t, sin_t, slot_mapping,
                     q_out, k_pool, v_pool, stream=None):
    """bi_gemm of A and W (rows [q | k | v]) then bi_rope_kv_append, in one pass."""
    M, K = A.shape
    if tuple(W.shape) != ((h + 2 * h_kv) * d_h, K) or tuple(q_out.shape) != (M, h, d_h):
        raise ValueError(f"shape mismatch A{tuple(A.shape)} W{tuple(W.shape)} "
                         f"q_out{tuple(q_out.shape)}")
    if any(t.dtype != torch.bfloat16 for t in (A, W, q_out, k_pool, v_pool)):
        raise TypeError("bi_gemm_qkv_rope takes bf16 A, W, q_out and pools")
    page_size = k_pool.shape[2]
    wp, _keep = _wptr(W, stream)
    _check("bi_gemm_qkv_rope", load().bi_gemm_qkv_rope(
        _ptr(A), wp, M, K, h, h_kv, d_h, _i32(pos) if pos is not None else None,
        _ptr(cos_t), _ptr(sin_t), _i32(slot_mapping), page_size, _ptr(q_out), _ptr(k_pool),
        _ptr(v_pool), _stream(stream)))
    return q_out


def _check_norm_args(fn: str, h, o, gamma, h_out, x_out, W, K: int) -> int:
    """Host checks of the norm-prologue products; returns M."""
    _need(h.dim() == 2 and h.shape[1] == K, fn, f"h{tuple(h.shape)} is not [M][{K}]")
    _need(gamma.numel() == K, fn, f"gamma has {gamma.numel()} entries, not {K}")
    for name, t in (("o", o), ("h_out", h_out), ("x_out", x_out)):
        _need(t is None or tuple(t.shape) == tuple(h.shape), fn,
              f"{name}{tuple(t.shape) if t is not None else ()} is not h's shape {tuple(h.shape)}")
    _need((o is None) == (h_out is None), fn, "o and h_out must both be given or both be None")
    _need(all(t is None or t.dtype == torch.bfloat16 for t in (h, o, gamma, h_out, x_out, W)),
          fn, "h, o, gamma, h_out, x_out and W must be bf16")
    return h.shape[0]


def bi_norm_gemm(h, o, gamma, eps: float, h_out, x_out, W, C, stream=None):
    """h_out = round(h + o) (o may be None: no add), x = RMSNorm(.) * gamma
    (stored to x_out unless None), then C = x W^T: bi_add_rmsnorm (or
    bi_rmsnorm) followed by bi_gemm, in one launch (at most 4 rows)."""
    N, K = W.shape
    M = _check_norm_args("bi_norm_gemm", h, o, gamma, h_out, x_out, W, K)
    _need(tuple(C.shape) == (M, N), "bi_norm_gemm", f"C{tuple(C.shape)} is not [{M}][{N}]")
    wp, _keep = _wptr(W, stream)
    _check("bi_norm_gemm", load().bi_norm_gemm(
        _ptr(h), _ptr(o), _ptr(gamma), eps, _ptr(h_out), _ptr(x_out), wp, _ptr(C), M, N, K,
        _dt(C), _stream(stream)))
    return C


def bi_norm_gemm_swiglu(h, o, gamma, eps: float, h_out, x_out, W, act, stream=None):
    """The norm prologue of bi_norm_gemm, then bi_gemm_swiglu's product."""
    K = W.shape[1]
    I = act.shape[1]
    M = _check_norm_args("bi_norm_gemm_swiglu", h, o, gamma, h_out, x_out, W, K)
    _need(tuple(W.shape) == (2 * I, K) and act.shape[0] == M and act.dtype == torch.bfloat16,
          "bi_norm_gemm_swiglu", f"shape mismatch W{tuple(W.shape)} act{tuple(act.shape)}")
    wp, _keep = _wptr(W, stream)
    _check("bi_norm_gemm_swiglu", load().bi_norm_gemm_swiglu(
        _ptr(h), _ptr(o), _ptr(gamma), eps, _ptr(h_out), _ptr(x_out), wp, _ptr(act), M, I,
        K, _stream(stream)))
    return act


def bi_norm_gemm_qkv_rope(h, o, gamma, eps: float, h_out, x_out, W, h_q: int, h_kv: int,
                          d_h: int, pos, cos_t, sin_t, slot_mapping, q_out, k_pool, v_pool,
                          stream=None):
    """The norm prologue of bi_norm_gemm, then bi_gemm_qkv_rope's product."""
    K = W.shape[1]
    M = _check_norm_args("bi_norm_gemm_qkv_rope", h, o, gamma, h_out, x_out, W, K)
    _need(tuple(W.shape) == ((h_q + 2 * h_kv) * d_h, K) and tuple(q_out.shape) == (M, h_q, d_h),
          "bi_norm_gemm_qkv_rope", f"shape mismatch W{tuple(W.shape)} q_out{tuple(q_out.shape)}")
    _need(all(t.dtype == torch.bfloat16 for t in (q_out, k_pool, v_pool)),
          "bi_norm_gemm_qkv_rope", "q_out and the pools must be bf16")
    page_size = k_pool.shape[2]
    wp, _keep = _wptr(W, stream)
    _check("bi_norm_gemm_qkv_rope", load().bi_norm_gemm_qkv_rope(
        _ptr(h), _ptr(o), _ptr(gamma), eps, _ptr(h_out), _ptr(x_out), wp, M, K, h_q, h_kv,
        d_h, _i32(pos) if pos is not None else None, _ptr(cos_t), _ptr(sin_t),
        _i32(slot_mapping), page_size, _ptr(q_out), _ptr(k_pool), _ptr(v_pool),
        _stream(stream)))
    return q_out


def bi_decode_attn(q, k_pool, v_pool, block_table, kv_len, chunk_off, total_chunks: int,
                   kv_chunk: int, scale: float, part_ml, part_acc, stream=None):
    B, h, d_h = q.shape
    _check_attn_args("bi_decode_attn", q, k_pool, v_pool, block_table, B)
    _need(kv_len.numel() == B, "bi_decode_attn", f"kv_len has {kv_len.numel()} entries, not {B}")
    _need(chunk_off.numel() == B + 1, "bi_decode_attn",
          f"chunk_off has {chunk_off.numel()} entries, not B + 1 = {B + 1}")
    _check_partials("bi_decode_attn", part_ml, part_acc, total_chunks, h, d_h)
    _, h_kv, page_size, _ = k_pool.shape
    _check("bi_decode_attn", load().bi_decode_attn(
        _ptr(q), _ptr(k_pool), _ptr(v_pool), _i32(block_table), _i32(kv_len), _i32(chunk_off),
        B, total_chunks, h, h_kv, d_h, page_size, block_table.shape[1], kv_chunk, scale, _dt(q),
        _ptr(part_ml), _ptr(part_acc), _stream(stream)))


NOALLOC_SCRATCH_BYTES = 32 * 1024 * 1024      # BI_NOALLOC_SCRATCH_BYTES


def bi_decode_attn_noalloc(q, k_pool, v_pool, block_table, kv_len, chunk_off,
                           total_chunks: int, kv_chunk: int, scale: float, out, stream=None):
    """bi_decode_attn + bi_merge_partials into out, with the partials in the
    library's static device buffer (no allocation by the library or here)."""
    B, h, d_h = q.shape
    _check_attn_args("bi_decode_attn_noalloc", q, k_pool, v_pool, block_table, B)
    _need(kv_len.numel() == B, "bi_decode_attn_noalloc",
          f"kv_len has {kv_len.numel()} entries, not {B}")
    _need(chunk_off.numel() == B + 1, "bi_decode_attn_noalloc",
          f"chunk_off has {chunk_off.numel()} entries, not B + 1 = {B + 1}")
    _need(tuple(out.shape) == (B, h, d_h), "bi_decode_attn_noalloc",
          f"out {tuple(out.shape)} is not {(B, h, d_h)}")
    _, h_kv, page_size, _ = k_pool.shape
    _check("bi_decode_attn_noalloc", load().bi_decode_attn_noalloc(
        _ptr(q), _ptr(k_pool), _ptr(v_pool), _i32(block_table), _i32(kv_len), _i32(chunk_off),
        B, total_chunks, h, h_kv, d_h, page_size, block_table.shape[1], kv_chunk, scale, _dt(q),
        _ptr(out), _dt(out), _stream(stream)))
    return out


def bi_merge_partials(part_ml, part_acc, chunk_off, out, stream=None):
    B, h, d_h = out.shape
    _need(chunk_off.numel() == B + 1, "bi_merge_partials",
          f"chunk_off has {chunk_off.numel()} entries, not B + 1 = {B + 1}")
    _need(part_acc.dim() == 3 and tuple(part_acc.shape[1:]) == (h, d_h)
          and part_ml.dim() == 3 and tuple(part_ml.shape[1:]) == (h, 2)
          and part_ml.shape[0] == part_acc.shape[0], "bi_merge_partials",
          f"partials {tuple(part_ml.shape)} / {tuple(part_acc.shape)} do not match "
          f"[rows][{h}][2] / [rows][{h}][{d_h}]")
    _check_partials("bi_merge_partials", part_ml, part_acc, part_acc.shape[0], h, d_h)
    _check("bi_merge_partials", load().bi_merge_partials(
        _ptr(part_ml), _ptr(part_acc), _i32(chunk_off), B, h, d_h, _ptr(out), _dt(out),
        _stream(stream)))
    return out


def bi_prefill_attn(q, q_start, q_pos0, k_pool, v_pool, block_table, kv_chunk: int,
                    scale: float, out, stream=None):
    T, h, d_h = q.shape
    R = q_pos0.numel()
    _check_attn_args("bi_prefill_attn", q, k_pool, v_pool, block_table, R)
    _need(q_start.numel() == R + 1, "bi_prefill_attn",
          f"q_start has {q_start.numel()} entries, not R + 1 = {R + 1}")
    _need(tuple(out.shape) == (T, h, d_h), "bi_prefill_attn",
          f"out {tuple(out.shape)} is not {(T, h, d_h)}")
    _, h_kv, page_size, _ = k_pool.shape
    _check("bi_prefill_attn", load().bi_prefill_attn(
        _ptr(q), _i32(q_start), _i32(q_pos0), R, T, _ptr(k_pool), _ptr(v_pool),
        _i32(block_table), h, h_kv, d_h, page_size, block_table.shape[1], kv_chunk, scale,
        _dt(q), _ptr(out), _stream(stream)))
    return out


def bi_embed(table, ids, out, stream=None):
    M, d = out.shape
    _check("bi_embed", load().bi_embed(_ptr(table), _i32(ids), _ptr(out), M, d, _dt(table),
                                       _stream(stream)))
    return out


def bi_rope_kv_append(qkv, h: int, h_kv: int, d_h: int, pos, cos_t, sin_t, slot_mapping,
                      q_out, k_pool, v_pool, stream=None):
    M = qkv.shape[0]
    page_size = k_pool.shape[2]
    _check("bi_rope_kv_append", load().bi_rope_kv_append(
        _ptr(qkv), M, h, h_kv, d_h, _i32(pos) if pos is not None else None, _ptr(cos_t),
        _ptr(sin_t), _i32(slot_mapping), page_size, _ptr(q_out), _ptr(k_pool), _ptr(v_pool),
        _dt(qkv), _stream(stream)))


def bi_add(a, b, y, stream=None):
    _check("bi_add", load().bi_add(_ptr(a), _ptr(b), _ptr(y), a.numel(), _dt(a), _stream(stream)))
    return y


def bi_silu_mul(gu, y, stream=None):
    M, F = y.shape
    _check("bi_silu_mul", load().bi_silu_mul(_ptr(gu), _ptr(y), M, F, _dt(gu), _stream(stream)))
    return y


def bi_softmax_weights(x, p, p_bf16=None, stream=None):
    """p = the attention kernels' softmax weight exp(x) for x <= 0 (fp32),
    p_bf16 = its bf16 bits (int16 tensor, optional)."""
    n = x.numel()
    if x.dtype != torch.float32 or p.dtype != torch.float32 or p.numel() != n:
        raise ValueError("bi_softmax_weights: need fp32 x and p of one size")
    if p_bf16 is not None and (p_bf16.dtype != torch.int16 or p_bf16.numel() != n):
        raise ValueError("bi_softmax_weights: p_bf16 must be int16 with x's size")
    _check("bi_softmax_weights", load().bi_softmax_weights(
        _ptr(x), _ptr(p), _ptr(p_bf16) if p_bf16 is not None else None, n, _stream(stream)))
    return p


def bi_log_softmax(x, y, stream=None):
    """y = log_softmax(x) row by row (fp32 [M, V]); y may be x."""
    M, V = x.shape
    if tuple(y.shape) != (M, V) or x.dtype != torch.float32 or y.dtype != torch.float32:
        raise ValueError(f"bi_log_softmax: need fp32 x, y of one shape, got {tuple(x.shape)} "
                         f"{x.dtype} and {tuple(y.shape)} {y.dtype}")
    _check("bi_log_softmax", load().bi_log_softmax(_ptr(x), _ptr(y), M, V, _stream(stream)))
    return y


def bi_sample(x, seed, pos, temperature, out, stream=None):
    """Seeded Gumbel-max token per row.  seed: int32 tensor holding the uint32
    seed bits; pos: int32; temperature: fp32 (<= 0: argmax); out: int32."""
    M, V = x.shape
    for t, dt, name in ((seed, torch.int32, "seed"), (pos, torch.int32, "pos"),
                        (temperature, torch.float32, "temperature"), (out, torch.int32, "out")):
        if t.dtype != dt or t.numel() != M:
            raise ValueError(f"bi_sample: {name} must be {dt} with {M} entries")
    if x.dtype != torch.float32:
        raise ValueError("bi_sample: logits must be fp32")
    _check("bi_sample", load().bi_sample(_ptr(x), _ptr(seed), _ptr(pos), _ptr(temperature),
                                         _ptr(out), M, V, _stream(stream)))
    return out


def bi_argmax(x, idx, stream=None):
    M, V = x.shape
    _check("bi_argmax", load().bi_argmax(_ptr(x), _i32(idx), M, V, _stream(stream)))
    return idx


# ---------------------------------------------------------------------------
# batch-adaptive twins (same mathematics, split points chosen from the batch)
# ---------------------------------------------------------------------------

class Workspace:
    """A grow-only device byte buffer for the twins' workspace arguments."""

    def __init__(self, device=None):
        self.device = device or torch.device("cuda")
        self.buf = torch.empty(0, dtype=torch.uint8, device=self.device)

    def get(self, nbytes: int) -> torch.Tensor:
        if self.buf.numel() < nbytes:
            self.buf = torch.empty(max(nbytes, 2 * self.buf.numel()), dtype=torch.uint8,
                                   device=self.device)
        return self.buf


_ws = {}


def _workspace(nbytes: int, device) -> tuple:
    w = _ws.get(str(device))
    if w is None:
        w = _ws[str(device)] = Workspace(device)
    b = w.get(max(nbytes, 1))
    return ctypes.c_void_p(b.data_ptr()), b.numel()


def bi_rmsnorm_free(x, gamma, y, eps: float, stream=None):
    M, d = x.numel() // x.shape[-1], x.shape[-1]
    ws, n = _workspace(load().bi_rmsnorm_free_workspace_bytes(M, d), x.device)
    _check("bi_rmsnorm_free", load().bi_rmsnorm_free(_ptr(x), _ptr(gamma), _ptr(y), M, d, eps,
                                                     _dt(x), ws, n, _stream(stream)))
    return y


def bi_gemm_free(A, W, C, stream=None):
    M, N, K = _check_gemm_args("bi_gemm_free", A, W, C)
    ws, n = _workspace(load().bi_gemm_free_workspace_bytes(M, N, K), A.device)
    wp, _keep = _wptr(W, stream)
    _check("bi_gemm_free", load().bi_gemm_free(_ptr(A), wp, _ptr(C), M, N, K, _dt(A),
                                               _dt(C), ws, n, _stream(stream)))
    return C


def bi_decode_attn_free(q, k_pool, v_pool, block_table, kv_len, max_kv_len: int, scale: float,
                        out, stream=None):
    """Decode attention with the occupancy-driven split policy; writes the
    merged output directly.  max_kv_len: the host's bound on kv_len."""
    B, h, d_h = q.shape
    _check_attn_args("bi_decode_attn_free", q, k_pool, v_pool, block_table, B)
    _need(kv_len.numel() == B, "bi_decode_attn_free",
          f"kv_len has {kv_len.numel()} entries, not {B}")
    _need(tuple(out.shape) == (B, h, d_h), "bi_decode_attn_free",
          f"out {tuple(out.shape)} is not {(B, h, d_h)}")
    _, h_kv, page_size, _ = k_pool.shape
    ws, n = _workspace(load().bi_decode_attn_free_workspace_bytes(B, h, d_h, max_kv_len),
                       q.device)
    _check("bi_decode_attn_free", load().bi_decode_attn_free(
        _ptr(q), _ptr(k_pool), _ptr(v_pool), _i32(block_table), _i32(kv_len), B, max_kv_len, h,
        h_kv, d_h, page_size, block_table.shape[1], scale, _dt(q), ws, n, _ptr(out),
        _stream(stream)))
    return out


def bi_merge_partials_free(part_ml, part_acc, chunk_off, out, stream=None):
    B, h, d_h = out.shape
    _need(chunk_off.numel() == B + 1, "bi_merge_partials_free",
          f"chunk_off has {chunk_off.numel()} entries, not B + 1 = {B + 1}")
    _check_partials("bi_merge_partials_free", part_ml, part_acc, part_acc.shape[0], h, d_h)
    _check("bi_merge_partials_free", load().bi_merge_partials_free(
        _ptr(part_ml), _ptr(part_acc), _i32(chunk_off), B, h, d_h, _ptr(out), _dt(out),
        _stream(stream)))
    return out


def bi_prefill_attn_free(q, q_start, q_pos0, k_pool, v_pool, block_table, scale: float, out,
                         stream=None):
    T, h, d_h = q.shape
    R = q_pos0.numel()
    _check_attn_args("bi_prefill_attn_free", q, k_pool, v_pool, block_table, R)
    _need(q_start.numel() == R + 1, "bi_prefill_attn_free",
          f"q_start has {q_start.numel()} entries, not R + 1 = {R + 1}")
    _, h_kv, page_size, _ = k_pool.shape
    _check("bi_prefill_attn_free", load().bi_prefill_attn_free(
        _ptr(q), _i32(q_start), _i32(q_pos0), R, T, _ptr(k_pool), _ptr(v_pool),
        _i32(block_table), h, h_kv, d_h, page_size, block_table.shape[1], scale, _dt(q),
        _ptr(out), _stream(stream)))
    return out
