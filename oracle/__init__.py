"""CPU oracle for the batch-invariant forward-pass reductions.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this package; the product path never
does.  It wraps ``liboracle.so`` (plain C, see ``oracle.c`` for the fixed
reduction orders and the passages they follow) with numpy marshalling.

Every array argument is converted to a C-contiguous float32 (values of bf16
tensors are exactly representable) or int32 numpy array; ``round_bf16``
selects whether results are rounded to bfloat16 (returned widened to
float32).
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None
_F = ctypes.POINTER(ctypes.c_float)
_I = ctypes.POINTER(ctypes.c_int32)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_build.LIB) or (
            os.path.getmtime(_build.LIB) < os.path.getmtime(_build.SRC)):
        _build.build()
    lib = ctypes.CDLL(_build.LIB)
    sig = {
        "oracle_bf16_rne": (ctypes.c_float, [ctypes.c_float]),
        "oracle_exp": (ctypes.c_float, [ctypes.c_float]),
        "oracle_exp_vec": (None, [_F, _F, ctypes.c_long]),
        "oracle_sum_serial": (ctypes.c_float, [_F, ctypes.c_int]),
        "oracle_sum_pairwise": (ctypes.c_float, [_F, ctypes.c_int]),
        "oracle_num_threads": (ctypes.c_int, []),
        "oracle_num_chunks": (ctypes.c_int, [ctypes.c_int, ctypes.c_int]),
        "oracle_rmsnorm": (None, [_F, _F, _F, ctypes.c_int, ctypes.c_int, ctypes.c_float,
                                  ctypes.c_int]),
        "oracle_gemm": (None, [_F, _F, _F, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                               ctypes.c_int]),
        "oracle_decode_partials": (None, [_F, _F, _F, _I, _I, _I] + [ctypes.c_int] * 7
                                   + [ctypes.c_float, _F, _F, ctypes.c_int]),
        "oracle_merge_partials": (None, [_F, _F, _I, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         _F, ctypes.c_int]),
        "oracle_prefill_attn": (None, [_F, _I, _I, ctypes.c_int, _F, _F, _I] + [ctypes.c_int] * 6
                                + [ctypes.c_float, _F, ctypes.c_int, ctypes.c_int]),
        "oracle_rope": (None, [_F, _I, _F, _F, _F, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                               ctypes.c_int]),
        "oracle_add": (None, [_F, _F, _F, ctypes.c_long, ctypes.c_int]),
        "oracle_silu_mul": (None, [_F, _F, ctypes.c_int, ctypes.c_int, ctypes.c_int]),
        "oracle_argmax": (None, [_F, _I, ctypes.c_int, ctypes.c_int]),
        "oracle_log": (ctypes.c_float, [ctypes.c_float]),
        "oracle_log_vec": (None, [_F, _F, ctypes.c_long]),
        "oracle_log_softmax": (None, [_F, _F, ctypes.c_int, ctypes.c_int]),
        "oracle_murmur3_2w": (ctypes.c_uint32, [ctypes.c_uint32, ctypes.c_uint32,
                                                ctypes.c_uint32]),
        "oracle_log64_vec": (None, [ctypes.POINTER(ctypes.c_double),
                                    ctypes.POINTER(ctypes.c_double), ctypes.c_long]),
        "oracle_sample": (None, [_F, ctypes.POINTER(ctypes.c_uint32), _I, _F, _I,
                                 ctypes.c_int, ctypes.c_int]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _f32(a):
    if hasattr(a, "detach"):  # torch tensor
        a = a.detach().cpu().float().numpy()
    return np.ascontiguousarray(a, dtype=np.float32)


def _i32(a):
    if hasattr(a, "detach"):
        a = a.detach().cpu().numpy()
    return np.ascontiguousarray(a, dtype=np.int32)


def _pf(a):
    return a.ctypes.data_as(_F)


def _pi(a):
    return a.ctypes.data_as(_I)


def num_threads() -> int:
    return _load().oracle_num_threads()


def bf16_rne(x: float) -> float:
    return _load().oracle_bf16_rne(x)


def exp(x: float) -> float:
    return _load().oracle_exp(x)


def exp_array(x) -> np.ndarray:
    x = _f32(x)
    y = np.empty_like(x)
    _load().oracle_exp_vec(_pf(x), _pf(y), x.size)
    return y


def sum_serial(x) -> float:
    x = _f32(x)
    return _load().oracle_sum_serial(_pf(x), x.size)


def sum_pairwise(x) -> float:
    x = _f32(x)
    return _load().oracle_sum_pairwise(_pf(x), x.size)


def num_chunks(kv_len: int, chunk: int) -> int:
    return _load().oracle_num_chunks(kv_len, chunk)


def rmsnorm(x, gamma, eps: float, round_bf16: bool) -> np.ndarray:
    x = _f32(x)
    g = _f32(gamma)
    M, d = x.reshape(-1, x.shape[-1]).shape
    y = np.empty_like(x)
    _load().oracle_rmsnorm(_pf(x), _pf(g), _pf(y), M, d, eps, int(round_bf16))
    return y


def gemm(A, W, round_bf16: bool) -> np.ndarray:
    A = _f32(A)
    W = _f32(W)
    M, K = A.shape
    N = W.shape[0]
    assert W.shape[1] == K
    C = np.empty((M, N), dtype=np.float32)
    _load().oracle_gemm(_pf(A), _pf(W), _pf(C), M, N, K, int(round_bf16))
    return C


def chunk_offsets(kv_len, chunk: int) -> np.ndarray:
    kv = _i32(kv_len)
    off = np.zeros(kv.size + 1, dtype=np.int32)
    for r, s in enumerate(kv):
        off[r + 1] = off[r] + num_chunks(int(s), chunk)
    return off


def decode_partials(q, k_pool, v_pool, block_table, kv_len, chunk_off, h_kv: int,
                    page_size: int, chunk: int, scale: float, p_bf16: bool = False):
    q = _f32(q)
    B, h, d_h = q.shape
    kp, vp = _f32(k_pool), _f32(v_pool)
    bt = _i32(block_table)
    kv = _i32(kv_len)
    off = _i32(chunk_off)
    rows = int(off[B])
    ml = np.zeros((rows, h, 2), dtype=np.float32)
    acc = np.zeros((rows, h, d_h), dtype=np.float32)
    _load().oracle_decode_partials(_pf(q), _pf(kp), _pf(vp), _pi(bt), _pi(kv), _pi(off), B, h,
                                   h_kv, d_h, page_size, bt.shape[1], chunk, scale, _pf(ml),
                                   _pf(acc), int(p_bf16))
    return ml, acc


def merge_partials(part_ml, part_acc, chunk_off, round_bf16: bool) -> np.ndarray:
    ml, acc, off = _f32(part_ml), _f32(part_acc), _i32(chunk_off)
    _, h, d_h = acc.shape
    B = off.size - 1
    out = np.empty((B, h, d_h), dtype=np.float32)
    _load().oracle_merge_partials(_pf(ml), _pf(acc), _pi(off), B, h, d_h, _pf(out),
                                  int(round_bf16))
    return out


def decode_attn(q, k_pool, v_pool, block_table, kv_len, h_kv, page_size, chunk, scale,
                round_bf16: bool, p_bf16: bool = False):
    """Decode attention = partials + serial merge.  p_bf16: softmax weights
    rounded to bf16 before the sums (bf16 KV on matrix cores)."""
    off = chunk_offsets(kv_len, chunk)
    ml, acc = decode_partials(q, k_pool, v_pool, block_table, kv_len, off, h_kv, page_size,
                              chunk, scale, p_bf16)
    return merge_partials(ml, acc, off, round_bf16)


def prefill_attn(q, q_start, q_pos0, k_pool, v_pool, block_table, h_kv: int, page_size: int,
                 chunk: int, scale: float, round_bf16: bool, p_bf16: bool = False) -> np.ndarray:
    q = _f32(q)
    T, h, d_h = q.shape
    qs, qp, bt = _i32(q_start), _i32(q_pos0), _i32(block_table)
    kp, vp = _f32(k_pool), _f32(v_pool)
    R = qp.size
    out = np.empty_like(q)
    _load().oracle_prefill_attn(_pf(q), _pi(qs), _pi(qp), R, _pf(kp), _pf(vp), _pi(bt), h, h_kv,
                                d_h, page_size, bt.shape[1], chunk, scale, _pf(out),
                                int(round_bf16), int(p_bf16))
    return out


def rope(x, pos, cos_t, sin_t, round_bf16: bool) -> np.ndarray:
    x = _f32(x)
    M, nh, d_h = x.shape
    p, c, s = _i32(pos), _f32(cos_t), _f32(sin_t)
    y = np.empty_like(x)
    _load().oracle_rope(_pf(x), _pi(p), _pf(c), _pf(s), _pf(y), M, nh, d_h, int(round_bf16))
    return y


def add(a, b, round_bf16: bool) -> np.ndarray:
    a, b = _f32(a), _f32(b)
    y = np.empty_like(a)
    _load().oracle_add(_pf(a), _pf(b), _pf(y), a.size, int(round_bf16))
    return y


def silu_mul(gu, round_bf16: bool) -> np.ndarray:
    gu = _f32(gu)
    M, F2 = gu.shape
    y = np.empty((M, F2 // 2), dtype=np.float32)
    _load().oracle_silu_mul(_pf(gu), _pf(y), M, F2 // 2, int(round_bf16))
    return y


def argmax(x) -> np.ndarray:
    x = _f32(x)
    M, V = x.shape
    idx = np.empty(M, dtype=np.int32)
    _load().oracle_argmax(_pf(x), _pi(idx), M, V)
    return idx


def log(x) -> np.ndarray:
    """The fixed binary32 log (oracle.c: oracle_log), elementwise."""
    x = _f32(np.atleast_1d(x))
    y = np.empty_like(x)
    _load().oracle_log_vec(_pf(x), _pf(y), x.size)
    return y


def log_softmax(x) -> np.ndarray:
    """Row-wise log-softmax of fp32 rows in the fixed order of oracle.c."""
    x = _f32(x)
    M, V = x.shape
    y = np.empty_like(x)
    _load().oracle_log_softmax(_pf(x), _pf(y), M, V)
    return y


def murmur3(seed: int, w0: int, w1: int) -> int:
    """MurmurHash3_x86_32 of the key (w0, w1) as two little-endian uint32."""
    return int(_load().oracle_murmur3_2w(seed & 0xffffffff, w0 & 0xffffffff, w1 & 0xffffffff))


def log64(x) -> np.ndarray:
    """The sampler's fixed binary64 log, elementwise."""
    x = np.ascontiguousarray(np.atleast_1d(x), dtype=np.float64)
    y = np.empty_like(x)
    P = ctypes.POINTER(ctypes.c_double)
    _load().oracle_log64_vec(x.ctypes.data_as(P), y.ctypes.data_as(P), x.size)
    return y


def sample(x, seed, pos, temperature) -> np.ndarray:
    """Seeded Gumbel-max token per row (oracle.c: oracle_sample)."""
    x = _f32(x)
    M, V = x.shape
    sd = np.ascontiguousarray(seed, dtype=np.uint32)
    ps = _i32(pos)
    tp = _f32(temperature)
    out = np.empty(M, dtype=np.int32)
    _load().oracle_sample(_pf(x), sd.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32)), _pi(ps),
                          _pf(tp), _pi(out), M, V)
    return out
