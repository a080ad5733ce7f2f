"""Shared helpers for the GPU tests (inputs from synth, comparisons)."""
import math

import numpy as np
import torch

import synth

U = 2.0 ** -24


def dev():
    return torch.device("cuda:0")


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy()


def bits_equal(a, b) -> bool:
    a = np.ascontiguousarray(a, dtype=np.float32)
    b = np.ascontiguousarray(b, dtype=np.float32)
    return a.shape == b.shape and np.array_equal(a.view(np.uint32), b.view(np.uint32))


def gu_halves(gu) -> np.ndarray:
    """A gate/up product [rows, 2F] in the library's 8-column blocks (columns
    16p .. 16p + 7 gate, 16p + 8 .. 16p + 15 up) as [gate | up] columns, the
    oracle's silu_mul layout."""
    gu = np.asarray(gu, np.float32)
    n, f2 = gu.shape
    b = gu.reshape(n, f2 // 16, 2, 8)
    return np.concatenate([b[:, :, 0].reshape(n, f2 // 2), b[:, :, 1].reshape(n, f2 // 2)], 1)


def mismatch_report(a, b, n=5) -> str:
    a = np.asarray(a, np.float32).ravel()
    b = np.asarray(b, np.float32).ravel()
    bad = np.nonzero(a.view(np.uint32) != b.view(np.uint32))[0]
    return f"{bad.size} mismatches of {a.size}; first {[(int(i), float(a[i]), float(b[i])) for i in bad[:n]]}"


class PagedKV:
    """Paged K/V pools [pages][h_kv][page_size][d_h] (token-major rows, the
    oracle's layout) with random scattered placement of each request's
    pages, filled from synth normals; to() gives the device copies, K in the
    library's K page layout."""

    def __init__(self, kv_len, h_kv, d_h, page_size, seed, dtype, capacity=None, slack=1.25):
        cap = np.asarray(capacity if capacity is not None else kv_len)
        self.place = synth.scatter_pages(cap, page_size, seed=seed, slack=slack)
        shape = (self.place.num_pages, h_kv, page_size, d_h)
        self.k = synth.normal(shape, seed=seed + 1).to(dtype)
        self.v = synth.normal(shape, seed=seed + 2).to(dtype)
        self.bt = torch.from_numpy(self.place.block_table.copy())
        self.page_size = page_size

    def to(self, device):
        """K (in the library's K page layout), V and the block table on device."""
        from invariant_bi_rmsnorm_amd._lib import k_pool_from_rows
        return k_pool_from_rows(self.k).to(device), self.v.to(device), self.bt.to(device)


def gemm_bf16_tol(A: np.ndarray, W: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Bound on |gpu - oracle| for bf16 outputs of a K-long fp32 dot.  Each
    side's fp32 sum (G on the GPU, O in the oracle) is within (K+1) u
    sum|a w| of the exact value in any summation order, so |G - O| <= 2 (K+1)
    u sum|a w|; each side's rounding to bf16 moves at most half a bf16 ulp,
    i.e. 2^-8 of its own magnitude.  When G and O straddle a rounding
    boundary the two bf16 results sit one full bf16 ulp apart, so the bound
    is 2^-8 (|G| + |O|) + |G - O| <= 2^-7 |ref| + (1 + 2^-7) |G - O|."""
    K = A.shape[1]
    s = np.abs(A).astype(np.float64) @ np.abs(W).astype(np.float64).T
    dsum = 2.0 * (K + 1) * U * s
    return 2.0 ** -7 * np.abs(ref) + 1.01 * dsum + 1e-30


def gemm_f32_tol(A: np.ndarray, W: np.ndarray) -> np.ndarray:
    K = A.shape[1]
    s = np.abs(A).astype(np.float64) @ np.abs(W).astype(np.float64).T
    return 2.0 * (K + 1) * U * s + 1e-30


def scale_for(d_h: int) -> float:
    return float(np.float32(1.0 / math.sqrt(d_h)))
