"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This module only draws inputs -- activations, weights, KV histories, request
lengths, page placements, RoPE tables, token ids.  It holds none of the
method's arithmetic (no norm, product, softmax or merge).  Every draw uses
torch's CPU generator (or numpy's PCG64) with an explicit seed, so the same
seed gives the same tensor on every machine; callers move tensors to the GPU
themselves.

Workload recipes (distributions and sizes) follow the configurations the
build is measured on: N(0,1) activations and KV, N(0, 0.02) weights, KV
lengths uniform or log-uniform, 16-token pages scattered at random over a
pool about 1.25x the live pages.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np
import torch


def normal(shape, seed: int, std: float = 1.0, dtype=torch.float32) -> torch.Tensor:
    """N(0, std^2) draws from a seeded CPU generator, cast to ``dtype``."""
    g = torch.Generator().manual_seed(int(seed))
    t = torch.randn(tuple(shape), generator=g, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


def integers(shape, lo: int, hi: int, seed: int, dtype=torch.float32) -> torch.Tensor:
    """Uniform integers in [lo, hi] as ``dtype`` (exact in bf16 for |v| <= 256)."""
    g = torch.Generator().manual_seed(int(seed))
    return torch.randint(lo, hi + 1, tuple(shape), generator=g).to(dtype)


def uniform_lengths(n: int, lo: int, hi: int, seed: int) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.integers(lo, hi + 1, size=n).astype(np.int32)


def log_uniform_lengths(n: int, lo: int, hi: int, seed: int) -> np.ndarray:
    """s = round(exp(U(ln lo, ln hi)))."""
    rng = np.random.Generator(np.random.PCG64(seed))
    s = np.rint(np.exp(rng.uniform(math.log(lo), math.log(hi), size=n)))
    return np.clip(s, lo, hi).astype(np.int32)


def token_ids(n: int, vocab: int, seed: int) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.integers(0, vocab, size=n).astype(np.int32)


@dataclass
class PagePlacement:
    """Random placement of each request's pages in a shared pool."""
    block_table: np.ndarray  # [B, max_pages] int32, unused slots = -1
    num_pages: int           # pool size in pages
    max_pages: int


def scatter_pages(capacity_tokens, page_size: int, seed: int, slack: float = 1.25,
                  max_pages: int | None = None) -> PagePlacement:
    """Give request r ceil(capacity_tokens[r] / page_size) distinct pages drawn
    from a random permutation of a pool ``slack`` times the live page count."""
    cap = np.asarray(capacity_tokens, dtype=np.int64)
    need = (cap + page_size - 1) // page_size
    live = int(need.sum())
    pool = max(int(math.ceil(live * slack)), live, 1)
    rng = np.random.Generator(np.random.PCG64(seed))
    perm = rng.permutation(pool).astype(np.int32)
    mp = int(max_pages if max_pages is not None else max(int(need.max(initial=1)), 1))
    bt = np.full((len(cap), mp), -1, dtype=np.int32)
    pos = 0
    for r, k in enumerate(need):
        bt[r, :k] = perm[pos:pos + k]
        pos += k
    return PagePlacement(bt, pool, mp)


def rope_tables(max_pos: int, d_h: int, theta: float = 500000.0):
    """cos/sin [max_pos, d_h/2] in fp32, evaluated in fp64: angle(p, i) =
    p * theta^(-2i/d_h).  Model constants, handed to both sides as data."""
    half = d_h // 2
    inv = theta ** (-(np.arange(half, dtype=np.float64) * 2.0) / d_h)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * inv[None, :]
    return (torch.from_numpy(np.cos(ang).astype(np.float32)),
            torch.from_numpy(np.sin(ang).astype(np.float32)))


def seeds(base: int, n: int) -> list[int]:
    """n distinct derived seeds (recorded with every report)."""
    rng = np.random.Generator(np.random.PCG64(base))
    return [int(s) for s in rng.integers(1, 2**31 - 1, size=n)]
