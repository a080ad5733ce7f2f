"""Batch-invariant forward-pass kernels for MI355X (gfx950).

The product is libbi.so, a C-ABI library of hand-written HIP kernels whose
reductions run in one fixed order with split points fixed by the hidden
size or the request's own KV length (include/bi.h).  ``_lib`` is its thin
ctypes binding; ``model`` drives a Llama-shaped decoder through it and
``harness`` fuzzes schedules to check that every request's logits are bit
identical whatever it was batched with.

Importing the package loads nothing; the library is loaded on first use and
its absence is an error (there is no CPU fallback).
"""
from . import _lib  # noqa: F401

__all__ = ["_lib"]
