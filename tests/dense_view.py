"""Test helpers: dense per-sequence views of a paged batch and scatter of dense
sequences into a paged pool.  Written with numpy fancy indexing, separately
from the oracle's C gather loops, so the two can check each other."""
from __future__ import annotations

import numpy as np

from synth import bf16_bits_to_f32


def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """Stored values -> float64 (exact); f16 through numpy's IEEE binary16."""
    if dtype == "f32":
        return a.astype(np.float64)
    if dtype == "f16":
        return np.ascontiguousarray(a, dtype=np.uint16).view(np.float16).astype(np.float64)
    return bf16_bits_to_f32(a).astype(np.float64)


def dense_sequence(pool: np.ndarray, block_table: np.ndarray, s: int, length: int, page_size: int) -> np.ndarray:
    """Rows 0..length-1 of sequence s in logical order: [L, heads, width]."""
    t = np.arange(length)
    return pool[block_table[s, t // page_size], t % page_size]


def scatter_into_pool(dense_seqs, page_size: int, perm: np.ndarray, extra_pages: int, fill):
    """Inverse of dense_sequence: lay dense sequences [L, H, W] into a pool
    whose physical pages are given by `perm` in logical order.  Returns
    (pool, block_table)."""
    pages = [-(-len(x) // page_size) for x in dense_seqs]
    total = sum(pages) + extra_pages
    H, W = dense_seqs[0].shape[1:]
    pool = np.full((total, page_size, H, W), fill, dtype=dense_seqs[0].dtype)
    bt = np.full((len(dense_seqs), max(1, max(pages))), -1, dtype=np.int32)
    off = 0
    for s, x in enumerate(dense_seqs):
        for j in range(pages[s]):
            phys = int(perm[off + j])
            bt[s, j] = phys
            rows = x[j * page_size:(j + 1) * page_size]
            pool[phys, :len(rows)] = rows
        off += pages[s]
    return pool, bt
