"""Synthetic stage inputs written straight into paged caches, so that one stage of the GPU path and the
oracle read identical arrays (no value ever passes from the GPU path to the oracle)."""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

import synth
from oracle import codecs, compress as oc, paging


@dataclass
class PagedCache:
    ratio: int
    window: int
    dim: int
    dtype: str
    bt: np.ndarray
    pages: np.ndarray
    scales: Optional[np.ndarray]

    def oracle(self, rope_dims: int = 0) -> oc.Cache:
        return oc.Cache(self.ratio, self.window, self.dim, rope_dims, self.dtype, self.pages, self.scales, self.bt)


def paged_cache(config: int, ratio: int, dim: int, dtype: str, positions, grid: bool = False, spare: int = 3):
    """Cache whose every page row holds a synthetic entry (N(0,1) rows or exact-grid rows)."""
    g = synth.rng(config, synth.STREAM_IDX_KV)
    window = 8 if ratio == 4 else 128
    B = len(positions)
    n_blocks = max(positions) // 256 + 1
    n_phys = B * n_blocks + spare
    bt = synth.random_block_table(synth.rng(config, synth.STREAM_BT), B, n_blocks, n_phys)
    rows = n_phys * (256 // ratio)
    scales = None
    if grid:
        vals = synth.grid_values(g, (rows, dim))
        if dtype == codecs.F32:
            pages = vals
        elif dtype == codecs.BF16:
            pages = (vals.view(np.uint32) >> np.uint32(16)).astype(np.uint16)  # grid values are exact in bf16
        else:
            pages = grid_e4m3(vals)
            scales = np.ones(rows, np.float32)
    else:
        if dtype == codecs.F32:
            pages = synth.normal_f32(g, (rows, dim))
        elif dtype == codecs.BF16:
            pages = synth.normal_bf16_bits(g, (rows, dim))
        else:
            pages, scales = synth.e4m3_rows(g, rows, dim)
    return PagedCache(ratio, window, dim, dtype, bt, pages, scales)


def grid_e4m3(vals: np.ndarray) -> np.ndarray:
    """Codes of the exact-grid values {-2, -1.5, ..., 2} (all exactly representable in e4m3fn)."""
    table = {0.0: 0x00, 0.5: 0x30, 1.0: 0x38, 1.5: 0x3C, 2.0: 0x40}
    out = np.zeros(vals.shape, np.uint8)
    for v, code in table.items():
        out[vals == v] = code
        if v:
            out[vals == -v] = code | 0x80
    return out


def window_rows(config: int, dim: int, dtype: str, n_phys: int):
    g = synth.rng(config, synth.STREAM_SWA)
    if dtype == codecs.FP8:
        return synth.e4m3_rows(g, n_phys * 256, dim)
    if dtype == codecs.BF16:
        return synth.normal_bf16_bits(g, (n_phys * 256, dim)), None
    return synth.normal_f32(g, (n_phys * 256, dim)), None


def topk_lists(config: int, positions, ratio: int, k: int) -> np.ndarray:
    """Random ascending distinct entry lists < n_elig of each query, -1 padded to k (sampling only)."""
    g = synth.rng(config, 30)
    out = np.full((len(positions), k), -1, np.int32)
    for qi, p in enumerate(positions):
        n = paging.num_eligible(int(p), ratio, 8 if ratio == 4 else 128)
        take = min(k, n)
        out[qi, :take] = np.sort(g.choice(n, size=take, replace=False))
    return out


def grid_bf16(vals: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of exact-grid values (every grid value is exact in bf16)."""
    return (np.ascontiguousarray(vals, np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def grid_weights(g: np.random.Generator, shape) -> np.ndarray:
    """Indexer head weights on the grid {0, 1/16, ..., 1}: with exact-grid keys and queries every partial
    score is a multiple of 2^-6 below 2^15, so fp32 sums of them are exact in any order."""
    return (np.rint(g.uniform(0, 16, shape)) / 16).astype(np.float32)
