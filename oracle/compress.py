"""KV compressor: window softmax-weighted sum -> RMSNorm -> RoPE at anchor -> store (oracle, test infrastructure).

Sources:
* [P1] "DeepSeek V4 Attention Architecture": a c4a compressed token is a
  weighted sum of 8 raw tokens at stride 4, a c128a one of 128 raw tokens at
  stride 128. [P3] "KV 缓存压缩": entry i covers 4i .. 4i+7, anchor 4i.
* [P2] "3.2 內核": after compression K goes through RMSNorm, then RoPE, then is
  written into the cache (main or indexer instance), all in one fused step.
* [P2] "3.1 顯存": each compressor keeps a per-request rolling residual
  (8 tokens with overlap for c4a, 128 for c128a) registered as sliding-window
  KV, i.e. raw pages on the same 256-position paging.

Readings (the pages do not give the weight parametrisation):
* R4: the weights are a per-channel softmax over the window of per-token role
  logits: a raw token at window offset t contributes its role r = t // ratio
  logit vector, so G has shape [tokens][coff][D] with coff = window // ratio.
* R6: RMSNorm over all D channels, eps an input (1e-6 by default), gamma an input.
* R8: RoPE with the cos/sin table row of the anchor.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import codecs, paging, rope as rope_mod


@dataclass
class Cache:
    """Host copy of one compressed cache (main or indexer instance)."""
    ratio: int
    window: int
    dim: int
    rope_dims: int
    dtype: str               # "f32" | "bf16" | "fp8" | "fp4"
    pages: np.ndarray        # [n_phys * 256/ratio][dim] (float32 | uint16 | uint8); fp4: [..][dim/2] packed uint8
    scales: np.ndarray       # [n_phys * 256/ratio] float32 (fp8), [..][dim/32] uint8 E8M0 (fp4), else None
    block_table: np.ndarray  # [batch][bt_stride] int32


@dataclass
class Raw:
    """Host copy of raw per-position pages: compressor state (roles = coff) or sliding-window K=V (roles = 0)."""
    dtype: str
    dim: int
    roles: int
    kv_pages: np.ndarray     # [n_phys * 256][dim]
    logit_pages: np.ndarray  # [n_phys * 256][roles][dim] or None
    scales: np.ndarray       # [n_phys * 256] float32 (fp8 sliding window only) or None
    block_table: np.ndarray  # [batch][bt_stride] int32


def window_weighted_sum(x: np.ndarray, logits: np.ndarray) -> np.ndarray:
    """z[c] = sum_t softmax_t(logits[t, c]) * x[t, c]; x, logits: [w][D]."""
    x = np.asarray(x, dtype=np.float64)
    lg = np.asarray(logits, dtype=np.float64)
    ex = np.exp(lg - lg.max(axis=0, keepdims=True))
    a = ex / ex.sum(axis=0, keepdims=True)
    return (a * x).sum(axis=0)


def rmsnorm(z: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    z = np.asarray(z, dtype=np.float64)
    return z / np.sqrt(np.mean(z * z) + eps) * np.asarray(gamma, dtype=np.float64)


def compress_entry(x, logits, gamma, eps, cs_row, rope_dims) -> np.ndarray:
    """One compressed entry in fp64 from its window rows (before storage rounding)."""
    z = window_weighted_sum(x, logits)
    y = rmsnorm(z, gamma, eps)
    return rope_mod.rope(y, cs_row, rope_dims)


def window_rows(state: Raw, bt_row, i: int, ratio: int, window: int):
    """Raw kv rows and role logits of entry i's window, read from state pages, in fp64."""
    first, last, _ = paging.entry_window(i, ratio, window)
    xs, ls = [], []
    for j in range(first, last + 1):
        row = paging.raw_slot(bt_row, j)
        xs.append(codecs.load_rows(state.kv_pages[row], state.dtype))
        role = (j - first) // ratio
        ls.append(codecs.load_rows(state.logit_pages[row, role], state.dtype))
    return np.stack(xs), np.stack(ls)


def compress_insert(cache: Cache, state: Raw, start_pos, cu_new, kv_new, logit_new,
                    gamma, eps: float, table: np.ndarray, max_entries_out: int):
    """Append new raw tokens to the state pages, then build and store every entry they complete.

    kv_new [total_new][D] and logit_new [total_new][coff][D] hold the new tokens
    of all sequences back to back (sequence b owns rows cu_new[b] .. cu_new[b+1]-1,
    raw positions start_pos[b] ...). Both arrays are in the state's element type.
    Returns (slots [B][max_entries_out] int32, -1 padded; counts [B] int32) and
    updates cache / state in place.
    """
    paging.check_shape(cache.ratio, cache.window)
    batch = len(start_pos)
    slots = np.full((batch, max_entries_out), -1, dtype=np.int32)
    counts = np.zeros(batch, dtype=np.int32)
    for b in range(batch):
        s0, n = int(start_pos[b]), int(cu_new[b + 1] - cu_new[b])
        for t in range(n):
            row = paging.raw_slot(state.block_table[b], s0 + t)
            state.kv_pages[row] = kv_new[cu_new[b] + t]
            state.logit_pages[row] = logit_new[cu_new[b] + t]
        for c, i in enumerate(paging.new_entries(s0, n, cache.ratio, cache.window)):
            x, lg = window_rows(state, state.block_table[b], i, cache.ratio, cache.window)
            anchor = cache.ratio * i
            y = compress_entry(x, lg, gamma, eps, table[anchor], cache.rope_dims)
            stored, sc = codecs.store_row(y, cache.dtype)
            slot = paging.entry_slot(cache.block_table[b], i, cache.ratio)
            cache.pages[slot] = stored
            if cache.scales is not None:
                cache.scales[slot] = sc
            if c < max_entries_out:
                slots[b, c] = slot
            counts[b] += 1
    return slots, counts
