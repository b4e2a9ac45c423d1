"""Shared-K=V attention over selected compressed entries plus the raw sliding window (oracle, test infrastructure).

Sources:
* [P1] "DeepSeek V4 Attention Architecture": keys and values are one shared
  vector (2x memory saving); the output is inverse-rotated for translation
  invariance; a 128-token sliding window over uncompressed tokens gives local
  context before the compression boundary; DSA attends to the top-k entries.
* [P2] "二、注意力機制為什么這么麻煩": compress-then-sparse (CSA) and the
  heavier c128a variant with dense attention (HCA).
* [P3] "注意力计算剪枝": c128a layers leave few enough entries for full
  attention; recent tokens are reachable only through the window.

Readings: one joint softmax over selected entries and window rows, no
de-duplication and no sink (R14); softmax scale tau is an input (1/sqrt(D) in
the configurations, R15); V = K over all D dims, fp32 output, then optional
inverse RoPE at the query position (R16); the window is [max(0, p-W+1), p]
including the query's own row (R13); dense mode (no top-k list) uses every
eligible entry (R17).
"""
from __future__ import annotations

import numpy as np

from . import codecs, paging, rope as rope_mod
from .compress import Cache, Raw


def gather_keys(kv_cache: Cache, swa: Raw, swa_window: int, seq: int, q_pos: int, entries) -> np.ndarray:
    """Dequantised key rows: the given compressed entries, then the window rows in position order."""
    rows = []
    if len(entries):
        slots = [paging.entry_slot(kv_cache.block_table[seq], int(i), kv_cache.ratio) for i in entries]
        sc = kv_cache.scales[slots] if kv_cache.dtype == codecs.FP8 else None
        rows.append(codecs.load_rows(kv_cache.pages[slots], kv_cache.dtype, sc))
    lo = max(0, int(q_pos) - swa_window + 1)
    pos = list(range(lo, int(q_pos) + 1)) if swa_window > 0 else []
    if pos:
        rs = [paging.raw_slot(swa.block_table[seq], j) for j in pos]
        sc = swa.scales[rs] if swa.dtype == codecs.FP8 else None
        rows.append(codecs.load_rows(swa.kv_pages[rs], swa.dtype, sc))
    if not rows:
        return np.zeros((0, kv_cache.dim))
    return np.concatenate(rows, axis=0)


def attend_one(q: np.ndarray, keys: np.ndarray, scale: float):
    """o_h = sum_s softmax_s(scale * q_h . k_s) k_s for every head; returns (o [H][D], lse [H])."""
    q = np.asarray(q, dtype=np.float64)
    if keys.shape[0] == 0:
        return np.zeros_like(q), np.full(q.shape[0], -np.inf)
    lg = scale * (q @ keys.T)  # [H][n]
    mx = lg.max(axis=1, keepdims=True)
    ex = np.exp(lg - mx)
    den = ex.sum(axis=1, keepdims=True)
    o = (ex / den) @ keys
    lse = (mx + np.log(den))[:, 0]
    return o, lse


def selected_entries(topk_row, q_pos: int, kv_cache: Cache):
    if topk_row is None:
        return list(range(paging.num_eligible(int(q_pos), kv_cache.ratio, kv_cache.window)))
    return [int(i) for i in topk_row if i >= 0]


def attend(kv_cache: Cache, swa: Raw, swa_window: int, q_seq, q_pos, q, topk_idx, scale: float,
           fuse_inv_rope: bool, table):
    """All queries: (out [n_q][H][D] fp64, lse [n_q][H])."""
    n_q, h, d = q.shape
    out = np.zeros((n_q, h, d))
    lse = np.zeros((n_q, h))
    for qi in range(n_q):
        ent = selected_entries(None if topk_idx is None else topk_idx[qi], q_pos[qi], kv_cache)
        keys = gather_keys(kv_cache, swa, swa_window, int(q_seq[qi]), int(q_pos[qi]), ent)
        o, l = attend_one(q[qi], keys, scale)
        if fuse_inv_rope:
            o = rope_mod.inv_rope(o, table[int(q_pos[qi])], kv_cache.rope_dims)
        out[qi], lse[qi] = o, l
    return out, lse
