"""Indexer score over eligible compressed entries and top-k selection (oracle, test infrastructure).

Sources:
* [P1] "DeepSeek V4 Attention Architecture" and [P2] "二、注意力機制為什么這么麻煩":
  DeepSeek Sparse Attention keeps only the top-k compressed entries
  (k = 512 on c4a layers, k = 8192 on c128a layers for V4-Flash).
* [P2] "3.2 內核": the indexer has its own compressed K cache and runs as its
  own pipeline (compress -> score -> top-k).
* Eligibility from [P3] "注意力计算剪枝" (no entry containing future tokens).

The score formula is not on the pages. Two forms are provided:
* DOT   s_e = q . k_e                          (one indexer head)
* WRELU s_e = sum_h w_h * max(0, q_h . k_e)    (H indexer heads, per-query head weights)
fp8 keys are dequantised as scale_e * k8_e (R11), fp4 keys block by block as 2^X_b * e2m1
(R25). No extra scale is applied.

Top-k order (R12): score descending, then entry index ascending; -0.0 equals
+0.0; NaN ranks below every number. min(k, n_elig) entries are kept and
emitted in ascending index order, padded with -1.
"""
from __future__ import annotations

import numpy as np

from . import codecs, paging
from .compress import Cache

DOT, WRELU = 0, 1


def eligible_keys(cache: Cache, seq: int, q_pos: int) -> np.ndarray:
    """Dequantised rows [n_elig][D] of the entries usable at q_pos, in entry order."""
    n = paging.num_eligible(int(q_pos), cache.ratio, cache.window)
    slots = [paging.entry_slot(cache.block_table[seq], i, cache.ratio) for i in range(n)]
    if n == 0:
        return np.zeros((0, cache.dim))
    sc = cache.scales[slots] if cache.dtype in (codecs.FP8, codecs.FP4) else None
    return codecs.load_rows(cache.pages[slots], cache.dtype, sc)


def scores(keys: np.ndarray, q: np.ndarray, head_w, mode: int) -> np.ndarray:
    """Scores of rows `keys` [n][D] for one query q [H][D] (fp64)."""
    q = np.asarray(q, dtype=np.float64)
    if mode == DOT:
        if q.shape[0] != 1:
            raise ValueError("DOT scoring takes exactly one indexer head")
        return keys @ q[0]
    if mode == WRELU:
        logits = keys @ q.T  # [n][H]
        return np.maximum(logits, 0.0) @ np.asarray(head_w, dtype=np.float64)
    raise ValueError(mode)


def topk(s: np.ndarray, k: int):
    """(indices ascending padded with -1 to k, their scores, count) under the R12 order."""
    s = np.asarray(s)
    n = s.shape[0]
    idx = np.arange(n)
    nan = np.isnan(s)
    val = np.where(nan, 0.0, s).astype(np.float64)
    order = np.lexsort((idx, -val, nan))  # last key is primary: non-NaN first, then score desc, then index asc
    chosen = np.sort(order[: min(k, n)])
    out = np.full(k, -1, dtype=np.int32)
    out[: chosen.size] = chosen
    sc = np.full(k, np.nan)
    sc[: chosen.size] = s[chosen]
    return out, sc, int(chosen.size)


def index_topk(cache: Cache, q_seq, q_pos, q_idx, head_w, mode: int, k: int):
    """Full index stage for every query: (out_idx [n_q][k], out_count [n_q], out_scores [n_q][k])."""
    n_q = len(q_pos)
    out_idx = np.full((n_q, k), -1, dtype=np.int32)
    out_cnt = np.zeros(n_q, dtype=np.int32)
    out_sc = np.full((n_q, k), np.nan)
    for qi in range(n_q):
        keys = eligible_keys(cache, int(q_seq[qi]), int(q_pos[qi]))
        w = None if head_w is None else head_w[qi]
        s = scores(keys, q_idx[qi], w, mode)
        out_idx[qi], out_sc[qi], out_cnt[qi] = topk(s, k)
    return out_idx, out_cnt, out_sc
