"""Query norm + query RoPE + window-key RoPE + window-key insert (oracle, test infrastructure).

Source: [P1] "GPU Compute Saturation" and [P2] "3.2 內核": the elementwise work on the query and on the
uncompressed sliding-window key in front of the main attention is one horizontally fused step (some waves
take query heads, others the key; no communication between them).

Readings (the pages name the steps, not their formulas), labelled R24:
* query norm is an RMSNorm of each head's D channels with one weight vector gamma_q [D] shared by the heads and
  eps an input (the compressor's RMSNorm rule, R6), then RoPE at the token's position on the last R dims
  (R7/R8), rounded once to the query's element type;
* the window key is the new token's raw K=V row: RoPE at its position, rounded to the window pages' element type
  (fp8: the per-row amax rule, R20), written at the row of its raw position (paging R18/R19). It is not
  normalised (the window holds raw rotated rows, R5).
"""
from __future__ import annotations

import numpy as np

from . import codecs, paging, rope as rope_mod
from .compress import Raw, rmsnorm


def prepare_qk(q: np.ndarray, q_dtype: str, kv: np.ndarray, tok_seq, tok_pos, gamma, eps: float,
               table: np.ndarray, rope_dims: int, swa: Raw):
    """q [n][H][D] and kv [n][D] as exact fp64 values of the inputs; returns q_out [n][H][D] in q_dtype storage
    (float32 / uint16 bf16 bits) and writes the rotated window rows into swa (pages, and scales for fp8)."""
    n, h, d = q.shape
    q_out = np.zeros((n, h, d), dtype=np.float32 if q_dtype == codecs.F32 else np.uint16)
    for t in range(n):
        cs = table[int(tok_pos[t])]
        for k in range(h):
            y = rope_mod.rope(rmsnorm(q[t, k], gamma, eps), cs, rope_dims)
            q_out[t, k] = codecs.store_row(y, q_dtype)[0]
        y = rope_mod.rope(np.asarray(kv[t], dtype=np.float64), cs, rope_dims)
        stored, sc = codecs.store_row(y, swa.dtype)
        row = paging.raw_slot(swa.block_table[int(tok_seq[t])], int(tok_pos[t]))
        swa.kv_pages[row] = stored
        if swa.scales is not None:
            swa.scales[row] = sc
    return q_out
