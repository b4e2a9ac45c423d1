"""Inverse RoPE followed by fp8 quantisation of the attention output (oracle, test infrastructure).

Source: [P1] "GPU Compute Saturation" (kernel fusions) and [P2] "3.2 內核": after the main attention, the
output goes through the inverse RoPE and then into the fp8 batched matmul of the o_lora projection; the
two steps are fused so the output makes one trip through HBM instead of two.

The pages do not say how the output is quantised for that matmul. Reading R23: each
(query, head) output row of D channels is cut into consecutive groups of G channels; every group is stored
as OCP e4m3fn codes with one fp32 scale, by the same per-row rule as the fp8 caches (reading R20):
y32 = fl32(y), amax = max|y32|, code = e4m3(fl32(y32 * fl32(448 / amax))), scale = fl32(amax / 448); an
all-zero group stores zero codes with scale 1.
"""
from __future__ import annotations

import numpy as np

from . import codecs, rope as rope_mod


def quant_groups(y: np.ndarray, group: int):
    """Rows y [..., D] -> (codes uint8 [..., D], scales float32 [..., D // group]), group by group."""
    y = np.asarray(y, dtype=np.float64)
    d = y.shape[-1]
    if group < 1 or d % group:
        raise ValueError("group must divide the row length")
    flat = y.reshape(-1, d // group, group)
    codes = np.zeros(flat.shape, dtype=np.uint8)
    scales = np.zeros(flat.shape[:2], dtype=np.float32)
    for r in range(flat.shape[0]):
        for g in range(flat.shape[1]):
            codes[r, g], scales[r, g] = codecs.store_row(flat[r, g], codecs.FP8)
    return codes.reshape(y.shape), scales.reshape(y.shape[:-1] + (d // group,))


def inv_rope_quant(o: np.ndarray, q_pos, table: np.ndarray, rope_dims: int, group: int):
    """o [n_q][H][D] (attention output before the inverse rotation) -> (codes [n_q][H][D], scales [n_q][H][D/G])
    of the inverse-rotated output at each query's position."""
    y = rope_mod.inv_rope_queries(o, np.asarray(q_pos), table, rope_dims)
    return quant_groups(y, group)


def dequant(codes: np.ndarray, scales: np.ndarray, group: int) -> np.ndarray:
    """Exact fp64 values of grouped codes."""
    v = codecs.e4m3_to_f64(codes)
    d = codes.shape[-1]
    s = np.repeat(np.asarray(scales, dtype=np.float32).astype(np.float64), group, axis=-1)
    return (v.reshape(-1, d) * s.reshape(-1, d)).reshape(codes.shape)
