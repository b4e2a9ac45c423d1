"""Closed-form KV bytes per sequence (oracle, test infrastructure).

[P1] "DeepSeek V4 Attention Architecture" (and [P2], [P3]) quote 9.62 GiB of
bf16 KV per 1M-token sequence for DeepSeek V4 against 83.9 GiB for a 61-layer
V3.2-style stack (about 8.7x), and about 2x less again with an fp4 indexer and
fp8 attention cache. [P3] "注意力计算剪枝" gives the layer mix: about 30 c4a and
31 c128a layers. This module recomputes those numbers from entry counts so the
counting rule of the paging module is checked against the pages' figures.

Readings: 1M = 2^20 tokens (R1); main dim 512 and indexer dim 128, indexer on
c4a layers only; V3.2-style = 576 MLA dims + 128 indexer dims per token.
"""
from __future__ import annotations

from . import paging

GIB = float(1 << 30)


def v4_bytes(tokens: int, n_c4a: int = 30, n_c128a: int = 31, dim: int = 512, dim_idx: int = 128,
             main_bytes: float = 2.0, idx_bytes: float = 2.0, main_scale: int = 0, idx_scale: int = 0,
             swa_tokens: int = 0) -> float:
    """Bytes of compressed KV for one sequence of `tokens` raw tokens."""
    c4 = paging.num_entries(tokens, 4, 8)
    c128 = paging.num_entries(tokens, 128, 128)
    per_c4a = c4 * (dim * main_bytes + main_scale) + c4 * (dim_idx * idx_bytes + idx_scale)
    per_c128a = c128 * (dim * main_bytes + main_scale)
    swa = (n_c4a + n_c128a) * swa_tokens * dim * main_bytes
    return n_c4a * per_c4a + n_c128a * per_c128a + swa


def v32_bytes(tokens: int, layers: int = 61, mla_dims: int = 576, idx_dims: int = 128, elem: float = 2.0) -> float:
    return layers * tokens * (mla_dims + idx_dims) * elem
