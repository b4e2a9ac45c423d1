"""Seeded synthetic inputs for compressed sparse attention (c4a / c128a CSA).

This module only draws random numbers and random paging layouts. It holds none
of the method's arithmetic: no softmax, normalisation, rotation, rounding codec,
scoring or selection. Both the CPU oracle (through the tests) and the GPU path
receive exactly the arrays produced here.

Conventions
-----------
* Seeds follow ``seed = 1000 * config + stream`` with streams
  0 kv, 1 main logits, 2 indexer raw keys, 3 indexer logits, 4 q, 5 q_idx,
  6 head weights, 7 block tables, 8 lengths, 9 sliding-window rows.
* ``bf16`` samples are stored as ``uint16`` bit patterns. A bf16 sample is an
  fp32 N(0, 1) draw whose low 16 bits are dropped (sampling, not rounding).
* ``e4m3`` samples are stored as ``uint8`` codes plus an fp32 row scale.
  A row is drawn as N(0, 1) * (448 / 4), its fp32 pattern is truncated to three
  mantissa bits and clamped to the largest finite code; the row scale is 4/448.
  This mimics a per-row quantised N(0, 1) row without using any rounding rule.
"""
from __future__ import annotations

import numpy as np

STREAM_KV, STREAM_LOGIT, STREAM_IDX_KV, STREAM_IDX_LOGIT = 0, 1, 2, 3
STREAM_Q, STREAM_QIDX, STREAM_HEADW, STREAM_BT, STREAM_LEN, STREAM_SWA = 4, 5, 6, 7, 8, 9


def rng(config: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(1000 * config + stream))


def normal_f32(g: np.random.Generator, shape) -> np.ndarray:
    return g.standard_normal(size=shape, dtype=np.float32)


def normal_bf16_bits(g: np.random.Generator, shape) -> np.ndarray:
    """bf16 N(0,1) samples as uint16 bit patterns (fp32 draw, low half dropped)."""
    x = g.standard_normal(size=shape, dtype=np.float32)
    return (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def grid_values(g: np.random.Generator, shape, step: float = 0.5, lim: float = 2.0) -> np.ndarray:
    """Exact-grid values: round(N(0,1)/step) * step, clipped to [-lim, lim].

    Every value is a small multiple of a power of two, so sums of products of
    such values are exact in fp32 whatever the summation order.
    """
    x = np.rint(g.standard_normal(size=shape) / step) * step
    return np.clip(x, -lim, lim).astype(np.float32)


def uniform_f32(g: np.random.Generator, shape, lo=0.0, hi=1.0) -> np.ndarray:
    return g.uniform(lo, hi, size=shape).astype(np.float32)


def e4m3_rows(g: np.random.Generator, n_rows: int, dim: int):
    """Per-row 'quantised-looking' e4m3fn rows: (codes uint8 [n][dim], scale f32 [n])."""
    x = g.standard_normal(size=(n_rows, dim), dtype=np.float32) * np.float32(448.0 / 4.0)
    bits = x.view(np.uint32)
    sign = (bits >> np.uint32(31)).astype(np.uint8)
    mag = np.abs(x)
    # truncate magnitude to 3 mantissa bits (drop the low 20 bits of the fp32 pattern)
    tb = (mag.view(np.uint32) & np.uint32(0xFFF00000)).view(np.float32)
    tb = np.minimum(tb, np.float32(448.0))
    exp = ((tb.view(np.uint32) >> np.uint32(23)) & np.uint32(0xFF)).astype(np.int32) - 127
    man = ((tb.view(np.uint32) >> np.uint32(20)) & np.uint32(0x7)).astype(np.int32)
    code = np.zeros((n_rows, dim), dtype=np.int32)
    normal = exp >= -6
    code[normal] = ((exp[normal] + 7) << 3) | man[normal]
    # below the normal range: subnormal codes m * 2^-9, m = floor(|x| * 2^9)
    sub = ~normal
    code[sub] = np.minimum(np.floor(mag[sub].astype(np.float64) * 512.0), 7).astype(np.int32)
    code = code | (sign.astype(np.int32) << 7)
    scale = np.full((n_rows,), np.float32(4.0 / 448.0), dtype=np.float32)
    return code.astype(np.uint8), scale


def random_block_table(g: np.random.Generator, batch: int, n_blocks: int, n_phys: int) -> np.ndarray:
    """[batch][n_blocks] int32 physical ids drawn without replacement from range(n_phys)."""
    need = batch * n_blocks
    if need > n_phys:
        raise ValueError("pool too small for the requested block table")
    ids = g.permutation(n_phys)[:need] if n_phys <= 1 << 24 else g.choice(n_phys, size=need, replace=False)
    return ids.reshape(batch, n_blocks).astype(np.int32)


def lengths_uniform(g: np.random.Generator, batch: int, lo: int, hi: int) -> np.ndarray:
    """Per-sequence context lengths uniform in [lo, hi] (inclusive)."""
    return g.integers(lo, hi + 1, size=batch).astype(np.int32)
