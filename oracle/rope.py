"""Rotary position embedding and its inverse (oracle, test infrastructure).

Sources: the compressed entry is rotated at its anchor before insertion
([P2] "3.2 內核", compressor + RMSNorm + RoPE + cache write; [P3] "KV 缓存压缩",
anchor 4i). Because K and V are shared, the attention output carries absolute
position and an inverse rotation at the query position restores relative
position ([P1] "DeepSeek V4 Attention Architecture"; [P2] "二、注意力機制為什么這么麻煩").

Readings: interleaved pairs on the trailing R dims, theta = 10000, no context
scaling (R7); cos/sin are taken from an fp32 table [rows][R/2][2] built in fp64
and rounded to nearest (R8), so both sides rotate with table values.
"""
from __future__ import annotations

import numpy as np


def rope_table(rows: int, rope_dims: int, theta: float = 10000.0) -> np.ndarray:
    """fp32 [rows][R/2][2] (cos, sin) of angle p * theta^(-2j/R), computed in fp64."""
    half = rope_dims // 2
    j = np.arange(half, dtype=np.float64)
    inv_freq = theta ** (-2.0 * j / rope_dims)
    ang = np.arange(rows, dtype=np.float64)[:, None] * inv_freq[None, :]
    out = np.empty((rows, half, 2), dtype=np.float32)
    out[:, :, 0] = np.cos(ang)
    out[:, :, 1] = np.sin(ang)
    return out


def rope(y: np.ndarray, cs_row: np.ndarray, rope_dims: int) -> np.ndarray:
    """Rotate pairs (D-R+2j, D-R+2j+1) of y (last axis D) by the table row: (u,v) -> (uc - vs, us + vc)."""
    y = np.array(y, dtype=np.float64, copy=True)
    if rope_dims == 0:
        return y
    d = y.shape[-1]
    c = cs_row[:, 0].astype(np.float64)
    s = cs_row[:, 1].astype(np.float64)
    u = y[..., d - rope_dims::2].copy()
    v = y[..., d - rope_dims + 1::2].copy()
    y[..., d - rope_dims::2] = u * c - v * s
    y[..., d - rope_dims + 1::2] = u * s + v * c
    return y


def inv_rope(y: np.ndarray, cs_row: np.ndarray, rope_dims: int) -> np.ndarray:
    """Inverse rotation: (u,v) -> (uc + vs, -us + vc)."""
    y = np.array(y, dtype=np.float64, copy=True)
    if rope_dims == 0:
        return y
    d = y.shape[-1]
    c = cs_row[:, 0].astype(np.float64)
    s = cs_row[:, 1].astype(np.float64)
    u = y[..., d - rope_dims::2].copy()
    v = y[..., d - rope_dims + 1::2].copy()
    y[..., d - rope_dims::2] = u * c + v * s
    y[..., d - rope_dims + 1::2] = -u * s + v * c
    return y


def inv_rope_queries(x: np.ndarray, q_pos: np.ndarray, table: np.ndarray, rope_dims: int) -> np.ndarray:
    """Inverse RoPE of an output block [n_q][H][D] at each query's position."""
    out = np.array(x, dtype=np.float64, copy=True)
    for qi, p in enumerate(np.asarray(q_pos)):
        out[qi] = inv_rope(out[qi], table[int(p)], rope_dims)
    return out
