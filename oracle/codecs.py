"""Storage codecs of the caches: fp32, bf16 and OCP fp8 e4m3fn (oracle, test infrastructure).

Cache element types come from the pages: bf16 caches for prefill and a
token-wise fp8 attention cache for decode ([P2] "二、注意力機制為什么這么麻煩";
[P1] "Deployment and Hardware Support" names the fp8 KV cache). The per-entry
fp8 scale rule is a reading (R20): amax / 448 per entry.

bf16 and e4m3fn are written from their format definitions:
* bf16: 1 sign, 8 exponent (bias 127), 7 mantissa bits -> the top half of fp32.
* e4m3fn: 1 sign, 4 exponent (bias 7), 3 mantissa bits; no infinities; the
  pattern S.1111.111 is NaN; largest finite magnitude 448; subnormal step 2^-9.
Rounding is round-to-nearest, ties to even, applied once to the exact value.
"""
from __future__ import annotations

import numpy as np

F32, BF16, FP8 = "f32", "bf16", "fp8"
E4M3_MAX = 448.0


def f32(x) -> np.ndarray:
    """Round to the nearest fp32 (ties to even) and return as float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


# ---------------------------------------------------------------- bf16
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def _rne_to_grid(x: np.ndarray, min_exp: int, man_bits: int) -> np.ndarray:
    """Round x to the nearest value with `man_bits` fraction bits (ties to even).

    The spacing at |x| in [2^e, 2^(e+1)) is 2^(e - man_bits), with e clamped
    below at `min_exp` (gradual underflow). x / spacing is exact in fp64.
    """
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    with np.errstate(divide="ignore"):
        _, ex = np.frexp(ax)  # ax = f * 2^ex, f in [0.5, 1)
    e = np.maximum(ex.astype(np.int64) - 1, min_exp)
    spacing = np.ldexp(1.0, (e - man_bits).astype(np.int64))
    return np.rint(x / spacing) * spacing


def f64_to_bf16(x) -> np.ndarray:
    """Nearest bf16 (ties to even) of the exact value, as uint16 bits."""
    q = _rne_to_grid(x, -126, 7)
    return (q.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# ---------------------------------------------------------------- e4m3fn
def _e4m3_table() -> np.ndarray:
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        s = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            vals[code] = np.nan
        elif e == 0:
            vals[code] = s * m * 2.0 ** -9
        else:
            vals[code] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


E4M3_VALUES = _e4m3_table()


def e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    return E4M3_VALUES[np.asarray(codes, dtype=np.uint8)]


def f64_to_e4m3(x) -> np.ndarray:
    """Nearest e4m3fn code (ties to even), saturating at +-448."""
    x = np.asarray(x, dtype=np.float64)
    q = _rne_to_grid(x, -6, 3)
    q = np.clip(q, -E4M3_MAX, E4M3_MAX)
    sign = np.signbit(q)
    aq = np.abs(q)
    with np.errstate(divide="ignore"):
        _, ex = np.frexp(aq)
    e = ex.astype(np.int64) - 1
    normal = aq >= 2.0 ** -6
    code = np.zeros(q.shape, dtype=np.int64)
    code[normal] = ((e[normal] + 7) << 3) | np.rint((aq[normal] / np.ldexp(1.0, e[normal]) - 1.0) * 8).astype(np.int64)
    code[~normal] = np.rint(aq[~normal] * 512.0).astype(np.int64)
    code = code | (sign.astype(np.int64) << 7)
    return code.astype(np.uint8)


# ---------------------------------------------------------------- entry store (reading R20)
def store_row(y: np.ndarray, dtype: str):
    """Round one fp64 row to the cache element type.

    Returns (stored, scale): stored is float32 / uint16 bf16 bits / uint8 e4m3
    codes; scale is the fp32 per-row scale (1.0 except for fp8).

    fp8 follows the per-entry amax rule in fp32 so that both sides take the
    same quantisation decisions: y32 = fl32(y), amax = max|y32|,
    inv = fl32(448 / amax), code = e4m3(fl32(y32 * inv)), scale = fl32(amax / 448);
    an all-zero row stores zeros with scale 1.
    """
    if dtype == F32:
        return np.asarray(y, dtype=np.float64).astype(np.float32), np.float32(1.0)
    if dtype == BF16:
        return f64_to_bf16(y), np.float32(1.0)
    if dtype == FP8:
        y32 = f32(y)
        amax = np.max(np.abs(y32))
        if amax == 0.0:
            return np.zeros(y32.shape, dtype=np.uint8), np.float32(1.0)
        inv = f32(E4M3_MAX / amax)
        codes = f64_to_e4m3(f32(y32 * inv))
        return codes, np.float32(f32(amax / E4M3_MAX))
    raise ValueError(dtype)


def load_rows(stored: np.ndarray, dtype: str, scales=None) -> np.ndarray:
    """Exact fp64 values of stored rows (fp8 rows multiplied by their scale)."""
    if dtype == F32:
        return np.asarray(stored, dtype=np.float32).astype(np.float64)
    if dtype == BF16:
        return bf16_to_f64(stored)
    if dtype == FP8:
        v = e4m3_to_f64(stored)
        if scales is not None:
            v = v * np.asarray(scales, dtype=np.float32).astype(np.float64)[..., None]
        return v
    raise ValueError(dtype)
