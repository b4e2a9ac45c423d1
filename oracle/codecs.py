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

fp4 (the indexer cache; [P1] "DeepSeek V4 Attention Architecture" (its memory figures) and the fp4
indexer-cache flag of [P2] "一、官方部署 Recipe" name an fp4 indexer cache without a format; reading R25) is OCP MXFP4, written from the OCP Microscaling Formats v1.0
definition: e2m1 elements (1 sign, 2 exponent bits with bias 1, 1 mantissa bit; magnitudes 0, 0.5, 1,
1.5, 2, 3, 4, 6; no infinities or NaN), and one E8M0 scale 2^X per block of 32 consecutive channels of
an entry, with X = floor(log2(amax of the block)) - 2 and elements rounded to nearest (ties to the even
code) after dividing by 2^X, saturating at 6.
"""
from __future__ import annotations

import numpy as np

F32, BF16, FP8, FP4 = "f32", "bf16", "fp8", "fp4"
E4M3_MAX = 448.0
MX_BLOCK = 32  # channels per E8M0 scale
E2M1_MAGS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])  # code & 7 -> magnitude


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


# ---------------------------------------------------------------- e2m1 + E8M0 (MXFP4, reading R25)
def e2m1_to_f64(codes) -> np.ndarray:
    """Value of 4-bit e2m1 codes (bit 3 = sign)."""
    c = np.asarray(codes, dtype=np.int64)
    return np.where(c & 8, -1.0, 1.0) * E2M1_MAGS[c & 7]


def f64_to_e2m1(x) -> np.ndarray:
    """Nearest e2m1 code of each value (ties to the code with mantissa bit 0), saturating at +-6.

    The sign bit is set for every negative input, so a negative value that rounds to zero keeps
    its sign (-0).
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), 6.0)
    d = np.abs(a[..., None] - E2M1_MAGS)  # distance to every magnitude
    best = np.argmin(d, axis=-1)          # first minimum = the lower code on a tie
    nxt = np.minimum(best + 1, 7)
    dist_best = np.take_along_axis(d, best[..., None], -1)[..., 0]
    dist_next = np.take_along_axis(d, nxt[..., None], -1)[..., 0]
    tie = (nxt != best) & (dist_best == dist_next)
    code = np.where(tie & (best & 1 == 1), nxt, best)  # on a tie keep the even code
    return (code | np.where(x < 0, 8, 0)).astype(np.uint8)


def mx_block_exponent(amax: float) -> int:
    """Shared exponent X of one block: floor(log2(amax)) - 2 (2 = largest e2m1 exponent), within the
    E8M0 range [-127, 127]; an all-zero block takes X = 0."""
    if amax == 0.0:
        return 0
    _, ex = np.frexp(amax)  # amax = f * 2^ex, f in [0.5, 1)
    return int(min(max(int(ex) - 1 - 2, -127), 127))


def f32_to_mxfp4(y32) -> tuple[np.ndarray, np.ndarray]:
    """One entry row (fp32 values, length a multiple of 32) -> (packed codes [D/2] uint8, E8M0 [D/32] uint8).

    Element 2j sits in the low nibble of byte j, element 2j+1 in the high nibble.
    """
    y = np.asarray(y32, dtype=np.float64)
    if y.shape[-1] % MX_BLOCK:
        raise ValueError("fp4 rows need a multiple of 32 channels")
    blocks = y.reshape(-1, MX_BLOCK)
    codes = np.empty(blocks.shape, dtype=np.uint8)
    exps = np.empty(blocks.shape[0], dtype=np.uint8)
    for j, blk in enumerate(blocks):
        X = mx_block_exponent(float(np.max(np.abs(blk))))
        codes[j] = f64_to_e2m1(np.ldexp(blk, -X))
        exps[j] = X + 127
    c = codes.reshape(-1)
    return (c[0::2] | (c[1::2] << 4)).astype(np.uint8), exps


def mxfp4_to_f64(packed, exps) -> np.ndarray:
    """Exact values of packed MXFP4 rows: packed [..., D/2] uint8, exps [..., D/32] uint8 (E8M0, X + 127)."""
    p = np.asarray(packed, dtype=np.uint8).astype(np.int64)
    c = np.stack([p & 15, p >> 4], axis=-1).reshape(p.shape[:-1] + (2 * p.shape[-1],))
    v = e2m1_to_f64(c)
    X = np.asarray(exps, dtype=np.int64) - 127
    return v * np.repeat(np.ldexp(1.0, X), MX_BLOCK, axis=-1)


# ---------------------------------------------------------------- entry store (reading R20)
def store_row(y: np.ndarray, dtype: str):
    """Round one fp64 row to the cache element type.

    Returns (stored, scale): stored is float32 / uint16 bf16 bits / uint8 e4m3
    codes / packed e2m1 codes; scale is the fp32 per-row scale (1.0 except for
    fp8), or for fp4 the row's E8M0 block exponents (uint8, X + 127).

    fp8 follows the per-entry amax rule in fp32 so that both sides take the
    same quantisation decisions: y32 = fl32(y), amax = max|y32|,
    inv = fl32(448 / amax), code = e4m3(fl32(y32 * inv)), scale = fl32(amax / 448);
    an all-zero row stores zeros with scale 1. fp4 rounds the row to fp32 first,
    then applies the MXFP4 block rule (f32_to_mxfp4).
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
    if dtype == FP4:
        return f32_to_mxfp4(f32(y))
    raise ValueError(dtype)


def load_rows(stored: np.ndarray, dtype: str, scales=None) -> np.ndarray:
    """Exact fp64 values of stored rows (fp8 rows multiplied by their scale, fp4 rows by their block scales)."""
    if dtype == F32:
        return np.asarray(stored, dtype=np.float32).astype(np.float64)
    if dtype == BF16:
        return bf16_to_f64(stored)
    if dtype == FP8:
        v = e4m3_to_f64(stored)
        if scales is not None:
            v = v * np.asarray(scales, dtype=np.float32).astype(np.float64)[..., None]
        return v
    if dtype == FP4:
        return mxfp4_to_f64(stored, scales)
    raise ValueError(dtype)
