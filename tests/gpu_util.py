"""Helpers for GPU parity tests: host <-> device conversion of stored element types and the comparison rules."""
from __future__ import annotations

import numpy as np
import torch

from oracle import codecs

DEV = "cuda"


def dev_f32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def dev_i32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def dev_bf16(bits) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).to(DEV).view(torch.bfloat16)


def dev_u8(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(DEV)


def dev_store(arr, dtype: str) -> torch.Tensor:
    """Host storage array (float32 / uint16 bf16 bits / uint8 codes) -> device tensor of that element type."""
    if dtype == codecs.F32:
        return dev_f32(arr)
    if dtype == codecs.BF16:
        return dev_bf16(arr)
    return dev_u8(arr)


def host_store(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> host storage array (float32 / uint16 bits / uint8)."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.cpu().numpy()
    return t.cpu().numpy().view(np.uint8)


def canary(shape, dtype: str) -> np.ndarray:
    if dtype == codecs.F32:
        return np.full(shape, np.nan, dtype=np.float32)
    if dtype == codecs.BF16:
        return np.full(shape, 0x7FC0, dtype=np.uint16)
    return np.full(shape, 0x7F, dtype=np.uint8)


# ------------------------------------------------------------------ comparison rules
def bf16_ulp_diff(got_bits: np.ndarray, ref_bits: np.ndarray) -> np.ndarray:
    """Distance in bf16 ulps (sign-magnitude ordering; +0 and -0 are 0 apart)."""
    def ordv(b):
        b = b.astype(np.int32)
        return np.where(b & 0x8000, -(b & 0x7FFF), b)
    return np.abs(ordv(got_bits) - ordv(ref_bits))


def assert_bf16_rows(got_bits, ref_bits, max_ulp: int = 1, row_slack: float = 2.0 ** -16):
    """Each element within `max_ulp` bf16 ulps of the oracle's rounding, plus row_slack * max|row|.

    The slack covers fp32 cancellation in the window sum: an element much smaller than its row can
    carry an fp32 error above one of its own bf16 ulps while staying far below the row's scale.
    """
    g = codecs.bf16_to_f64(got_bits)
    r = codecs.bf16_to_f64(ref_bits)
    mag = np.maximum(np.abs(r), 2.0 ** -126)
    ulp = np.ldexp(1.0, np.floor(np.log2(mag)).astype(int) - 7)
    rowmax = np.abs(r).max(axis=-1, keepdims=True)
    excess = np.abs(g - r) - (max_ulp * ulp + row_slack * rowmax)
    assert excess.max() <= 0, f"bf16 rows differ beyond {max_ulp} ulp (+slack): worst excess {excess.max():.3e}"
    return float(bf16_ulp_diff(got_bits, ref_bits).max())


def assert_fp8_rows(got_codes, got_scale, ref_codes, ref_scale, scale_rel: float = 2.0 ** -14):
    """Scales within scale_rel relative; each dequantised element within one e4m3 step of the oracle's
    code (times the scale) plus scale_rel * max|row|."""
    gs = np.asarray(got_scale, np.float64)
    rs = np.asarray(ref_scale, np.float64)
    srel = np.abs(gs - rs) / rs
    assert srel.max() <= scale_rel, f"fp8 scales differ by {srel.max():.3e} relative"
    gv = codecs.e4m3_to_f64(got_codes) * gs[:, None]
    rv = codecs.e4m3_to_f64(ref_codes) * rs[:, None]
    mag = np.maximum(np.abs(codecs.e4m3_to_f64(ref_codes)), 2.0 ** -6)
    step = np.ldexp(1.0, np.floor(np.log2(mag)).astype(int) - 3) * rs[:, None]
    rowmax = np.abs(rv).max(axis=-1, keepdims=True)
    excess = np.abs(gv - rv) - (step + scale_rel * rowmax)
    assert excess.max() <= 0, f"fp8 values differ by more than one step: worst excess {excess.max():.3e}"
    codes_equal = (got_codes == ref_codes) | ((got_codes & 0x7F) == 0) & ((ref_codes & 0x7F) == 0)
    return float(codes_equal.mean())


def rowwise_rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max over rows of max_d |got - ref| / max_d |ref| (rows = all leading axes)."""
    g = got.reshape(-1, got.shape[-1]).astype(np.float64)
    r = ref.reshape(-1, ref.shape[-1]).astype(np.float64)
    den = np.maximum(np.abs(r).max(axis=1), 1e-30)
    return float((np.abs(g - r).max(axis=1) / den).max())


def check_topk_near_ties(gpu_idx, gpu_cnt, ref_scores, k, delta):
    """GPU top-k set must equal the oracle set except for swaps within the rounding bound.

    ref_scores: fp64 oracle scores of all eligible entries; delta: per-entry rounding bound of the
    GPU score. Returns the number of certified swaps; raises if a swap is not certified.
    """
    n = ref_scores.shape[0]
    kk = min(k, n)
    assert gpu_cnt == kk
    got = set(int(i) for i in gpu_idx[:kk])
    assert all(0 <= i < n for i in got) and len(got) == kk
    assert np.all(np.asarray(gpu_idx[kk:]) == -1)
    assert list(gpu_idx[:kk]) == sorted(got)
    order = np.lexsort((np.arange(n), -ref_scores))
    ref = set(int(i) for i in order[:kk])
    diff = got ^ ref
    if kk == 0 or not diff:
        return 0
    thr = order[kk - 1]
    for i in diff:
        gap = abs(ref_scores[i] - ref_scores[thr])
        assert gap <= delta[i] + delta[thr] + 1e-300, f"uncertified top-k swap at entry {i} (gap {gap})"
    return len(diff) // 2


# ------------------------------------------------------------------ rounding-aware element bounds
def _bf16_spacing(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values at |x| (8 significant bits; the normal range suffices for N(0,1)-scale rows)."""
    mag = np.maximum(np.abs(np.asarray(x, np.float64)), 2.0 ** -126)
    return np.ldexp(1.0, np.floor(np.log2(mag)).astype(int) - 7)


def _e4m3_spacing(t: np.ndarray) -> np.ndarray:
    """Spacing of e4m3fn codes at |t| (4 significant bits, subnormal step 2^-9 below 2^-6)."""
    mag = np.maximum(np.abs(np.asarray(t, np.float64)), 2.0 ** -6)
    return np.ldexp(1.0, np.floor(np.log2(mag)).astype(int) - 3)


def _near_midpoint(v: np.ndarray, spacing: np.ndarray, eta: np.ndarray) -> np.ndarray:
    """True where v lies within eta of a midpoint between two neighbours of spacing `spacing`."""
    r = v / spacing
    return np.abs((r - np.floor(r)) - 0.5) * spacing <= eta


def stored_elem_bound(dtype: str, y_ref, ref, ref_scales, got, got_scales, row_slack: float = 2.0 ** -16):
    """Per-element bound u on |stored_gpu - stored_oracle| of compressed rows, asserted on the GPU rows.

    y_ref: the oracle's rows before storage rounding (fp32). The GPU computes the same row in fp32 with an
    error of at most eta = row_slack * max|row| (window sum, norm and rotation; the bf16 storage bar's
    slack). A stored element can therefore differ from the oracle's rounding only where y lies within that
    error of a rounding midpoint, and then by one step of the format. Elsewhere the codes must be equal.
    bf16: u = eta + one bf16 spacing where y is near a midpoint.
    fp8:  t = y * 448 / amax (the code domain); the GPU's t differs by at most 2 * 448 * row_slack plus
          fp32 rounding, so u = scale * (one e4m3 step where t is near a midpoint) + |value| * 2^-13
          (the scale's own tolerance).
    fp32: u = 1e-5 * max|row| (the fp32 cache bar).
    Returns u as an fp64 array of the rows' shape (dequantised units).
    """
    y = np.asarray(y_ref, np.float64)
    rowmax = np.abs(y).max(axis=-1, keepdims=True)
    if dtype == codecs.F32:
        u = np.broadcast_to(1e-5 * rowmax, y.shape).copy()
        gv, rv = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    elif dtype == codecs.BF16:
        rv, gv = codecs.bf16_to_f64(ref), codecs.bf16_to_f64(got)
        eta = row_slack * rowmax + 2.0 ** -23 * np.abs(y)
        sp = _bf16_spacing(rv)
        near = _near_midpoint(y, _bf16_spacing(y), eta)
        u = eta + np.where(near, sp, 0.0)
    elif dtype == codecs.FP8:
        rs = np.asarray(ref_scales, np.float64)[:, None]
        gs = np.asarray(got_scales, np.float64)[:, None]
        assert np.all(np.abs(gs - rs) <= 2.0 ** -14 * rs), "fp8 row scales differ beyond 2^-14 relative"
        rc, gc = codecs.e4m3_to_f64(ref), codecs.e4m3_to_f64(got)
        rv, gv = rc * rs, gc * gs
        amax = np.maximum(rowmax, 1e-300)
        t = y * (codecs.E4M3_MAX / amax)
        eta_t = 2.0 * codecs.E4M3_MAX * row_slack + 2.0 ** -20 * np.abs(t)
        near = _near_midpoint(t, _e4m3_spacing(t), eta_t)
        u = rs * np.where(near, _e4m3_spacing(rc), 0.0) + (np.abs(rv) + rs * _e4m3_spacing(rc)) * 2.0 ** -13
    else:
        raise ValueError(dtype)
    excess = np.abs(gv - rv) - u
    assert excess.max() <= 0, f"{dtype} stored rows differ beyond the rounding-aware bound: worst {excess.max():.3e}"
    return u


def wrelu_score_delta(keys_ref, u, q, head_w, mode: int, d_idx: int, h_idx: int):
    """Bound on |score_gpu(e) - score_oracle(e)| for every row of keys_ref [n][D] (fp64, the oracle's stored
    keys): the stored keys differ by at most u [n][D] (stored_elem_bound), and the GPU accumulates in fp32
    (2 (D + H + 2) 2^-24 of the absolute sum). ReLU and the non-negative head weights are 1-Lipschitz, so
    sum_h w_h sum_d |q_hd| u_ed bounds the storage part."""
    aq = np.abs(np.asarray(q, np.float64))                 # [H][D]
    w = np.ones(aq.shape[0]) if head_w is None else np.asarray(head_w, np.float64)
    store = (u @ aq.T) @ w                                   # [n]
    absum = ((np.abs(keys_ref) + u) @ aq.T) @ w
    return store + 2.0 * (d_idx + h_idx + 2) * 2.0 ** -24 * absum
