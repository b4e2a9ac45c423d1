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
