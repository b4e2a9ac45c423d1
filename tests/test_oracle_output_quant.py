"""Pins of the oracle's inverse-RoPE + fp8 output quantisation (oracle/output_quant.py).

The quantisation is checked against torch's own e4m3fn cast (an implementation independent of the oracle's
codec) group by group; the rotation against the closed form at position 0 and against the forward rotation.
"""
import numpy as np
import pytest
import torch

from oracle import codecs, output_quant as oq, rope as orope


def _torch_group(y32: np.ndarray):
    """One group by the scale rule written with torch fp32 ops and torch's e4m3fn cast."""
    t = torch.from_numpy(y32.astype(np.float32))
    amax = t.abs().max()
    if amax == 0:
        return np.zeros(y32.shape, np.uint8), np.float32(1.0)
    inv = torch.tensor(448.0, dtype=torch.float32) / amax
    codes = (t * inv).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, np.float32((amax / torch.tensor(448.0, dtype=torch.float32)).item())


@pytest.mark.parametrize("group", [8, 32, 128, 512])
def test_groups_match_torch_cast(group):
    g = np.random.default_rng(group)
    y = g.standard_normal((3, 4, 512)) * g.uniform(0.01, 50, (3, 4, 1))
    codes, scales = oq.quant_groups(y, group)
    assert codes.shape == y.shape and scales.shape == (3, 4, 512 // group)
    y32 = y.astype(np.float32)
    for i in range(3):
        for h in range(4):
            for k in range(512 // group):
                sl = slice(k * group, (k + 1) * group)
                rc, rs = _torch_group(y32[i, h, sl])
                assert np.array_equal(codes[i, h, sl], rc)
                assert scales[i, h, k] == rs


def test_group_maximum_maps_to_448_and_zero_group():
    y = np.zeros((1, 1, 256))
    y[0, 0, 5] = -3.25          # group 0: a single non-zero
    y[0, 0, 128:] = np.linspace(-1, 2, 128)
    codes, scales = oq.quant_groups(y, 64)
    assert codes[0, 0, 5] == 0xFE and scales[0, 0, 0] == np.float32(3.25 / 448)
    assert not codes[0, 0, 64:128].any() and scales[0, 0, 1] == 1.0  # all-zero group
    assert codes[0, 0, 255] == 0x7E                                  # the group maximum 2.0
    with pytest.raises(ValueError):
        oq.quant_groups(y, 100)


def test_position_zero_is_plain_quantisation():
    g = np.random.default_rng(7)
    o = g.standard_normal((2, 3, 128))
    table = orope.rope_table(4, 64)
    assert np.all(table[0, :, 0] == 1.0) and np.all(table[0, :, 1] == 0.0)
    c1, s1 = oq.inv_rope_quant(o, [0, 0], table, 64, 32)
    c2, s2 = oq.quant_groups(o, 32)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)
    c3, s3 = oq.inv_rope_quant(o, [3, 1], table, 0, 32)  # no rotated dims
    assert np.array_equal(c3, c2) and np.array_equal(s3, s2)


@pytest.mark.parametrize("p", [1, 1000, 65536])
def test_inverse_of_forward_rotation_within_one_step(p):
    """Quantising inv_rope(rope(y, p), p) gives y back to within one e4m3 step of each group's scale."""
    g = np.random.default_rng(p)
    y = g.standard_normal((1, 8, 512))
    table = orope.rope_table(p + 1, 64)
    rotated = np.stack([orope.rope(y[0, h], table[p], 64) for h in range(8)])[None]
    codes, scales = oq.inv_rope_quant(rotated, [p], table, 64, 128)
    deq = oq.dequant(codes, scales, 128)
    step = np.repeat(scales.astype(np.float64), 128, axis=-1) * 32.0  # e4m3 step at the top binade (256..448)
    assert np.all(np.abs(deq - y) <= step)
    ref_codes, _ = oq.quant_groups(y, 128)
    assert np.mean(codes == ref_codes) > 0.95  # only elements at rounding ties of the rotation may move
