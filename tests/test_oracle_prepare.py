"""Pins of the oracle's fused query/window-key preparation (oracle/prepare.py): closed forms of the norm,
the identity rotation at position 0, translation back by the inverse rotation, and brute-force placement of
the window rows (every other row untouched)."""
import numpy as np
import pytest

from oracle import codecs, compress as oc, paging, prepare as op, rope as orope


def _swa(dtype, n_pages, dim, bt):
    if dtype == codecs.FP8:
        return oc.Raw(dtype, dim, 0, np.full((n_pages * 256, dim), 0x7F, np.uint8), None,
                      np.full(n_pages * 256, np.nan, np.float32), bt)
    fill = np.float32(np.nan) if dtype == codecs.F32 else np.uint16(0x7FC0)
    return oc.Raw(dtype, dim, 0, np.full((n_pages * 256, dim), fill,
                                          np.float32 if dtype == codecs.F32 else np.uint16), None, None, bt)


def test_norm_closed_form_at_position_zero():
    g = np.random.default_rng(1)
    q = g.standard_normal((2, 3, 64)) * 5.0
    table = orope.rope_table(4, 32)
    bt = np.array([[0], [1]], np.int32)
    out = op.prepare_qk(q, codecs.F32, g.standard_normal((2, 64)), [0, 1], [0, 0], np.ones(64), 0.0, table, 32,
                        _swa(codecs.F32, 2, 64, bt))
    ref = q / np.sqrt(np.mean(q * q, axis=-1, keepdims=True))  # rotation is the identity at position 0
    assert np.allclose(out, ref, rtol=1e-6, atol=1e-6)
    assert np.allclose(np.linalg.norm(out, axis=-1), 8.0, rtol=1e-6)  # |y| = sqrt(D) for gamma = 1, eps = 0


@pytest.mark.parametrize("p", [1, 300, 70000])
def test_inverse_rotation_recovers_the_normed_query(p):
    g = np.random.default_rng(p)
    q = g.standard_normal((1, 4, 128))
    gamma = g.uniform(0.5, 1.5, 128)
    table = orope.rope_table(p + 1, 64)
    bt = np.full((1, p // 256 + 1), -1, np.int32)
    bt[0, p // 256] = 0
    out = op.prepare_qk(q, codecs.F32, g.standard_normal((1, 128)), [0], [p], gamma, 1e-6, table, 64,
                        _swa(codecs.F32, 1, 128, bt))
    back = orope.inv_rope(out[0].astype(np.float64), table[p], 64)
    want = q[0] / np.sqrt(np.mean(q[0] ** 2, axis=-1, keepdims=True) + 1e-6) * gamma
    assert np.allclose(back, want, rtol=2e-6, atol=2e-6)


@pytest.mark.parametrize("dtype", [codecs.F32, codecs.BF16, codecs.FP8])
def test_window_rows_land_at_their_raw_slots(dtype):
    g = np.random.default_rng(5)
    positions, seqs = [0, 255, 256, 1000, 513], [0, 0, 1, 1, 0]
    bt = np.array([[3, 0, 5, 2], [1, 4, 6, 7]], np.int32)
    swa = _swa(dtype, 8, 32, bt)
    kv = g.standard_normal((5, 32))
    table = orope.rope_table(1001, 16)
    op.prepare_qk(g.standard_normal((5, 2, 32)), codecs.BF16, kv, seqs, positions, np.ones(32), 1e-6, table, 16, swa)
    written = set()
    for t, (s, p) in enumerate(zip(seqs, positions)):
        row = int(bt[s][p // 256]) * 256 + p % 256  # brute force: block table entry, then the offset
        assert row == paging.raw_slot(bt[s], p)
        written.add(row)
        want, sc = codecs.store_row(orope.rope(kv[t], table[p], 16), dtype)
        assert np.array_equal(swa.kv_pages[row], want)
        if dtype == codecs.FP8:
            assert swa.scales[row] == sc
    others = [r for r in range(8 * 256) if r not in written]
    if dtype == codecs.FP8:
        assert np.all(swa.kv_pages[others] == 0x7F)
    elif dtype == codecs.BF16:
        assert np.all(swa.kv_pages[others] == 0x7FC0)
    else:
        assert np.all(np.isnan(swa.kv_pages[others]))
