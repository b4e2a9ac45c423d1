"""Pins of the oracle's indexer score, top-k and attention: brute force, closed forms, torch SDPA, invariants."""
import numpy as np
import pytest
import torch

import synth
from oracle import attend as oa, codecs, compress as oc, index as oi, paging, rope
from tests import bruteforce as bf
from tests.oracle_fixtures import empty_cache


def _filled_cache(ratio, window, dim, rdims, dtype, lens, seed=21, grid=False):
    g = np.random.default_rng(seed)
    n_blocks = max(lens) // 256 + 2
    n_phys = len(lens) * n_blocks + 2
    c = empty_cache(ratio, window, dim, rdims, dtype, len(lens), n_blocks, n_phys, g)
    for b, n_tok in enumerate(lens):
        for i in range(paging.num_entries(n_tok, ratio, window)):
            y = synth.grid_values(g, (dim,)) if grid else g.standard_normal(dim)
            st, sc = codecs.store_row(y, dtype)
            sl = paging.entry_slot(c.block_table[b], i, ratio)
            c.pages[sl] = st
            if c.scales is not None:
                c.scales[sl] = sc
    return c


def _swa(dim, dtype, bt, n_phys, seed=22):
    g = synth.rng(seed, synth.STREAM_SWA)
    if dtype == "fp8":
        codes, sc = synth.e4m3_rows(g, n_phys * 256, dim)
        return oc.Raw("fp8", dim, 0, codes, None, sc, bt.copy())
    if dtype == "bf16":
        return oc.Raw("bf16", dim, 0, synth.normal_bf16_bits(g, (n_phys * 256, dim)), None, None, bt.copy())
    return oc.Raw("f32", dim, 0, synth.normal_f32(g, (n_phys * 256, dim)), None, None, bt.copy())


# ------------------------------------------------------------------ top-k
def test_topk_matches_bruteforce_sort():
    g = np.random.default_rng(30)
    for n in (0, 1, 5, 64, 300):
        s = np.round(g.standard_normal(n) * 4) / 4  # many ties
        for k in (1, 3, 64, 512):
            idx, sc, cnt = oi.topk(s, k)
            ref = bf.topk_sorted(list(map(float, s)), k)
            assert cnt == len(ref) == min(k, n)
            assert list(idx[:cnt]) == ref and np.all(idx[cnt:] == -1)
            assert np.array_equal(sc[:cnt], s[ref])


def test_topk_ties_take_lower_index_and_k_ge_n_takes_all():
    s = np.array([1.0, 2.0, 2.0, 2.0, 0.5, 2.0])
    assert list(oi.topk(s, 2)[0]) == [1, 2]
    assert list(oi.topk(s, 4)[0]) == [1, 2, 3, 5]
    assert list(oi.topk(s, 9)[0]) == [0, 1, 2, 3, 4, 5, -1, -1, -1]


def test_topk_signed_zero_and_nan():
    s = np.array([-0.0, 0.0, np.nan, -1.0, -0.0], dtype=np.float32)
    assert list(oi.topk(s, 2)[0]) == [0, 1]      # -0 == +0, lower index first
    assert list(oi.topk(s, 4)[0]) == [0, 1, 3, 4]  # NaN ranks below -1
    assert list(oi.topk(s, 5)[0]) == [0, 1, 2, 3, 4]


# ------------------------------------------------------------------ index score
@pytest.mark.parametrize("dtype", ["f32", "bf16", "fp8"])
def test_index_scores_match_bruteforce(dtype):
    c = _filled_cache(4, 8, 16, 8, dtype, [300, 90])
    g = np.random.default_rng(31)
    q = g.standard_normal((2, 3, 16))
    w = g.uniform(0, 1, (2, 3))
    q_pos = np.array([299, 77])
    for qi, (s, p) in enumerate(zip([0, 1], q_pos)):
        keys = oi.eligible_keys(c, s, p)
        assert keys.shape[0] == paging.num_eligible(int(p), 4, 8)
        got = oi.scores(keys, q[qi], w[qi], oi.WRELU)
        ref = [bf.wrelu_score(q[qi].tolist(), w[qi].tolist(), k.tolist()) for k in keys]
        assert np.allclose(got, ref, rtol=1e-13, atol=1e-12)
        got1 = oi.scores(keys, q[qi][:1], None, oi.DOT)
        assert np.allclose(got1, [bf.dot(q[qi][0].tolist(), k.tolist()) for k in keys], atol=1e-12)


def test_fp8_scale_factors_out_of_wrelu():
    c = _filled_cache(4, 8, 16, 8, "fp8", [400])
    g = np.random.default_rng(32)
    q, w = g.standard_normal((4, 16)), g.uniform(0, 1, 4)
    keys = oi.eligible_keys(c, 0, 399)
    raw = codecs.e4m3_to_f64(c.pages[[paging.entry_slot(c.block_table[0], i, 4) for i in range(keys.shape[0])]])
    sc = c.scales[[paging.entry_slot(c.block_table[0], i, 4) for i in range(keys.shape[0])]].astype(np.float64)
    assert np.allclose(oi.scores(keys, q, w, oi.WRELU), sc * oi.scores(raw, q, w, oi.WRELU), rtol=1e-13)


def test_index_topk_is_causal():
    c = _filled_cache(4, 8, 16, 8, "bf16", [600])
    g = np.random.default_rng(33)
    pos = np.array([6, 7, 8, 11, 100, 599])
    q = g.standard_normal((len(pos), 2, 16))
    w = g.uniform(0, 1, (len(pos), 2))
    idx, cnt, _ = oi.index_topk(c, np.zeros(len(pos), int), pos, q, w, oi.WRELU, 8)
    for qi, p in enumerate(pos):
        n = paging.num_eligible(int(p), 4, 8)
        assert cnt[qi] == min(8, n)
        assert np.all(idx[qi][: cnt[qi]] < n) and np.all(idx[qi][cnt[qi]:] == -1)
        for i in idx[qi][: cnt[qi]]:
            assert paging.entry_window(int(i), 4, 8)[1] <= p


# ------------------------------------------------------------------ attention
@pytest.mark.parametrize("dtype", ["f32", "bf16", "fp8"])
def test_dense_equals_topk_with_k_ge_n_elig_and_matches_sdpa(dtype):
    lens = [700, 301]
    c = _filled_cache(4, 8, 32, 16, dtype, lens)
    n_phys = c.pages.shape[0] // 64
    swa = _swa(32, dtype, c.block_table, n_phys)
    g = np.random.default_rng(34)
    q_pos = np.array([699, 300])
    q = g.standard_normal((2, 4, 32))
    table = rope.rope_table(1024, 16)
    dense, lse_d = oa.attend(c, swa, 128, [0, 1], q_pos, q, None, 0.3, False, table)
    n_el = [paging.num_eligible(int(p), 4, 8) for p in q_pos]
    tk = np.full((2, 256), -1, np.int32)
    for qi in range(2):
        tk[qi, : n_el[qi]] = np.arange(n_el[qi])
    sparse, lse_s = oa.attend(c, swa, 128, [0, 1], q_pos, q, tk, 0.3, False, table)
    assert np.allclose(dense, sparse, atol=1e-13) and np.allclose(lse_d, lse_s, atol=1e-12)
    for qi in range(2):
        keys = oa.gather_keys(c, swa, 128, qi, int(q_pos[qi]), list(range(n_el[qi])))
        assert keys.shape[0] == n_el[qi] + 128
        kt = torch.from_numpy(keys)[None, None]
        qt = torch.from_numpy(q[qi])[None, :, None, :]
        ref = torch.nn.functional.scaled_dot_product_attention(
            qt, kt.expand(1, 4, -1, -1), kt.expand(1, 4, -1, -1), scale=0.3)[0, :, 0].numpy()
        assert np.allclose(dense[qi], ref, atol=1e-12)
        bo, bl = bf.attend(q[qi].tolist(), keys.tolist(), 0.3)
        assert np.allclose(dense[qi], bo, atol=1e-12) and np.allclose(lse_d[qi], bl, atol=1e-12)


def test_single_key_and_zero_scale():
    keys = np.random.default_rng(35).standard_normal((7, 8))
    q = np.random.default_rng(36).standard_normal((3, 8))
    o, l = oa.attend_one(q, keys[:1], 0.7)
    assert np.allclose(o, np.tile(keys[0], (3, 1)), atol=1e-15)
    o0, l0 = oa.attend_one(q, keys, 0.0)
    assert np.allclose(o0, np.tile(keys.mean(axis=0), (3, 1)), atol=1e-15)
    assert np.allclose(l0, np.log(7.0), atol=1e-15)


def test_window_positions_and_selected_entries():
    c = _filled_cache(4, 8, 16, 8, "f32", [900])
    swa = _swa(16, "f32", c.block_table, c.pages.shape[0] // 64)
    for p, expect in ((0, 1), (5, 6), (127, 128), (700, 128)):
        k = oa.gather_keys(c, swa, 128, 0, p, [])
        assert k.shape[0] == expect
        lo = max(0, p - 127)
        assert np.array_equal(k[0], swa.kv_pages[paging.raw_slot(swa.block_table[0], lo)])
        assert np.array_equal(k[-1], swa.kv_pages[paging.raw_slot(swa.block_table[0], p)])


def test_translation_invariance_of_rotated_attention():
    """Shift every RoPE position by delta: output after inverse RoPE is unchanged (relative-position property)."""
    g = np.random.default_rng(37)
    dim, rd = 32, 16
    table = rope.rope_table(5000, rd)
    y_entries = g.standard_normal((20, dim))
    x_raw = g.standard_normal((300, dim))
    q0 = g.standard_normal((4, dim))
    outs = []
    for delta in (0, 256, 3584):
        n_phys = 30
        c = empty_cache(4, 8, dim, rd, "f32", 1, 20, n_phys, np.random.default_rng(38))
        swa = oc.Raw("f32", dim, 0, np.zeros((n_phys * 256, dim), np.float32), None, None, c.block_table.copy())
        base = 20 * 4 + delta  # entries are anchored at 4i + delta via a shifted sequence origin
        for i in range(20):
            c.pages[paging.entry_slot(c.block_table[0], i + delta // 4, 4)] = rope.rope(y_entries[i], table[4 * i + delta], rd)
        p = 180 + delta
        for j in range(p - 127, p + 1):
            swa.kv_pages[paging.raw_slot(swa.block_table[0], j)] = rope.rope(x_raw[j - delta], table[j], rd)
        q = np.stack([rope.rope(q0[h], table[p], rd) for h in range(4)])[None]
        tk = np.full((1, 32), -1, np.int32)
        tk[0, :20] = np.arange(20) + delta // 4
        o, _ = oa.attend(c, swa, 128, [0], [p], q, tk, 0.25, True, table)
        outs.append(o[0])
    for o in outs[1:]:
        assert np.allclose(o, outs[0], rtol=0, atol=2e-6 * np.abs(outs[0]).max())
