"""Pins of the oracle's compressor (weighted window sum, RMSNorm, RoPE, insert) and its streaming behaviour."""
import numpy as np
import pytest

import synth
from oracle import codecs, compress as oc, paging, rope
from tests import bruteforce as bf
from tests.oracle_fixtures import empty_cache, empty_state, pure_table, raw_tokens


def test_equal_logits_give_window_mean():
    g = np.random.default_rng(5)
    x = g.standard_normal((8, 16))
    z = oc.window_weighted_sum(x, np.full((8, 16), 0.37))
    assert np.allclose(z, x.mean(axis=0), rtol=0, atol=1e-14)
    x128 = g.standard_normal((128, 4))
    assert np.allclose(oc.window_weighted_sum(x128, np.zeros((128, 4))), x128.mean(axis=0), atol=1e-14)


def test_dominant_logit_copies_that_token():
    g = np.random.default_rng(6)
    x = g.standard_normal((8, 16))
    lg = g.standard_normal((8, 16))
    lg[5] += 800.0
    assert np.allclose(oc.window_weighted_sum(x, lg), x[5], atol=1e-12)


def test_constant_sequence_preserved_before_norm():
    x = np.tile(np.linspace(-2, 2, 16), (8, 1))
    lg = np.random.default_rng(7).standard_normal((8, 16))
    assert np.allclose(oc.window_weighted_sum(x, lg), x[0], atol=1e-14)


def test_rmsnorm_invariants():
    g = np.random.default_rng(8)
    z = g.standard_normal(512)
    y = oc.rmsnorm(z, np.ones(512), 1e-6)
    assert abs(np.sqrt(np.mean(y * y)) - 1.0) < 1e-6
    assert np.allclose(oc.rmsnorm(3.5 * z, np.ones(512), 0.0), oc.rmsnorm(z, np.ones(512), 0.0), atol=1e-14)
    gam = g.standard_normal(512)
    assert np.allclose(oc.rmsnorm(z, gam, 0.0), oc.rmsnorm(z, np.ones(512), 0.0) * gam, atol=1e-14)


def test_rope_table_against_pure_python_and_closed_form():
    t = rope.rope_table(300, 16)
    assert np.array_equal(t, np.array(pure_table(300, 16), dtype=np.float32))
    assert np.all(t[0, :, 0] == 1.0) and np.all(t[0, :, 1] == 0.0)
    assert np.allclose(t[:, 0, 0], np.cos(np.arange(300)), atol=6e-8)  # j = 0 has frequency 1
    big = rope.rope_table(1 << 20, 64)[(1 << 20) - 1]
    assert np.allclose(big[:, 0].astype(np.float64) ** 2 + big[:, 1].astype(np.float64) ** 2, 1.0, atol=2e-7)


def test_rope_inverse_and_norm():
    g = np.random.default_rng(9)
    t = rope.rope_table(5000, 64)
    y = g.standard_normal((3, 512))
    for p in (0, 1, 4095, 4999):
        r = rope.rope(y, t[p], 64)
        assert np.array_equal(r[:, :448], y[:, :448])
        pr = r[:, 448:].reshape(3, 32, 2)
        py = y[:, 448:].reshape(3, 32, 2)
        cs2 = t[p, :, 0].astype(np.float64) ** 2 + t[p, :, 1].astype(np.float64) ** 2
        assert np.allclose((pr ** 2).sum(-1), (py ** 2).sum(-1) * cs2, rtol=1e-12)
        back = rope.inv_rope(r, t[p], 64)
        assert np.allclose(back, y, rtol=0, atol=4e-7 * np.abs(y).max())


def test_rope_pairs_rotate_by_closed_form_angle():
    # D = R = 4: pair j = 0 turns at frequency 1, pair j = 1 at 10000^(-1/2) = 0.01
    t = rope.rope_table(50, 4)
    r = rope.rope(np.array([1.0, 0.0, 0.0, 1.0]), t[7], 4)
    assert np.allclose(r, [np.cos(7.0), np.sin(7.0), -np.sin(0.07), np.cos(0.07)], atol=1e-7)


@pytest.mark.parametrize("ratio,window,dim,rdims", [(4, 8, 16, 8), (4, 8, 8, 4), (128, 128, 8, 4)])
def test_compress_matches_pure_python_bruteforce(ratio, window, dim, rdims):
    n_tok = 300 if ratio == 128 else 45
    coff = window // ratio
    x, lg = raw_tokens(11, n_tok, dim, coff, "f32")
    gamma = synth.normal_f32(synth.rng(11, 20), (dim,))
    table = rope.rope_table(n_tok + 1, rdims)
    ref = bf.compress([list(map(float, r)) for r in x],
                      [[list(map(float, rr)) for rr in r] for r in lg],
                      ratio, window, list(map(float, gamma)), 1e-6,
                      [[(float(c), float(s)) for c, s in row] for row in table], rdims)
    n = paging.num_entries(n_tok, ratio, window)
    assert len(ref) == n
    for i in range(n):
        sl = slice(ratio * i, ratio * i + window)
        lrole = np.stack([lg[ratio * i + t, t // ratio] for t in range(window)])
        y = oc.compress_entry(x[sl], lrole, gamma, 1e-6, table[ratio * i], rdims)
        assert np.allclose(y, ref[i], rtol=0, atol=1e-12)


def _build(ratio, window, dim, rdims, dtype, lens, chunks, seed=12, bt_seed=13):
    """Run the oracle compress_insert over per-sequence chunk lists; returns (cache, state, slots list)."""
    batch = len(lens)
    g = np.random.default_rng(bt_seed)
    n_blocks = max(lens) // 256 + 2
    n_phys = batch * n_blocks + 3
    cache = empty_cache(ratio, window, dim, rdims, dtype, batch, n_blocks, n_phys, g)
    coff = window // ratio
    state = empty_state(dim, coff, "f32" if dtype == "f32" else "bf16", cache.block_table, n_phys)
    toks = [raw_tokens(seed + b, lens[b], dim, coff, state.dtype) for b in range(batch)]
    gamma = np.ones(dim, dtype=np.float32)
    table = rope.rope_table(max(lens) + 1, rdims)
    pos = [0] * batch
    all_slots = []
    for step in chunks:
        start = np.array(pos, dtype=np.int32)
        cu = np.concatenate([[0], np.cumsum(step)]).astype(np.int32)
        kv = np.concatenate([toks[b][0][pos[b]:pos[b] + step[b]] for b in range(batch)])
        lgn = np.concatenate([toks[b][1][pos[b]:pos[b] + step[b]] for b in range(batch)])
        slots, cnt = oc.compress_insert(cache, state, start, cu, kv, lgn, gamma, 1e-6, table, 64)
        all_slots.append((slots, cnt))
        pos = [pos[b] + step[b] for b in range(batch)]
    return cache, state, all_slots


@pytest.mark.parametrize("ratio,window", [(4, 8), (128, 128)])
@pytest.mark.parametrize("dtype", ["f32", "bf16", "fp8"])
def test_chunk_split_invariance(ratio, window, dtype):
    lens = [600, 517]
    one, _, s1 = _build(ratio, window, 16, 8, dtype, lens, [lens])
    parts, _, s2 = _build(ratio, window, 16, 8, dtype, lens, [[100, 3], [1, 250], [499, 264]])
    e = 256 // ratio
    for b, n_tok in enumerate(lens):
        for i in range(paging.num_entries(n_tok, ratio, window)):
            sl = paging.entry_slot(one.block_table[b], i, ratio)
            assert np.array_equal(one.pages[sl], parts.pages[sl], equal_nan=True)
    tot1 = s1[0][1]
    tot2 = sum(c for _, c in s2)
    assert np.array_equal(tot1, tot2)
    assert list(tot1) == [paging.num_entries(n, ratio, window) for n in lens]


def test_decode_one_token_at_a_time_equals_bulk():
    lens = [40]
    one, _, _ = _build(4, 8, 8, 4, "bf16", lens, [lens])
    steps, _, s = _build(4, 8, 8, 4, "bf16", lens, [[1]] * 40)
    n = paging.num_entries(40, 4, 8)
    for i in range(n):
        sl = paging.entry_slot(one.block_table[0], i, 4)
        assert np.array_equal(one.pages[sl], steps.pages[sl])
    completed = [int(c[0]) for _, c in s]
    # token at position p completes an entry iff p % 4 == 3 and p >= 7
    assert completed == [1 if (p % 4 == 3 and p >= 7) else 0 for p in range(40)]


def test_physical_placement_does_not_change_values():
    a, _, _ = _build(4, 8, 16, 8, "bf16", [700], [[700]], bt_seed=1)
    b, _, _ = _build(4, 8, 16, 8, "bf16", [700], [[700]], bt_seed=2)
    assert not np.array_equal(a.block_table, b.block_table)
    for i in range(paging.num_entries(700, 4, 8)):
        assert np.array_equal(a.pages[paging.entry_slot(a.block_table[0], i, 4)],
                              b.pages[paging.entry_slot(b.block_table[0], i, 4)])


def test_untouched_slots_stay_untouched():
    c, _, _ = _build(4, 8, 16, 8, "f32", [300], [[300]])
    written = {paging.entry_slot(c.block_table[0], i, 4) for i in range(paging.num_entries(300, 4, 8))}
    for r in range(c.pages.shape[0]):
        assert np.isnan(c.pages[r]).all() == (r not in written)


@pytest.mark.parametrize("ratio,window", [(4, 8), (128, 128)])
def test_compress_insert_through_pages_matches_bruteforce(ratio, window):
    lens = [389]
    cache, _, _ = _build(ratio, window, 8, 4, "f32", lens, [[200], [189]], seed=40)
    coff = window // ratio
    x, lg = raw_tokens(40, lens[0], 8, coff, "f32")
    table = rope.rope_table(lens[0] + 1, 4)
    ref = bf.compress([list(map(float, r)) for r in x], [[list(map(float, rr)) for rr in r] for r in lg],
                      ratio, window, [1.0] * 8, 1e-6, [[(float(c), float(s)) for c, s in row] for row in table], 4)
    assert len(ref) == paging.num_entries(lens[0], ratio, window)
    for i, r in enumerate(ref):
        got = cache.pages[paging.entry_slot(cache.block_table[0], i, ratio)].astype(np.float64)
        assert np.allclose(got, r, rtol=2 ** -23, atol=1e-7)
