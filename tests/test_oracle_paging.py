"""Pins of entry counts, windows, eligibility and slot mapping against the numbers the pages print."""
import json
import os

import numpy as np

from oracle import memory_model, paging

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_counts_match_printed_numbers():
    # context N with the query at position N means raw tokens 0..N exist
    assert paging.num_eligible(131072, 4, 8) == 32767
    assert paging.num_eligible(1048576, 4, 8) == 262143
    assert paging.num_eligible(65536, 128, 128) == 512
    assert paging.num_eligible(262144, 128, 128) == 2048
    assert paging.num_eligible(1024, 4, 8) == 255
    # about 250K c4a entries at 1M ([P1] architecture section), fewer than 8K c128a entries at 10^6 ([P3])
    assert 240_000 < paging.num_entries(1 << 20, 4, 8) < 270_000
    assert paging.num_entries(10 ** 6, 128, 128) < 8000
    assert paging.num_entries(1 << 20, 128, 128) == 8192


def test_entries_per_block():
    assert paging.entries_per_block(4) == 64
    assert paging.entries_per_block(128) == 2


def test_c4a_window_and_anchor_rule():
    for i in (0, 1, 5, 1000):
        assert paging.entry_window(i, 4, 8) == (4 * i, 4 * i + 7, 4 * i)
    assert paging.entry_window(3, 128, 128) == (384, 511, 384)


def test_worked_example_13_tokens():
    with open(os.path.join(GOLD, "c4a_13_tokens.json"), encoding="utf-8") as f:
        ex = json.load(f)
    m, w = ex["ratio"], ex["window"]
    n = paging.num_entries(ex["tokens"], m, w)
    assert [list(paging.entry_window(i, m, w)) for i in range(n)] == ex["entries_built"]
    p = ex["query_pos"]
    assert paging.num_eligible(p, m, w) == ex["n_eligible_at_query"]
    for pos, cnt in ex["eligible_steps"].items():
        assert paging.num_eligible(int(pos), m, w) == cnt
    lo = max(0, p - ex["swa_window"] + 1)
    assert (lo, p) == (ex["swa_first"], ex["swa_last"])
    assert paging.num_eligible(p, m, w) + (p - lo + 1) == ex["n_keys_with_k_ge_2"]


def test_eligibility_steps_exactly_at_window_ends():
    for m, w in ((4, 8), (128, 128)):
        prev = paging.num_eligible(0, m, w)
        for p in range(1, 2000):
            cur = paging.num_eligible(p, m, w)
            if (p - (w - 1)) % m == 0 and p >= w - 1:
                assert cur == prev + 1
            else:
                assert cur == prev
            # newest eligible entry's window ends at or before p; the next one's does not
            if cur:
                assert paging.entry_window(cur - 1, m, w)[1] <= p
            assert paging.entry_window(cur, m, w)[1] > p
            prev = cur


def test_slot_map_bruteforce_injective():
    g = np.random.default_rng(4)
    for m in (4, 128):
        e = paging.entries_per_block(m)
        bt = g.permutation(40)[:30].reshape(3, 10).astype(np.int32)
        seen = set()
        for s in range(3):
            for i in range(10 * e):
                slot = paging.entry_slot(bt[s], i, m)
                assert slot == bt[s][i // e] * e + i % e
                assert 0 <= slot < 40 * e
                seen.add(slot)
        assert len(seen) == 30 * e
        seen = set()
        for s in range(3):
            for j in range(10 * 256):
                seen.add(paging.raw_slot(bt[s], j))
        assert len(seen) == 30 * 256


def test_memory_model_reproduces_pages_figures():
    tok = 1 << 20
    v4 = memory_model.v4_bytes(tok) / memory_model.GIB
    v4_swa = memory_model.v4_bytes(tok, swa_tokens=128) / memory_model.GIB
    v32 = memory_model.v32_bytes(tok) / memory_model.GIB
    assert round(v4, 2) == 9.62 and round(v4_swa, 2) == 9.62
    assert round(v32, 1) == 83.9
    assert round(v32 / v4, 1) == 8.7
    small = memory_model.v4_bytes(tok, main_bytes=1.0, main_scale=4, idx_bytes=0.5, idx_scale=4) / memory_model.GIB
    assert 1.9 < v4 / small < 2.3  # about 2x further with fp8 attention + fp4 indexer
    # 1M = 10^6 does not reproduce the figures
    assert abs(memory_model.v4_bytes(10 ** 6) / memory_model.GIB - 9.62) > 0.3
