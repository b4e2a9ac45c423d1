"""GPU parity at the configurations' full sizes, in the launch configuration the benchmark times.

The oracle cannot run every query of these workloads in seconds, so each test checks
* integer results in full: entry counts, slots, and the top-k sets of every query it computes (exact-grid
  indexer keys, queries and head weights make every fp32 score exact in any summation order, so the sets
  and the scores must match bit for bit), plus size-independent properties of the top-k lists of all
  queries (count, order, range);
* floating-point results (compressed entries, attention outputs) on entries and queries the oracle computes
  one by one.
Compressed-cache rows and pool pages that the step must not read hold NaN codes, so a gather from a wrong row
shows up as a NaN or a mismatch. Inputs are drawn by `synth` on the host and copied to the device; no value
produced by the GPU path is handed to the oracle.
"""
import math

import numpy as np
import pytest
import torch

import long_context_compressed_compress_amd as csa
import synth
from oracle import attend as oa, codecs, compress as oc, index as oi, paging, rope as orope
from tests import gpu_util as gu
from tests import stage_inputs as si

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-3, "fp8": 5e-2}
H, D, R = 64, 512, 64
H_IDX, D_IDX, R_IDX = 64, 128, 64
K_TOP, SWA = 512, 128
BF16_NAN, FP8_NAN = 0x7FC0, 0x7F


def _log(msg):
    print(msg, flush=True)


def _fresh():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _ragged_table(g, n_blocks, n_phys):
    """[B][max blocks] int32 table of distinct physical ids drawn from range(n_phys), -1 beyond each row's blocks."""
    need = int(sum(n_blocks))
    ids = g.permutation(n_phys)[:need].astype(np.int32)
    bt = np.full((len(n_blocks), max(n_blocks)), -1, np.int32)
    o = 0
    for b, nb in enumerate(n_blocks):
        bt[b, :nb] = ids[o:o + nb]
        o += nb
    return bt


def _tail_table(g, positions, bt_stride, first_rel=-1, last_rel=0):
    """Table mapping only logical blocks p//256 + first_rel .. p//256 + last_rel of each sequence (window and
    compressor-state pages), onto a small pool of its own; returns (table, n_pages)."""
    B = len(positions)
    per = last_rel - first_rel + 1
    ids = g.permutation(B * per).astype(np.int32)
    bt = np.full((B, bt_stride), -1, np.int32)
    for b, p in enumerate(positions):
        for j, rel in enumerate(range(first_rel, last_rel + 1)):
            blk = int(p) // 256 + rel
            if 0 <= blk < bt_stride:
                bt[b, blk] = ids[b * per + j]
    return bt, B * per


def _slot_array(bt_row, entries, ratio):
    return np.array([paging.entry_slot(bt_row, int(i), ratio) for i in entries], np.int64)


def _topk_properties(out, cnt, positions, ratio, window, k):
    """Size-independent facts of every top-k row: count, ascending distinct eligible indices, -1 padding."""
    for q, p in enumerate(positions):
        n = min(k, paging.num_eligible(int(p), ratio, window))
        assert cnt[q] == n, f"query {q}: count {cnt[q]} != {n}"
        row = out[q]
        assert np.all(row[n:] == -1)
        sel = row[:n]
        assert np.all(sel >= 0) and np.all(sel < paging.num_eligible(int(p), ratio, window))
        assert np.all(np.diff(sel) > 0)


def _run_index(cache, q_seq, q_pos, max_elig, q_idx, w, k):
    """index_score + index_select as two calls on one workspace (the benchmark's launch configuration)."""
    n_q = q_idx.shape[0]
    ws = csa.index_workspace(n_q, max_elig, k, q_idx.shape[1])
    out = torch.full((n_q, k), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((n_q,), -7, dtype=torch.int32, device="cuda")
    sc = torch.zeros((n_q, k), dtype=torch.float32, device="cuda")
    csa.index_score(cache, q_seq, q_pos, max_elig, q_idx, w, oi.WRELU, k, ws)
    csa.index_select(cache, q_seq, q_pos, max_elig, k, out, ws, cnt, sc)
    torch.cuda.synchronize()
    del ws
    return out.cpu().numpy(), cnt.cpu().numpy(), sc.cpu().numpy()


def _run_attend(cache, swa, q_seq, q_pos, q, topk, max_elig, rope_cs):
    n_q = q.shape[0]
    k = 0 if topk is None else topk.shape[1]
    need = csa.attend_workspace(n_q, H, D, (k if topk is not None else max_elig) + SWA)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    out = torch.full((n_q, H, D), -7.0, device="cuda")
    lse = torch.full((n_q, H), -7.0, device="cuda")
    csa.attend(cache, swa, SWA, q_seq, q_pos, q, topk, max_elig, 1.0 / math.sqrt(D), True, rope_cs, out, lse,
               workspace=ws)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def _check_attend(out, lse, o_out, o_lse, dtype, label):
    err = gu.rowwise_rel_err(out, o_out)
    _log(f"{label}: attention rowwise rel err {err:.3e} over {out.shape[0]} queries")
    assert np.all(np.isfinite(out))
    assert err <= TOL[dtype]
    assert np.allclose(lse, o_lse, rtol=0, atol=1e-4)


# ------------------------------------------------------------------ c4a bf16 decode: batch 32, context 96K-128K
C3 = 3


def _c3_lengths():
    return synth.lengths_uniform(synth.rng(C3, synth.STREAM_LEN), 32, 98304, 131072)


def test_c3_decode_full_size_index_and_attend():
    """Index score + select and attention for all 32 queries of the benchmark workload, at its sizes and launch
    configuration: top-k sets and scores bit-exact on exact-grid indexer inputs, outputs within 2e-3."""
    _fresh()
    lens = _c3_lengths()
    B = len(lens)
    _log(f"c3 full size: batch {B}, contexts {lens.min()}..{lens.max()}")
    n_blocks = [int(L) // 256 + 1 for L in lens]
    n_phys = int(math.ceil(1.25 * sum(n_blocks)))
    bt = _ragged_table(synth.rng(C3, synth.STREAM_BT), n_blocks, n_phys)
    # indexer cache: exact-grid rows on every mapped page, NaN on the spare pages
    ipages = np.full((n_phys, 64, D_IDX), BF16_NAN, np.uint16)
    mapped = bt[bt >= 0]
    ipages[mapped] = si.grid_bf16(synth.grid_values(synth.rng(C3, synth.STREAM_IDX_KV), (mapped.size, 64, D_IDX)))
    ipages = ipages.reshape(n_phys * 64, D_IDX)
    q_idx = si.grid_bf16(synth.grid_values(synth.rng(C3, synth.STREAM_QIDX), (B, H_IDX, D_IDX)))
    w = si.grid_weights(synth.rng(C3, synth.STREAM_HEADW), (B, H_IDX))
    pos = lens.astype(np.int64)
    max_elig = max(paging.num_eligible(int(p), 4, 8) for p in pos)

    o_idx, o_cnt, o_sc = oi.index_topk(oc.Cache(4, 8, D_IDX, R_IDX, "bf16", ipages, None, bt), np.arange(B), pos,
                                       codecs.load_rows(q_idx, "bf16"), w, oi.WRELU, K_TOP)
    g_bt = gu.dev_i32(bt)
    g_seq, g_pos = gu.dev_i32(np.arange(B)), gu.dev_i32(pos)
    icache = csa.Cache(4, 8, D_IDX, R_IDX, gu.dev_bf16(ipages), g_bt)
    out, cnt, sc = _run_index(icache, g_seq, g_pos, max_elig, gu.dev_bf16(q_idx), gu.dev_f32(w), K_TOP)
    del icache
    assert np.array_equal(cnt, o_cnt)
    assert np.array_equal(out, o_idx)
    m = o_idx >= 0
    assert np.array_equal(sc[m].astype(np.float64), o_sc[m])
    _topk_properties(out, cnt, pos, 4, 8, K_TOP)
    _log("c3 full size: 32 top-k sets and scores bit-exact")

    # attention: selected rows hold N(0,1) bf16 entries, every other row of the main cache is NaN
    mpages = np.full((n_phys * 64, D), BF16_NAN, np.uint16)
    g = synth.rng(C3, synth.STREAM_KV)
    for b in range(B):
        mpages[_slot_array(bt[b], o_idx[b][o_idx[b] >= 0], 4)] = synth.normal_bf16_bits(g, (int(o_cnt[b]), D))
    tail, n_tail = _tail_table(synth.rng(C3, 17), pos, bt.shape[1])
    swa_pages = synth.normal_bf16_bits(synth.rng(C3, synth.STREAM_SWA), (n_tail * 256, D))
    q = synth.normal_bf16_bits(synth.rng(C3, synth.STREAM_Q), (B, H, D))
    rows = int(pos.max()) + 2
    table = orope.rope_table(rows, R)
    o_out, o_lse = oa.attend(oc.Cache(4, 8, D, R, "bf16", mpages, None, bt), oc.Raw("bf16", D, 0, swa_pages, None,
                             None, tail), SWA, np.arange(B), pos, codecs.load_rows(q, "bf16"), o_idx,
                             1.0 / math.sqrt(D), True, table)
    cache = csa.Cache(4, 8, D, R, gu.dev_bf16(mpages), g_bt)
    swa = csa.Raw(D, 0, gu.dev_bf16(swa_pages), gu.dev_i32(tail))
    g_out, g_lse = _run_attend(cache, swa, g_seq, g_pos, gu.dev_bf16(q), gu.dev_i32(out), max_elig,
                               csa.rope_table(rows, R))
    _check_attend(g_out, g_lse, o_out, o_lse, "bf16", "c3 full size")


@pytest.mark.parametrize("which", ["main", "indexer"])
def test_c3_compress_full_length(which):
    """compress_insert of the shortest and the longest sequence of the benchmark workload from position 0 in one
    call (the way the benchmark builds its caches): counts and slots in full, unwritten rows untouched, and 400
    entries per sequence (first, last and random ones) against the oracle within one bf16 ulp."""
    _fresh()
    lens = _c3_lengths()
    pick = [int(np.argmin(lens)), int(np.argmax(lens))]
    Ls = [int(lens[b]) + 1 for b in pick]  # raw tokens 0..L_b
    dim, rdim = (D, R) if which == "main" else (D_IDX, R_IDX)
    _log(f"c3 compress {which}: sequences of {Ls} tokens, dim {dim}")
    g = synth.rng(C3, 50 if which == "main" else 51)
    n_blocks = [L // 256 + 1 for L in Ls]
    n_phys = sum(n_blocks) + 3
    bt = _ragged_table(synth.rng(C3, 52), n_blocks, n_phys)
    kv = [synth.normal_bf16_bits(g, (L, dim)) for L in Ls]
    lg = [synth.normal_bf16_bits(g, (L, 2, dim)) for L in Ls]
    gamma = synth.uniform_f32(g, (dim,), 0.5, 1.5)
    rows = max(Ls) + 1
    # state pages: only the last two blocks of each sequence are mapped (the rest of a chunk is read from the input)
    tail, n_tail = _tail_table(synth.rng(C3, 53), [L - 1 for L in Ls], bt.shape[1])
    max_out = (max(Ls) + 3) // 4
    cache = csa.Cache(4, 8, dim, rdim, gu.dev_bf16(np.full((n_phys * 64, dim), BF16_NAN, np.uint16)), gu.dev_i32(bt))
    state = csa.Raw(dim, 2, torch.zeros((n_tail * 256, dim), dtype=torch.bfloat16, device="cuda"), gu.dev_i32(tail),
                    torch.zeros((n_tail * 256, 2, dim), dtype=torch.bfloat16, device="cuda"))
    slots = torch.full((2, max_out), -7, dtype=torch.int32, device="cuda")
    counts = torch.full((2,), -7, dtype=torch.int32, device="cuda")
    cu = np.array([0, Ls[0], Ls[0] + Ls[1]], np.int32)
    csa.compress_insert(cache, state, gu.dev_i32([0, 0]), gu.dev_i32(cu), gu.dev_bf16(np.concatenate(kv)),
                        gu.dev_bf16(np.concatenate(lg)), gu.dev_f32(gamma), 1e-6, csa.rope_table(rows, rdim),
                        max(Ls), slots, counts)
    torch.cuda.synchronize()
    gp = gu.host_store(cache.pages)
    slots, counts = slots.cpu().numpy(), counts.cpu().numpy()
    del cache, state
    table = orope.rope_table(rows, rdim)
    written = np.zeros(gp.shape[0], bool)
    sample_rng = synth.rng(C3, 54)
    for b, L in enumerate(Ls):
        n = paging.num_entries(L, 4, 8)
        assert counts[b] == n
        want = _slot_array(bt[b], range(n), 4)
        assert np.array_equal(slots[b, :n], want) and np.all(slots[b, n:] == -1)
        written[want] = True
        # the oracle reads the window rows of the sequence through an identity table over its own tokens
        nb = L // 256 + 1
        kvp = np.zeros((nb * 256, dim), np.uint16)
        lgp = np.zeros((nb * 256, 2, dim), np.uint16)
        kvp[:L], lgp[:L] = kv[b], lg[b]
        ostate = oc.Raw("bf16", dim, 2, kvp, lgp, None, np.arange(nb, dtype=np.int32)[None])
        ents = np.unique(np.concatenate([[0, 1, 2, n - 3, n - 2, n - 1], sample_rng.choice(n, 394, replace=False)]))
        ref = np.stack([codecs.store_row(oc.compress_entry(*oc.window_rows(ostate, ostate.block_table[0], int(i), 4, 8),
                                                           gamma, 1e-6, table[4 * int(i)], rdim), "bf16")[0]
                        for i in ents])
        ulp = gu.assert_bf16_rows(gp[want[ents]], ref)
        _log(f"c3 compress {which} seq {b}: {n} entries, {ents.size} checked, max ulp diff {ulp:.0f}")
    assert np.all(gp[~written] == BF16_NAN), "a slot outside the new entries changed"


# ------------------------------------------------------------------ c4a fp8 decode at 1M: batch 4, 200 GB pool
C4 = 4
POOL_BYTES = 200 * 10 ** 9


def test_c4_1m_fp8_index_and_attend():
    """Batch 4 at position 2^20 with fp8 indexer, main and window caches, pages drawn uniformly from a 200 GB pool
    (byte offsets far beyond 32 bits): top-k sets bit-exact, attention within 5e-2."""
    _fresh()
    B, P = 4, 1 << 20
    nb = P // 256 + 1
    per_page = 64 * D + 64 * D_IDX + 2 * 64 * 4
    n_phys = POOL_BYTES // per_page
    _log(f"c4 1M fp8: batch {B}, {nb} blocks per sequence over a pool of {n_phys} pages ({POOL_BYTES / 1e9:.0f} GB)")
    bt = synth.random_block_table(synth.rng(C4, synth.STREAM_BT), B, nb, n_phys)
    compact = np.arange(B * nb, dtype=np.int32).reshape(B, nb)  # the oracle sees the same pages packed together
    ids = gu.dev_i32(bt.reshape(-1)).long()
    # indexer: exact-grid e4m3 codes with scale 1 on the sequences' pages, NaN codes everywhere else
    icodes = si.grid_e4m3(synth.grid_values(synth.rng(C4, synth.STREAM_IDX_KV), (B * nb * 64, D_IDX)))
    iscale = np.ones(B * nb * 64, np.float32)
    g_ipages = torch.full((n_phys * 64, D_IDX), FP8_NAN, dtype=torch.uint8, device="cuda")
    g_iscales = torch.full((n_phys * 64,), float("nan"), device="cuda")
    g_ipages.view(n_phys, 64 * D_IDX)[ids] = gu.dev_u8(icodes).view(B * nb, 64 * D_IDX)
    g_iscales.view(n_phys, 64)[ids] = gu.dev_f32(iscale).view(B * nb, 64)
    q_idx = si.grid_bf16(synth.grid_values(synth.rng(C4, synth.STREAM_QIDX), (B, H_IDX, D_IDX)))
    w = si.grid_weights(synth.rng(C4, synth.STREAM_HEADW), (B, H_IDX))
    pos = np.full(B, P, np.int64)
    max_elig = paging.num_eligible(P, 4, 8)
    o_idx, o_cnt, o_sc = oi.index_topk(oc.Cache(4, 8, D_IDX, R_IDX, "fp8", icodes, iscale, compact), np.arange(B), pos,
                                       codecs.load_rows(q_idx, "bf16"), w, oi.WRELU, K_TOP)
    del icodes
    g_bt = gu.dev_i32(bt)
    g_seq, g_pos = gu.dev_i32(np.arange(B)), gu.dev_i32(pos)
    icache = csa.Cache(4, 8, D_IDX, R_IDX, g_ipages, g_bt, g_iscales)
    out, cnt, sc = _run_index(icache, g_seq, g_pos, max_elig, gu.dev_bf16(q_idx), gu.dev_f32(w), K_TOP)
    del icache, g_ipages, g_iscales
    _fresh()
    assert np.array_equal(cnt, o_cnt)
    assert np.array_equal(out, o_idx)
    m = o_idx >= 0
    assert np.array_equal(sc[m].astype(np.float64), o_sc[m])
    _log("c4 1M fp8: 4 top-k sets over 262143 entries bit-exact")

    # main cache: e4m3 rows (per-entry scale) on the selected entries only, NaN codes and scales everywhere else
    g_mpages = torch.full((n_phys * 64, D), FP8_NAN, dtype=torch.uint8, device="cuda")
    g_mscales = torch.full((n_phys * 64,), float("nan"), device="cuda")
    mpages = np.full((B * nb * 64, D), FP8_NAN, np.uint8)
    mscales = np.full(B * nb * 64, np.nan, np.float32)
    g = synth.rng(C4, synth.STREAM_KV)
    for b in range(B):
        sel = o_idx[b][o_idx[b] >= 0]
        codes, scl = synth.e4m3_rows(g, sel.size, D)
        cs = _slot_array(compact[b], sel, 4)
        mpages[cs], mscales[cs] = codes, scl
        ps = torch.from_numpy(_slot_array(bt[b], sel, 4)).cuda()
        g_mpages[ps] = gu.dev_u8(codes)
        g_mscales[ps] = gu.dev_f32(scl)
    tail, n_tail = _tail_table(synth.rng(C4, 17), pos, nb)
    swa_codes, swa_scales = synth.e4m3_rows(synth.rng(C4, synth.STREAM_SWA), n_tail * 256, D)
    q = synth.normal_bf16_bits(synth.rng(C4, synth.STREAM_Q), (B, H, D))
    rows = P + 1
    table = orope.rope_table(rows, R)
    o_out, o_lse = oa.attend(oc.Cache(4, 8, D, R, "fp8", mpages, mscales, compact),
                             oc.Raw("fp8", D, 0, swa_codes, None, swa_scales, tail), SWA, np.arange(B), pos,
                             codecs.load_rows(q, "bf16"), o_idx, 1.0 / math.sqrt(D), True, table)
    cache = csa.Cache(4, 8, D, R, g_mpages, g_bt, g_mscales)
    swa = csa.Raw(D, 0, gu.dev_u8(swa_codes), gu.dev_i32(tail), None, gu.dev_f32(swa_scales))
    g_out, g_lse = _run_attend(cache, swa, g_seq, g_pos, gu.dev_bf16(q), gu.dev_i32(out), max_elig,
                               csa.rope_table(rows, R))
    del cache, g_mpages, g_mscales
    _fresh()
    _check_attend(g_out, g_lse, o_out, o_lse, "fp8", "c4 1M fp8")


def test_c4_1m_fp4_indexer_index():
    """The 1M decode with an MXFP4 indexer cache (the benchmark's fp4 variant): batch 4 at position 2^20, indexer pages
    drawn uniformly from the 200 GB pool sized for fp8 main + fp4 indexer pages; exact-grid e2m1 keys with block
    exponents -2..0 on the sequences' pages, code 6 with the E8M0 NaN exponent everywhere else; top-k sets and scores
    bit-exact."""
    _fresh()
    B, P = 4, 1 << 20
    nb = P // 256 + 1
    per_page = 64 * D + 64 * (D_IDX // 2) + 2 * 64 * 4
    n_phys = POOL_BYTES // per_page
    _log(f"c4 1M fp4 indexer: batch {B}, {nb} blocks per sequence over a pool of {n_phys} pages")
    bt = synth.random_block_table(synth.rng(C4 + 40, synth.STREAM_BT), B, nb, n_phys)
    compact = np.arange(B * nb, dtype=np.int32).reshape(B, nb)
    ids = gu.dev_i32(bt.reshape(-1)).long()
    g = synth.rng(C4 + 40, synth.STREAM_IDX_KV)
    rows = B * nb * 64
    codes = (g.integers(0, 5, size=(rows, D_IDX)) | (g.integers(0, 2, size=(rows, D_IDX)) << 3)).astype(np.uint8)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    del codes
    exps = (127 - g.integers(0, 3, size=(rows, D_IDX // 32))).astype(np.uint8)
    g_ipages = torch.full((n_phys * 64, D_IDX // 2), 0x77, dtype=torch.uint8, device="cuda")
    g_iexps = torch.full((n_phys * 64, D_IDX // 32), 0xFF, dtype=torch.uint8, device="cuda")
    g_ipages.view(n_phys, 64 * D_IDX // 2)[ids] = gu.dev_u8(packed).view(B * nb, 64 * D_IDX // 2)
    g_iexps.view(n_phys, 64 * D_IDX // 32)[ids] = gu.dev_u8(exps).view(B * nb, 64 * D_IDX // 32)
    q_idx = si.grid_bf16(synth.grid_values(synth.rng(C4 + 40, synth.STREAM_QIDX), (B, H_IDX, D_IDX)))
    w = si.grid_weights(synth.rng(C4 + 40, synth.STREAM_HEADW), (B, H_IDX))
    pos = np.full(B, P, np.int64)
    max_elig = paging.num_eligible(P, 4, 8)
    o_idx, o_cnt, o_sc = oi.index_topk(oc.Cache(4, 8, D_IDX, R_IDX, "fp4", packed, exps, compact), np.arange(B), pos,
                                       codecs.load_rows(q_idx, "bf16"), w, oi.WRELU, K_TOP)
    del packed, exps
    icache = csa.Cache(4, 8, D_IDX, R_IDX, g_ipages.view(torch.float4_e2m1fn_x2), gu.dev_i32(bt), g_iexps)
    out, cnt, sc = _run_index(icache, gu.dev_i32(np.arange(B)), gu.dev_i32(pos), max_elig, gu.dev_bf16(q_idx),
                              gu.dev_f32(w), K_TOP)
    del icache, g_ipages, g_iexps
    _fresh()
    assert np.array_equal(cnt, o_cnt)
    assert np.array_equal(out, o_idx)
    m = o_idx >= 0
    assert np.array_equal(sc[m].astype(np.float64), o_sc[m])
    _log("c4 1M fp4 indexer: 4 top-k sets over 262143 entries bit-exact")


# ------------------------------------------------------------------ c128a bf16 dense decode: batch 16, context 64K
C2 = 2


def test_c2_c128a_compress_full_length():
    """c128a compress_insert of two 65537-token sequences in one call: every one of their 512 entries against
    the oracle, counts and slots in full."""
    _fresh()
    Ls = [65537, 65537]
    _log(f"c2 c128a compress: {Ls} tokens")
    g = synth.rng(C2, 50)
    n_blocks = [L // 256 + 1 for L in Ls]
    n_phys = 2 * sum(n_blocks)
    bt = _ragged_table(synth.rng(C2, synth.STREAM_BT), n_blocks, n_phys)
    kv = [synth.normal_bf16_bits(g, (L, D)) for L in Ls]
    lg = [synth.normal_bf16_bits(g, (L, 1, D)) for L in Ls]
    gamma = synth.uniform_f32(g, (D,), 0.5, 1.5)
    rows = max(Ls) + 1
    tail, n_tail = _tail_table(synth.rng(C2, 53), [L - 1 for L in Ls], bt.shape[1])
    cache = csa.Cache(128, 128, D, R, gu.dev_bf16(np.full((n_phys * 2, D), BF16_NAN, np.uint16)), gu.dev_i32(bt))
    state = csa.Raw(D, 1, torch.zeros((n_tail * 256, D), dtype=torch.bfloat16, device="cuda"), gu.dev_i32(tail),
                    torch.zeros((n_tail * 256, 1, D), dtype=torch.bfloat16, device="cuda"))
    max_out = max(Ls) // 128 + 1
    slots = torch.full((2, max_out), -7, dtype=torch.int32, device="cuda")
    counts = torch.full((2,), -7, dtype=torch.int32, device="cuda")
    csa.compress_insert(cache, state, gu.dev_i32([0, 0]), gu.dev_i32([0, Ls[0], Ls[0] + Ls[1]]),
                        gu.dev_bf16(np.concatenate(kv)), gu.dev_bf16(np.concatenate(lg)), gu.dev_f32(gamma), 1e-6,
                        csa.rope_table(rows, R), max(Ls), slots, counts)
    torch.cuda.synchronize()
    gp = gu.host_store(cache.pages)
    slots, counts = slots.cpu().numpy(), counts.cpu().numpy()
    table = orope.rope_table(rows, R)
    written = np.zeros(gp.shape[0], bool)
    for b, L in enumerate(Ls):
        n = paging.num_entries(L, 128, 128)
        assert n == 512 and counts[b] == n
        want = _slot_array(bt[b], range(n), 128)
        assert np.array_equal(slots[b, :n], want) and np.all(slots[b, n:] == -1)
        written[want] = True
        nb = L // 256 + 1
        kvp = np.zeros((nb * 256, D), np.uint16)
        lgp = np.zeros((nb * 256, 1, D), np.uint16)
        kvp[:L], lgp[:L] = kv[b], lg[b]
        ostate = oc.Raw("bf16", D, 1, kvp, lgp, None, np.arange(nb, dtype=np.int32)[None])
        ref = np.stack([codecs.store_row(oc.compress_entry(*oc.window_rows(ostate, ostate.block_table[0], i, 128, 128),
                                                           gamma, 1e-6, table[128 * i], R), "bf16")[0]
                        for i in range(n)])
        _log(f"c2 compress seq {b}: max ulp diff {gu.assert_bf16_rows(gp[want], ref):.0f}")
    assert np.all(gp[~written] == BF16_NAN)


def test_c2_c128a_dense_attend_full_size():
    """Batch 16 at position 65536, dense over all 512 eligible c128a entries plus the 128-row window, 64 heads x 512:
    every query against the oracle. The two entries of block 256 are not eligible yet and hold NaN."""
    _fresh()
    B, P = 16, 65536
    nb = P // 256 + 1
    n_phys = 2 * B * nb
    bt = synth.random_block_table(synth.rng(C2, synth.STREAM_BT), B, nb, n_phys)
    n_elig = paging.num_eligible(P, 128, 128)
    assert n_elig == 512
    pages = np.full((n_phys * 2, D), BF16_NAN, np.uint16)
    g = synth.rng(C2, synth.STREAM_KV)
    for b in range(B):
        pages[_slot_array(bt[b], range(n_elig), 128)] = synth.normal_bf16_bits(g, (n_elig, D))
    pos = np.full(B, P, np.int64)
    tail, n_tail = _tail_table(synth.rng(C2, 17), pos, nb)
    swa_pages = synth.normal_bf16_bits(synth.rng(C2, synth.STREAM_SWA), (n_tail * 256, D))
    q = synth.normal_bf16_bits(synth.rng(C2, synth.STREAM_Q), (B, H, D))
    rows = P + 1
    o_out, o_lse = oa.attend(oc.Cache(128, 128, D, R, "bf16", pages, None, bt),
                             oc.Raw("bf16", D, 0, swa_pages, None, None, tail), SWA, np.arange(B), pos,
                             codecs.load_rows(q, "bf16"), None, 1.0 / math.sqrt(D), True, orope.rope_table(rows, R))
    cache = csa.Cache(128, 128, D, R, gu.dev_bf16(pages), gu.dev_i32(bt))
    swa = csa.Raw(D, 0, gu.dev_bf16(swa_pages), gu.dev_i32(tail))
    g_out, g_lse = _run_attend(cache, swa, gu.dev_i32(np.arange(B)), gu.dev_i32(pos), gu.dev_bf16(q), None, n_elig,
                               csa.rope_table(rows, R))
    _check_attend(g_out, g_lse, o_out, o_lse, "bf16", "c2 c128a dense")


# ------------------------------------------------------------------ prefill chunk: 2 x 2048 tokens at context 262144
C5 = 5
CTX, CHUNK = 262144, 2048


def _c5_sample():
    """Queries the oracle computes: the first and last four of each chunk (every phase of the c4a eligibility
    step) and every 128th one in between."""
    t = sorted(set([0, 1, 2, 3, CHUNK - 4, CHUNK - 3, CHUNK - 2, CHUNK - 1] + list(range(64, CHUNK, 128))))
    return np.array([b * CHUNK + i for b in range(2) for i in t])


class _C5:
    """Shared block table (1032 logical blocks per sequence), raw pages for blocks 1023..1031 (the compressor
    state before the chunk and the sliding window), queries at every chunk position."""

    def __init__(self):
        self.B = 2
        self.nb = (CTX + CHUNK - 1) // 256 + 1
        self.n_phys = self.B * self.nb + 40
        self.bt = synth.random_block_table(synth.rng(C5, synth.STREAM_BT), self.B, self.nb, self.n_phys)
        self.tail, self.n_tail = _tail_table(synth.rng(C5, 17), [CTX] * self.B, self.nb, -1, (CHUNK - 1) // 256)
        self.q_pos = np.concatenate([np.arange(CTX, CTX + CHUNK)] * self.B).astype(np.int64)
        self.q_seq = np.repeat(np.arange(self.B), CHUNK)
        self.rows = CTX + CHUNK + 1
        self.table = orope.rope_table(self.rows, R)
        self.g_bt, self.g_tail = gu.dev_i32(self.bt), gu.dev_i32(self.tail)
        self.g_seq, self.g_pos = gu.dev_i32(self.q_seq), gu.dev_i32(self.q_pos)
        self.g_rope = csa.rope_table(self.rows, R)

    def compress_chunk(self, ratio, dim, seed, pre_pages):
        """compress_insert of the chunk on both sides from caches holding `pre_pages`; checks counts, slots, the
        new entries (one bf16 ulp) and that nothing else changed. Returns the new entries' slots per sequence."""
        window = 8 if ratio == 4 else 128
        roles = window // ratio
        g = synth.rng(C5, seed)
        pre = np.zeros((self.n_tail * 256, dim), np.uint16)
        pre_lg = np.zeros((self.n_tail * 256, roles, dim), np.uint16)
        for b in range(self.B):  # raw rows of block 1023: the positions just before the chunk
            r0 = int(self.tail[b, CTX // 256 - 1]) * 256
            pre[r0:r0 + 256] = synth.normal_bf16_bits(g, (256, dim))
            pre_lg[r0:r0 + 256] = synth.normal_bf16_bits(g, (256, roles, dim))
        kv = synth.normal_bf16_bits(g, (self.B * CHUNK, dim))
        lg = synth.normal_bf16_bits(g, (self.B * CHUNK, roles, dim))
        gamma = synth.uniform_f32(g, (dim,), 0.5, 1.5)
        cu = np.arange(self.B + 1, dtype=np.int32) * CHUNK
        start = np.full(self.B, CTX, np.int32)
        max_out = CHUNK // ratio
        ocache = oc.Cache(ratio, window, dim, R, "bf16", pre_pages.copy(), None, self.bt)
        ostate = oc.Raw("bf16", dim, roles, pre.copy(), pre_lg.copy(), None, self.tail)
        o_slots, o_counts = oc.compress_insert(ocache, ostate, start, cu, kv, lg, gamma, 1e-6, self.table, max_out)
        cache = csa.Cache(ratio, window, dim, R, gu.dev_bf16(pre_pages), self.g_bt)
        state = csa.Raw(dim, roles, gu.dev_bf16(pre), self.g_tail, gu.dev_bf16(pre_lg))
        slots = torch.full((self.B, max_out), -7, dtype=torch.int32, device="cuda")
        counts = torch.full((self.B,), -7, dtype=torch.int32, device="cuda")
        csa.compress_insert(cache, state, gu.dev_i32(start), gu.dev_i32(cu), gu.dev_bf16(kv), gu.dev_bf16(lg),
                            gu.dev_f32(gamma), 1e-6, self.g_rope, CHUNK, slots, counts)
        torch.cuda.synchronize()
        slots, counts = slots.cpu().numpy(), counts.cpu().numpy()
        assert np.array_equal(counts, o_counts) and np.all(counts == CHUNK // ratio)
        assert np.array_equal(slots, o_slots)
        gp = gu.host_store(cache.pages)
        new = o_slots.reshape(-1)
        ulp = gu.assert_bf16_rows(gp[new], ocache.pages[new])
        old = np.ones(gp.shape[0], bool)
        old[new] = False
        assert np.array_equal(gp[old], pre_pages[old]), "compress_insert changed a row outside the new entries"
        assert np.array_equal(gu.host_store(state.kv_pages), ostate.kv_pages)
        assert np.array_equal(gu.host_store(state.logit_pages), ostate.logit_pages)
        _log(f"c5 compress ratio {ratio} dim {dim}: {counts.tolist()} new entries, max ulp diff {ulp:.0f}")
        return o_slots


def test_c5_prefill_chunk_c4a():
    """c4a prefill chunk: compress_insert of 2 x 2048 tokens into the main and the indexer cache, then index +
    top-512 for all 4096 queries (sampled ones bit-exact against the oracle, all checked for count, order and
    range) and causal top-k + window attention for all 4096 (sampled ones within 2e-3, all finite)."""
    _fresh()
    c = _C5()
    n_pre = paging.num_eligible(CTX - 1, 4, 8)  # entries complete before the chunk
    max_elig = paging.num_eligible(CTX + CHUNK - 1, 4, 8)
    _log(f"c5 c4a: batch 2, {n_pre} entries before the chunk, up to {max_elig} eligible, 4096 queries")
    # pre-chunk caches: indexer exact-grid rows, main N(0,1) rows, NaN on every slot no entry uses yet
    ipages = np.full((c.n_phys * 64, D_IDX), BF16_NAN, np.uint16)
    mpages = np.full((c.n_phys * 64, D), BF16_NAN, np.uint16)
    gi, gm = synth.rng(C5, synth.STREAM_IDX_KV), synth.rng(C5, synth.STREAM_KV)
    for b in range(c.B):
        s = _slot_array(c.bt[b], range(n_pre), 4)
        ipages[s] = si.grid_bf16(synth.grid_values(gi, (n_pre, D_IDX)))
        mpages[s] = synth.normal_bf16_bits(gm, (n_pre, D))
    new_m = c.compress_chunk(4, D, 60, mpages)
    new_i = c.compress_chunk(4, D_IDX, 61, ipages)
    # stage inputs for index and attention: the new entries' slots get fresh synthetic rows on both sides
    for b in range(c.B):
        ipages[new_i[b]] = si.grid_bf16(synth.grid_values(gi, (new_i.shape[1], D_IDX)))
        mpages[new_m[b]] = synth.normal_bf16_bits(gm, (new_m.shape[1], D))
    n_q = c.q_pos.size
    q_idx = si.grid_bf16(synth.grid_values(synth.rng(C5, synth.STREAM_QIDX), (n_q, H_IDX, D_IDX)))
    w = si.grid_weights(synth.rng(C5, synth.STREAM_HEADW), (n_q, H_IDX))
    icache = csa.Cache(4, 8, D_IDX, R_IDX, gu.dev_bf16(ipages), c.g_bt)
    out, cnt, sc = _run_index(icache, c.g_seq, c.g_pos, max_elig, gu.dev_bf16(q_idx), gu.dev_f32(w), K_TOP)
    del icache
    _fresh()
    _topk_properties(out, cnt, c.q_pos, 4, 8, K_TOP)
    smp = _c5_sample()
    o_idx, o_cnt, o_sc = oi.index_topk(oc.Cache(4, 8, D_IDX, R_IDX, "bf16", ipages, None, c.bt), c.q_seq[smp],
                                       c.q_pos[smp], codecs.load_rows(q_idx[smp], "bf16"), w[smp], oi.WRELU, K_TOP)
    assert np.array_equal(cnt[smp], o_cnt)
    assert np.array_equal(out[smp], o_idx)
    m = o_idx >= 0
    assert np.array_equal(sc[smp][m].astype(np.float64), o_sc[m])
    _log(f"c5 c4a: {smp.size} sampled top-k sets bit-exact, all {n_q} well formed")

    swa_pages = synth.normal_bf16_bits(synth.rng(C5, synth.STREAM_SWA), (c.n_tail * 256, D))
    q = synth.normal_bf16_bits(synth.rng(C5, synth.STREAM_Q), (n_q, H, D))
    cache = csa.Cache(4, 8, D, R, gu.dev_bf16(mpages), c.g_bt)
    swa = csa.Raw(D, 0, gu.dev_bf16(swa_pages), c.g_tail)
    g_out, g_lse = _run_attend(cache, swa, c.g_seq, c.g_pos, gu.dev_bf16(q), gu.dev_i32(out), max_elig, c.g_rope)
    del cache
    assert np.all(np.isfinite(g_out))
    o_out, o_lse = oa.attend(oc.Cache(4, 8, D, R, "bf16", mpages, None, c.bt),
                             oc.Raw("bf16", D, 0, swa_pages, None, None, c.tail), SWA, c.q_seq[smp], c.q_pos[smp],
                             codecs.load_rows(q[smp], "bf16"), o_idx, 1.0 / math.sqrt(D), True, c.table)
    _check_attend(g_out[smp], g_lse[smp], o_out, o_lse, "bf16", "c5 c4a prefill")


def test_c5_prefill_chunk_c128a():
    """c128a layer on the same block table: compress_insert of the chunk (16 new entries per sequence), then dense
    attention over the 2048-2064 eligible entries plus the window for all 4096 queries (sampled ones within 2e-3)."""
    _fresh()
    c = _C5()
    n_pre = paging.num_eligible(CTX - 1, 128, 128)
    max_elig = paging.num_eligible(CTX + CHUNK - 1, 128, 128)
    _log(f"c5 c128a: {n_pre} entries before the chunk, up to {max_elig} eligible, 4096 queries")
    pages = np.full((c.n_phys * 2, D), BF16_NAN, np.uint16)
    g = synth.rng(C5, 70)
    for b in range(c.B):
        pages[_slot_array(c.bt[b], range(n_pre), 128)] = synth.normal_bf16_bits(g, (n_pre, D))
    new = c.compress_chunk(128, D, 71, pages)
    for b in range(c.B):
        pages[new[b]] = synth.normal_bf16_bits(g, (new.shape[1], D))
    n_q = c.q_pos.size
    swa_pages = synth.normal_bf16_bits(synth.rng(C5, synth.STREAM_SWA), (c.n_tail * 256, D))
    q = synth.normal_bf16_bits(synth.rng(C5, synth.STREAM_Q), (n_q, H, D))
    cache = csa.Cache(128, 128, D, R, gu.dev_bf16(pages), c.g_bt)
    swa = csa.Raw(D, 0, gu.dev_bf16(swa_pages), c.g_tail)
    g_out, g_lse = _run_attend(cache, swa, c.g_seq, c.g_pos, gu.dev_bf16(q), None, max_elig, c.g_rope)
    assert np.all(np.isfinite(g_out))
    smp = _c5_sample()
    o_out, o_lse = oa.attend(oc.Cache(128, 128, D, R, "bf16", pages, None, c.bt),
                             oc.Raw("bf16", D, 0, swa_pages, None, None, c.tail), SWA, c.q_seq[smp], c.q_pos[smp],
                             codecs.load_rows(q[smp], "bf16"), None, 1.0 / math.sqrt(D), True, c.table)
    _check_attend(g_out[smp], g_lse[smp], o_out, o_lse, "bf16", "c5 c128a prefill")
