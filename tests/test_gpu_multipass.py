"""GPU parity of attention with more key rows per workgroup than its row table holds (several passes).

Dense c128a attention keeps every eligible entry ([P2] "二、注意力機制為什么這么麻煩", [P3] "注意力计算剪枝":
c128a layers attend densely up to 1M tokens, 8191 entries at 2^20). The attention workgroups resolve the page
rows of at most 3072 keys at a time; a query (or a key split of one) with more keys walks them in passes.
Cases:
* 512 prefill queries of two sequences past 2^19 tokens (4200-4700 keys each): one key split per query, two
  passes, 64 heads in one workgroup;
* 32 heads near 2^20 (the 16-head-group kernel, no key splits): three passes, bf16 and fp8;
* 256 queries near 2^20 with 64 heads: two key splits per query of 4160 keys each (two passes per split, merged
  by the split-combine step), bf16 and fp8;
* a decode batch of 4 at position 2^20 (8192 eligible entries), 64 heads.
Entries that are not eligible for any query of a sequence hold NaN codes, so a gather beyond the eligible range
shows up. The oracle computes a sample of the queries one by one (first, last and a seeded draw); every query's
output is checked finite and its top-level shape right.
"""
import math

import numpy as np
import pytest
import torch

import long_context_compressed_compress_amd as csa
import synth
from oracle import attend as oa, codecs, compress as oc, paging, rope as orope
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-3, "fp8": 5e-2}
D, R, SWA = 512, 64, 128
NAN = {"bf16": 0x7FC0, "fp8": 0x7F}


def _log(msg):
    print(msg, flush=True)


def _queries(spec):
    """spec: list of (sequence, first position, count) -> (q_seq, q_pos) of consecutive positions."""
    seqs, pos = [], []
    for s, p0, n in spec:
        seqs += [s] * n
        pos += list(range(p0, p0 + n))
    return np.array(seqs, np.int32), np.array(pos, np.int64)


def _window_table(g, q_seq, q_pos, B, bt_stride):
    """Table mapping only the blocks the windows of the queries touch, onto a pool of their own."""
    need = []
    for b in range(B):
        ps = q_pos[q_seq == b]
        if len(ps):
            lo, hi = max(0, int(ps.min()) - SWA + 1) // 256, int(ps.max()) // 256
            need.append((b, lo, hi))
    n = sum(hi - lo + 1 for _, lo, hi in need)
    ids = g.permutation(n).astype(np.int32)
    bt = np.full((B, bt_stride), -1, np.int32)
    o = 0
    for b, lo, hi in need:
        bt[b, lo:hi + 1] = ids[o:o + hi - lo + 1]
        o += hi - lo + 1
    return bt, n


CASES = [
    ("512 queries, one split, two passes", 64, "bf16", [(0, 600000, 256), (1, 540001, 256)]),
    ("32 heads near 2^20, three passes", 32, "bf16",
     [(0, 1048576, 1), (0, 1048447, 1), (1, 1048575, 1), (1, 700000, 1), (2, 524287, 1), (2, 900003, 1)]),
    ("32 heads near 2^20, three passes", 32, "fp8",
     [(0, 1048576, 1), (0, 1048447, 1), (1, 1048575, 1), (1, 700000, 1), (2, 524287, 1), (2, 900003, 1)]),
    ("256 queries near 2^20, two splits of two passes", 64, "bf16", [(0, 1048449, 128), (1, 1048321, 128)]),
    ("256 queries near 2^20, two splits of two passes", 64, "fp8", [(0, 1048449, 128), (1, 1048321, 128)]),
    ("decode batch 4 at 2^20", 64, "bf16", [(b, 1048576, 1) for b in range(4)]),
]


@pytest.mark.parametrize("label,heads,dtype,spec", CASES)
def test_dense_c128a_multipass(label, heads, dtype, spec):
    cfg = 300 + heads + len(spec)
    q_seq, q_pos = _queries(spec)
    n_q = len(q_pos)
    B = int(q_seq.max()) + 1
    p_max = [int(q_pos[q_seq == b].max()) for b in range(B)]
    nb = max(p_max) // 256 + 1
    n_phys = B * nb + 3
    _log(f"multipass: {label} heads={heads} dtype={dtype} n_q={n_q} max keys "
         f"{max(paging.num_eligible(int(p), 128, 128) for p in q_pos) + SWA}")
    bt = synth.random_block_table(synth.rng(cfg, synth.STREAM_BT), B, nb, n_phys)
    rows = n_phys * 2
    g = synth.rng(cfg, synth.STREAM_KV)
    if dtype == "bf16":
        pages, scales = synth.normal_bf16_bits(g, (rows, D)), None
    else:
        pages, scales = synth.e4m3_rows(g, rows, D)
    for b in range(B):  # entries no query of the sequence may read
        n_ok = paging.num_eligible(p_max[b], 128, 128)
        bad = [paging.entry_slot(bt[b], i, 128) for i in range(n_ok, nb * 2)]
        pages[bad] = NAN[dtype]
    wbt, n_w = _window_table(synth.rng(cfg, 17), q_seq, q_pos, B, nb)
    gw = synth.rng(cfg, synth.STREAM_SWA)
    if dtype == "bf16":
        wpages, wscales = synth.normal_bf16_bits(gw, (n_w * 256, D)), None
    else:
        wpages, wscales = synth.e4m3_rows(gw, n_w * 256, D)
    q = synth.normal_bf16_bits(synth.rng(cfg, synth.STREAM_Q), (n_q, heads, D))
    scale = 1.0 / math.sqrt(D)
    table_rows = int(q_pos.max()) + 1
    max_elig = max(paging.num_eligible(int(p), 128, 128) for p in q_pos)
    # GPU: every query in one launch
    cache = csa.Cache(128, 128, D, R, gu.dev_store(pages, dtype), gu.dev_i32(bt),
                      gu.dev_f32(scales) if scales is not None else None)
    swa = csa.Raw(D, 0, gu.dev_store(wpages, dtype), gu.dev_i32(wbt), None,
                  gu.dev_f32(wscales) if wscales is not None else None)
    need = csa.attend_workspace(n_q, heads, D, max_elig + SWA)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    out = torch.full((n_q, heads, D), -7.0, device="cuda")
    lse = torch.full((n_q, heads), -7.0, device="cuda")
    csa.attend(cache, swa, SWA, gu.dev_i32(q_seq), gu.dev_i32(q_pos), gu.dev_bf16(q), None, max_elig, scale, True,
               csa.rope_table(table_rows, R), out, lse, workspace=ws)
    torch.cuda.synchronize()
    g_out, g_lse = out.cpu().numpy(), lse.cpu().numpy()
    assert np.all(np.isfinite(g_out)) and np.all(np.isfinite(g_lse))
    # oracle: a sample of the queries
    gs = synth.rng(cfg, 31)
    sample = sorted(set([0, n_q - 1] + list(gs.choice(n_q, size=min(n_q, 8), replace=False))))
    table = orope.rope_table(table_rows, R)
    o_out, o_lse = oa.attend(oc.Cache(128, 128, D, R, dtype, pages, scales, bt),
                             oc.Raw(dtype, D, 0, wpages, None, wscales, wbt), SWA, q_seq[sample], q_pos[sample],
                             codecs.load_rows(q[sample], "bf16"), None, scale, True, table)
    err = gu.rowwise_rel_err(g_out[sample], o_out)
    _log(f"{label}: rowwise rel err {err:.3e} over {len(sample)} sampled queries")
    assert err <= TOL[dtype]
    assert np.allclose(g_lse[sample], o_lse, rtol=0, atol=1e-4)
