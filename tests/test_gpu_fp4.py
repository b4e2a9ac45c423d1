"""MXFP4 indexer cache (reading R25) on the GPU against the oracle.

* compress_insert into an fp4 cache: E8M0 exponents and e2m1 codes equal the oracle's wherever the fp32
  row is not within rounding distance of a decision (a power-of-two block amax, an e2m1 midpoint); every
  dequantised element is within one e2m1 step of the oracle's.
* index score + select over fp4 pages (few queries: the per-query kernel; >= 256 queries: the kernel whose
  workgroups share each page among 8 queries): exact-grid keys (e2m1 codes with block exponents -2..0), queries
  and weights make every score exact in fp32, so top-k sets and scores are bit-exact.
* compress_insert_pair with an fp8 main cache and an fp4 indexer cache equals the two separate calls.
"""
import numpy as np
import pytest
import torch

import long_context_compressed_compress_amd as csa
import synth
from oracle import codecs, compress as oc, index as oi, paging, rope as orope
import gpu_util as gu
import stage_inputs as si

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def _fp4_tensors(rows, dim, dev="cuda"):
    pages = torch.full((rows, dim // 2), 0xA5, dtype=torch.uint8, device=dev)  # canary codes
    scales = torch.full((rows, dim // 32), 0xA5, dtype=torch.uint8, device=dev)
    return pages, scales


def _cache(ratio, dim, rope, pages_u8, scales_u8, bt):
    return csa.Cache(ratio, 8 if ratio == 4 else 128, dim, rope, pages_u8.view(torch.float4_e2m1fn_x2), bt, scales_u8)


# gap from each e2m1 magnitude to the next larger one (6 has none)
_E2M1_UP = {0.0: 0.5, 0.5: 0.5, 1.0: 0.5, 1.5: 0.5, 2.0: 1.0, 3.0: 1.0, 4.0: 2.0}


def _check_fp4_elements(y, gv, ov, ge, oe, row_slack=2.0 ** -16):
    """Each GPU element against the oracle's at its own magnitude.

    y: the oracle's fp32 rows before rounding; gv / ov: dequantised GPU / oracle rows; ge / oe: E8M0 bytes.
    In blocks with the same exponent 2^X, an element may differ only if (a) the two values are neighbours on the
    e2m1 grid (|gv - ov| / 2^X is the gap from the smaller magnitude to the next, signs agreeing or one of them
    zero) and (b) y lies within the fp32 compute error eta = row_slack * max|row| of their midpoint, i.e. both are
    correct roundings of a value the two sides compute differently. Blocks whose exponents differ (a block amax
    within rounding of a power of two) may differ by one step of the larger grid (2 * 2^max(X))."""
    n, D = y.shape
    Xo = np.repeat(oe.astype(int) - 127, 32, axis=-1)
    Xg = np.repeat(ge.astype(int) - 127, 32, axis=-1)
    s = np.ldexp(1.0, Xo)
    eta = row_slack * np.abs(y).max(axis=1, keepdims=True) + 2.0 ** -22 * np.abs(y)
    diff = gv != ov
    same = Xo == Xg
    bad = []
    for r, c in zip(*np.nonzero(diff & same)):
        a, b = abs(ov[r, c]) / s[r, c], abs(gv[r, c]) / s[r, c]
        lo, hi = min(a, b), max(a, b)
        signs_ok = (ov[r, c] * gv[r, c] >= 0)
        neighbours = lo in _E2M1_UP and hi - lo == _E2M1_UP[lo] and signs_ok
        at_mid = abs(y[r, c] - 0.5 * (ov[r, c] + gv[r, c])) <= eta[r, c]
        if not (neighbours and at_mid):
            bad.append((r, c, y[r, c], ov[r, c], gv[r, c]))
    assert not bad, f"fp4 elements differ without a rounding tie between them: {bad[:4]}"
    other = diff & ~same
    if other.any():
        big = np.ldexp(2.0, np.maximum(Xo, Xg))
        assert np.all(np.abs(gv - ov)[other] <= big[other]), "fp4 values of a re-scaled block differ by > one step"
    _log(f"fp4 elements: {int((diff & same).sum())} neighbour-at-midpoint differences, "
         f"{int(other.sum())} in re-scaled blocks, of {diff.size}")


@pytest.mark.parametrize("ratio,dim,rope,ind,lens,zero_seq", [
    (4, 128, 64, "bf16", [700, 259, 303], None),
    (4, 32, 16, "f32", [517, 6], None),
    (4, 128, 64, "f32", [300], None),
    (128, 64, 32, "bf16", [900, 255], None),
    (4, 512, 64, "bf16", [400, 129], None),
    (4, 128, 64, "bf16", [300, 260], 1),   # sequence 1's raw rows are all zero: every block of its entries is zero
])
def test_compress_insert_fp4_parity(ratio, dim, rope, ind, lens, zero_seq):
    _log(f"fp4 compress ratio={ratio} dim={dim} rope={rope} in={ind} lens={lens} zero_seq={zero_seq}")
    seed = 500 + dim + ratio
    window = 8 if ratio == 4 else 128
    roles = window // ratio
    B = len(lens)
    nb = max(lens) // 256 + 1
    n_phys = B * nb + 2
    bt = synth.random_block_table(synth.rng(seed, synth.STREAM_BT), B, nb, n_phys)
    g = synth.rng(seed, synth.STREAM_KV)
    n = sum(lens)
    kv = synth.normal_f32(g, (n, dim))
    lg = synth.normal_f32(g, (n, roles, dim))
    gamma = (1.0 + 0.25 * g.standard_normal(dim)).astype(np.float32)
    if zero_seq is not None:
        c0 = sum(lens[:zero_seq])
        kv[c0:c0 + lens[zero_seq]] = 0.0
    if ind == "bf16":
        kv_s, lg_s = codecs.f64_to_bf16(kv), codecs.f64_to_bf16(lg)
    else:
        kv_s, lg_s = kv, lg
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    start = np.zeros(B, np.int32)
    rows = n_phys * (256 // ratio)
    table = csa.rope_table(max(lens) + 2, rope)
    # oracle: the same inputs into an fp4 cache and into an fp32 cache (the unrounded rows)
    st = lambda: oc.Raw(ind, dim, roles, np.zeros((n_phys * 256, dim), kv_s.dtype),
                        np.zeros((n_phys * 256, roles, dim), lg_s.dtype), None, bt.copy())
    o4 = oc.Cache(ratio, window, dim, rope, "fp4", np.full((rows, dim // 2), 0xA5, np.uint8),
                  np.full((rows, dim // 32), 0xA5, np.uint8), bt.copy())
    o32 = oc.Cache(ratio, window, dim, rope, "f32", np.zeros((rows, dim), np.float32), None, bt.copy())
    tab = orope.rope_table(max(lens) + 2, rope)
    for c in (o4, o32):
        oc.compress_insert(c, st(), start, cu, kv_s, lg_s, gamma, 1e-6, tab, 0)
    # GPU
    pages, scales = _fp4_tensors(rows, dim)
    cache = _cache(ratio, dim, rope, pages, scales, gu.dev_i32(bt))
    dev_in = gu.dev_bf16 if ind == "bf16" else gu.dev_f32
    state = csa.Raw(dim, roles, dev_in(np.zeros((n_phys * 256, dim), kv_s.dtype)), gu.dev_i32(bt),
                    dev_in(np.zeros((n_phys * 256, roles, dim), lg_s.dtype)))
    csa.compress_insert(cache, state, gu.dev_i32(start), gu.dev_i32(cu), dev_in(kv_s), dev_in(lg_s),
                        gu.dev_f32(gamma), 1e-6, table, max(lens))
    torch.cuda.synchronize()
    gp, gs = pages.cpu().numpy(), scales.cpu().numpy()
    written = np.zeros(rows, bool)
    for b, L in enumerate(lens):
        for i in range(paging.num_entries(L, ratio, window)):
            written[paging.entry_slot(bt[b], i, ratio)] = True
    assert written.any()
    assert np.all(gp[~written] == 0xA5) and np.all(gs[~written] == 0xA5), "unwritten slot changed"
    y = o32.pages[written].astype(np.float64)             # fp32 rows before the fp4 rounding
    ge, oe = gs[written].astype(int), o4.scales[written].astype(int)
    # exponents: equal unless the block amax is within fp32 rounding of a power of two
    amax = np.abs(y.reshape(len(y), -1, 32)).max(-1)
    frac = amax / np.ldexp(1.0, np.floor(np.log2(np.maximum(amax, 1e-300))).astype(int))
    near_pow2 = (frac < 1 + 1e-5) | (frac > 2 - 1e-5)
    assert np.all((ge == oe) | near_pow2), "E8M0 block exponents differ"
    gv = codecs.mxfp4_to_f64(gp[written], gs[written])
    ov = codecs.mxfp4_to_f64(o4.pages[written], o4.scales[written])
    _check_fp4_elements(y, gv, ov, ge, oe)
    if zero_seq is not None:
        for i in range(paging.num_entries(lens[zero_seq], ratio, window)):
            slot = paging.entry_slot(bt[zero_seq], i, ratio)
            assert np.all(gp[slot] == 0) and np.all(gs[slot] == 127), f"zero entry {i}"
    same = np.mean(gp[written] == o4.pages[written])
    _log(f"fp4 identical code bytes {same:.5f}, identical exponents {np.mean(ge == oe):.5f}")
    assert same > 0.99


def _grid_fp4_cache(cfg, positions, spare=3):
    """fp4 pages whose entries are exact-grid values: e2m1 codes with magnitude <= 2 and exponents X in -2..0,
    so every key value is a multiple of 2^-3 of at most 2."""
    g = synth.rng(cfg, synth.STREAM_IDX_KV)
    B = len(positions)
    n_blocks = max(positions) // 256 + 1
    n_phys = B * n_blocks + spare
    bt = synth.random_block_table(synth.rng(cfg, synth.STREAM_BT), B, n_blocks, n_phys)
    rows = n_phys * 64
    mags = g.integers(0, 5, size=(rows, 128))          # codes 0..4: 0, 0.5, 1, 1.5, 2
    sign = g.integers(0, 2, size=(rows, 128)) << 3
    codes = (mags | sign).astype(np.uint8)
    pages = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    scales = (127 - g.integers(0, 3, size=(rows, 4))).astype(np.uint8)
    return si.PagedCache(4, 8, 128, "fp4", bt, pages, scales)


@pytest.mark.parametrize("heads,k,positions", [
    (64, 512, [20000, 131, 6, 2060, 2063, 8000]),
    (16, 64, [5000, 300]),
    (64, 2048, [12000, 8203]),
    (32, 512, [300000, 70000]),                       # > 2^16 entries: the mark-pass select
    (64, 512, [300 + 13 * i for i in range(270)]),   # many queries: pages shared through LDS by 8 queries
    (16, 100, [5000 - 17 * i for i in range(260)]),  # the same with one 16-head tile
])
def test_index_topk_fp4_exact_grid_bit_exact(heads, k, positions):
    _log(f"fp4 index grid H={heads} k={k} n_q={len(positions)} max_pos={max(positions)}")
    cfg = 71 + k + heads
    pc = _grid_fp4_cache(cfg, positions)
    qv = synth.grid_values(synth.rng(cfg, synth.STREAM_QIDX), (len(positions), heads, 128))
    w = si.grid_weights(synth.rng(cfg, synth.STREAM_HEADW), (len(positions), heads))
    q_store = si.grid_bf16(qv)
    o_idx, o_cnt, o_sc = oi.index_topk(pc.oracle(), np.arange(len(positions)), positions,
                                       codecs.load_rows(q_store, "bf16"), w, oi.WRELU, k)
    B = len(positions)
    max_elig = max(paging.num_eligible(p, 4, 8) for p in positions)
    out = torch.full((B, k), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    sc = torch.zeros((B, k), dtype=torch.float32, device="cuda")
    cache = _cache(4, 128, 0, gu.dev_u8(pc.pages), gu.dev_u8(pc.scales), gu.dev_i32(pc.bt))
    csa.index_topk(cache, gu.dev_i32(np.arange(B)), gu.dev_i32(positions), max_elig, gu.dev_bf16(q_store),
                   gu.dev_f32(w), csa.SCORE_WRELU, k, out, cnt, sc)
    torch.cuda.synchronize()
    out, cnt, sc = out.cpu().numpy(), cnt.cpu().numpy(), sc.cpu().numpy()
    assert np.array_equal(cnt, o_cnt)
    assert np.array_equal(out, o_idx)
    m = o_idx >= 0
    assert np.array_equal(sc[m].astype(np.float64), o_sc[m])
    assert np.all(np.isnan(sc[~m]))


def test_compress_insert_pair_fp8_main_fp4_indexer():
    """The fused pair launch (fp8 main cache of dim 512, fp4 indexer cache of dim 128) writes exactly what
    the two separate calls write."""
    lens = [700, 259, 303]
    _log(f"pair fp8 + fp4 lens={lens}")
    B = len(lens)
    nb = max(lens) // 256 + 1
    n_phys = B * nb + 2
    bt = gu.dev_i32(synth.random_block_table(synth.rng(91, synth.STREAM_BT), B, nb, n_phys))
    g = torch.Generator(device="cuda")
    g.manual_seed(91)
    n = sum(lens)
    bf = torch.bfloat16
    r = lambda *s: torch.randn(s, generator=g, device="cuda", dtype=bf)
    ins = {d: (r(n, d), r(n, 2, d), torch.rand(d, generator=g, device="cuda") + 0.5) for d in (512, 128)}
    cu = gu.dev_i32(np.concatenate([[0], np.cumsum(lens)]))
    start = torch.zeros(B, dtype=torch.int32, device="cuda")
    table = csa.rope_table(max(lens) + 2, 64)
    res = []
    for fused in (True, False):
        main = csa.Cache(4, 8, 512, 64, torch.zeros((n_phys * 64, 512), dtype=torch.uint8, device="cuda"), bt,
                         torch.zeros(n_phys * 64, device="cuda"))
        p4, s4 = _fp4_tensors(n_phys * 64, 128)
        idx = _cache(4, 128, 64, p4, s4, bt)
        z = lambda d: csa.Raw(d, 2, torch.zeros((n_phys * 256, d), dtype=bf, device="cuda"), bt,
                              torch.zeros((n_phys * 256, 2, d), dtype=bf, device="cuda"))
        sm, si_ = z(512), z(128)
        if fused:
            csa.compress_insert_pair(main, sm, *ins[512][:2], ins[512][2], table, idx, si_, *ins[128][:2],
                                     ins[128][2], table, start, cu, 1e-6, max(lens))
        else:
            csa.compress_insert(main, sm, start, cu, *ins[512][:2], ins[512][2], 1e-6, table, max(lens))
            csa.compress_insert(idx, si_, start, cu, *ins[128][:2], ins[128][2], 1e-6, table, max(lens))
        torch.cuda.synchronize()
        res.append([main.pages, main.scales, p4, s4])
    for a, b in zip(*res):
        assert torch.equal(a, b)
    assert int((res[0][3] != 0xA5).sum()) > 0
