"""GPU parity of every stage against the CPU oracle, through the C ABI (needs an MI355X).

Each stage is fed synthetic inputs from `synth` that both sides read identically (caches written straight
into pages, top-k lists drawn at random); the chain test runs the oracle end to end from the raw tokens.
No value produced by the GPU path is ever handed to the oracle.
Bars: integer outputs (counts, slots, top-k sets on exact-grid inputs) bit-exact; cache values within one
storage ulp (plus a 2^-16 row-scale slack for fp32 cancellation); attention outputs within the normwise
bounds fp32 1e-5, bf16 2e-3, fp8 5e-2 (max over rows of max|diff| / max|ref|).
"""
import numpy as np
import pytest
import torch

import long_context_compressed_compress_amd as csa
from oracle import attend as oa, codecs, compress as oc, index as oi, paging, rope as orope
from tests import gpu_util as gu
from tests import stage_inputs as si
from tests.chain import Step, StepConfig

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-3, "fp8": 5e-2}


def _log(msg):
    print(msg, flush=True)


# ------------------------------------------------------------------ RoPE table
def test_rope_table_matches_oracle():
    _log("rope_table rows=1048577 R=64")
    g = csa.rope_table((1 << 20) + 1, 64).cpu().numpy()
    o = orope.rope_table((1 << 20) + 1, 64)
    diff = np.abs(g.astype(np.float64) - o.astype(np.float64))
    _log(f"rope table: exact {np.mean(g == o):.6f}, max abs diff {diff.max():.3e}")
    assert diff.max() <= 2.0 ** -24
    assert np.mean(g == o) > 0.999


# ------------------------------------------------------------------ compress_insert
COMPRESS_CASES = [
    # ratio, dim, rope, in dtype, cache dtype, lens
    (4, 128, 64, "f32", "f32", [1024]),
    (4, 32, 16, "f32", "f32", [700, 6, 517]),
    (4, 512, 64, "bf16", "bf16", [700, 517, 300]),
    (4, 512, 64, "bf16", "fp8", [700, 259, 300]),
    (4, 128, 64, "bf16", "bf16", [643, 11]),
    (4, 128, 64, "bf16", "fp8", [643, 511]),
    (128, 512, 64, "bf16", "bf16", [1100, 127, 640]),
    (128, 512, 64, "bf16", "fp8", [1100, 383]),
    (128, 64, 32, "f32", "f32", [900, 255]),
    (4, 256, 0, "bf16", "bf16", [300]),
]


@pytest.mark.parametrize("ratio,dim,rope,ind,cd,lens", COMPRESS_CASES)
def test_compress_insert_parity(ratio, dim, rope, ind, cd, lens):
    _log(f"compress ratio={ratio} dim={dim} rope={rope} in={ind} cache={cd} lens={lens}")
    cfg = StepConfig(seed=100 + dim + ratio, ratio=ratio, lens=lens, dim=dim, rope_dims=rope, heads=16 if cd != "f32" else 4,
                     cache_dtype=cd, in_dtype=ind, indexer=False, random_gamma=True)
    st = Step(cfg)
    st.run_gpu()
    st.run_oracle_compress()
    for (gs, gc), (os_, oc_) in ((st.g_prefill, st.o_prefill), (st.g_decode, st.o_decode)):
        gs, gc = gs.cpu().numpy(), gc.cpu().numpy()
        assert np.array_equal(gc, oc_)
        assert np.array_equal(gs[:, : os_.shape[1]], os_[:, : gs.shape[1]])
    assert np.array_equal(gu.host_store(st.g_state.kv_pages), st.o_state.kv_pages)
    assert np.array_equal(gu.host_store(st.g_state.logit_pages), st.o_state.logit_pages)
    gp = gu.host_store(st.g_cache.pages)
    op = st.o_cache.pages
    written = np.zeros(gp.shape[0], bool)
    for b, L in enumerate(lens):
        for i in range(paging.num_entries(L + 1, ratio, st.window)):
            written[paging.entry_slot(st.bt[b], i, ratio)] = True
    canary = gu.canary((1, dim), cd)[0]
    assert all(np.array_equal(gp[r], canary, equal_nan=True) for r in np.nonzero(~written)[0]), "unwritten slot changed"
    if cd == "f32":
        err = gu.rowwise_rel_err(gp[written], op[written])
        _log(f"f32 cache rowwise err {err:.3e}")
        assert err <= 1e-5
    elif cd == "bf16":
        _log(f"bf16 cache max ulp diff {gu.assert_bf16_rows(gp[written], op[written]):.0f}")
    else:
        frac = gu.assert_fp8_rows(gp[written], st.g_cache.scales.cpu().numpy()[written], op[written],
                                  st.o_cache.scales[written])
        _log(f"fp8 identical codes {frac:.5f}")


def test_compress_chunk_split_and_determinism():
    _log("compress chunk split")
    cfg = StepConfig(seed=7, ratio=4, lens=[900, 613], dim=512, rope_dims=64, heads=16, cache_dtype="bf16",
                     in_dtype="bf16", indexer=False)
    a = Step(cfg)
    a.run_gpu()
    b = Step(cfg)
    b.run_gpu()
    assert torch.equal(a.g_cache.pages.view(torch.int16), b.g_cache.pages.view(torch.int16))
    c = Step(cfg)
    c.g_rope = csa.rope_table(c.rows, 64)
    c.g_cache = c._gpu_cache(512, 64, "bf16")
    c.g_state = c._gpu_state(512, 2)
    cuts = [[0, 1, 250, 251, 900, 901], [0, 300, 301, 613, 614, 614]]
    for j in range(5):
        lo = [cuts[0][j], cuts[1][j]]
        hi = [cuts[0][j + 1], cuts[1][j + 1]]
        c._gpu_compress(c.g_cache, c.g_state, c.kv, c.lg, c.gamma, c.g_rope, lo, hi)
    torch.cuda.synchronize()
    assert torch.equal(a.g_cache.pages.view(torch.int16), c.g_cache.pages.view(torch.int16))


@pytest.mark.parametrize("cd,dims,lens,n_new", [("bf16", (512, 128), [700, 259, 300, 1031, 7, 64], 1),
                                                 ("fp8", (512, 128), [700, 259, 303, 1031], 1),
                                                 ("bf16", (512, 128), [700, 259, 300], 37),
                                                 ("bf16", (256, 64), [700, 259, 300], 5)])
def test_compress_insert_pair_matches_two_calls(cd, dims, lens, n_new):
    """compress_insert_pair (one launch for a 512 main + 128 indexer c4a pair, two launches otherwise) writes exactly
    what two compress_insert calls write: caches, scales and compressor state, bit for bit."""
    _log(f"compress pair cache={cd} dims={dims} lens={lens} n_new={n_new}")
    import synth
    g = synth.rng(88, dims[0] + n_new)
    B = len(lens)
    nb = max(lens) // 256 + 2
    n_phys = B * nb + 2
    bt = gu.dev_i32(synth.random_block_table(synth.rng(88, synth.STREAM_BT), B, nb, n_phys))
    sides = []
    for _ in range(2):
        per = []
        for d in dims:
            pages = torch.zeros((n_phys * 64, d), dtype=torch.uint8 if cd == "fp8" else torch.bfloat16, device="cuda")
            sc = torch.zeros(n_phys * 64, device="cuda") if cd == "fp8" else None
            cache = csa.Cache(4, 8, d, 64 if d >= 128 else 32, pages, bt, sc)
            state = csa.Raw(d, 2, torch.zeros((n_phys * 256, d), dtype=torch.bfloat16, device="cuda"), bt,
                            torch.zeros((n_phys * 256, 2, d), dtype=torch.bfloat16, device="cuda"))
            per.append((cache, state))
        sides.append(per)
    # history: positions 0..L-1 already in the caches (identical on both sides), then n_new tokens per sequence
    rows = max(lens) + n_new + 1
    ropes = [csa.rope_table(rows, 64 if d >= 128 else 32) for d in dims]
    gammas = [gu.dev_f32(synth.uniform_f32(g, (d,), 0.5, 1.5)) for d in dims]
    hist = [(gu.dev_bf16(synth.normal_bf16_bits(g, (sum(lens), d))), gu.dev_bf16(synth.normal_bf16_bits(g, (sum(lens), 2, d))))
            for d in dims]
    new = [(gu.dev_bf16(synth.normal_bf16_bits(g, (B * n_new, d))), gu.dev_bf16(synth.normal_bf16_bits(g, (B * n_new, 2, d))))
           for d in dims]
    cu_h = gu.dev_i32(np.concatenate([[0], np.cumsum(lens)]))
    zero = gu.dev_i32(np.zeros(B))
    start = gu.dev_i32(lens)
    cu_n = gu.dev_i32(np.arange(B + 1) * n_new)
    for per in sides:
        for (cache, state), (kv, lg), gm, rp in zip(per, hist, gammas, ropes):
            csa.compress_insert(cache, state, zero, cu_h, kv, lg, gm, 1e-6, rp, max(lens))
    (ca, sa), (cb, sb) = sides[0]
    csa.compress_insert_pair(ca, sa, new[0][0], new[0][1], gammas[0], ropes[0], cb, sb, new[1][0], new[1][1], gammas[1],
                             ropes[1], start, cu_n, 1e-6, n_new)
    for (cache, state), (kv, lg), gm, rp in zip(sides[1], new, gammas, ropes):
        csa.compress_insert(cache, state, start, cu_n, kv, lg, gm, 1e-6, rp, n_new)
    torch.cuda.synchronize()
    for (c0, s0), (c1, s1) in zip(sides[0], sides[1]):
        assert torch.equal(c0.pages.view(torch.uint8), c1.pages.view(torch.uint8))
        if cd == "fp8":
            assert torch.equal(c0.scales, c1.scales)
        assert torch.equal(s0.kv_pages.view(torch.uint8), s1.kv_pages.view(torch.uint8))
        assert torch.equal(s0.logit_pages.view(torch.uint8), s1.logit_pages.view(torch.uint8))


# ------------------------------------------------------------------ index_topk
def _gpu_cache(pc: si.PagedCache) -> csa.Cache:
    return csa.Cache(pc.ratio, pc.window, pc.dim, 0, gu.dev_store(pc.pages, pc.dtype), gu.dev_i32(pc.bt),
                     gu.dev_f32(pc.scales) if pc.scales is not None else None)


def _run_index(pc, positions, q, w, mode, k, q_dtype):
    B = len(positions)
    max_elig = max(paging.num_eligible(p, 4, 8) for p in positions)
    out = torch.full((B, k), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    sc = torch.zeros((B, k), dtype=torch.float32, device="cuda")
    qd = gu.dev_f32(q) if q_dtype == "f32" else gu.dev_bf16(q)
    csa.index_topk(_gpu_cache(pc), gu.dev_i32(np.arange(B)), gu.dev_i32(positions), max_elig, qd,
                   gu.dev_f32(w) if w is not None else None, mode, k, out, cnt, sc)
    torch.cuda.synchronize()
    return out.cpu().numpy(), cnt.cpu().numpy(), sc.cpu().numpy()


INDEX_GRID_CASES = [
    ("bf16", 64, 128, oi.WRELU, 512, [20000, 131, 6, 2060, 2063, 8000]),
    ("fp8", 64, 128, oi.WRELU, 512, [9000, 2051, 30, 7]),
    ("bf16", 16, 128, oi.WRELU, 64, [5000, 300]),
    ("bf16", 64, 128, oi.WRELU, 2048, [12000, 8203]),
    ("f32", 1, 32, oi.DOT, 64, [1024, 900, 3]),
    ("bf16", 4, 64, oi.WRELU, 100, [3000, 1500]),
    ("fp8", 2, 32, oi.WRELU, 1, [4000, 10]),
    # more than 2^18 eligible entries: the chosen-entry bitmap lives in the workspace, not in LDS
    ("bf16", 16, 128, oi.WRELU, 512, [1200000, 40000]),
    # few queries of more than 2^16 entries (separate mark pass, bitmap in LDS) at the largest k
    ("fp8", 64, 128, oi.WRELU, 2048, [400000, 300000]),
    # many queries in one launch: pages shared by the queries of a workgroup (one sequence per query here, so
    # every workgroup runs one round per query), bf16 and fp8 pages, 64 and 16 heads
    ("bf16", 64, 128, oi.WRELU, 512, [300 + 13 * i for i in range(300)]),
    ("fp8", 64, 128, oi.WRELU, 512, [700 + 29 * i for i in range(288)]),
    ("bf16", 16, 128, oi.WRELU, 100, [5000 - 17 * i for i in range(260)]),
    # many queries at the largest k: the half-size select writes four output slots per thread
    ("bf16", 64, 128, oi.WRELU, 2048, [9000 + 7 * i for i in range(256)]),
    # many queries with few or no eligible entries (positions 0..39: 0..9 entries each)
    ("bf16", 64, 128, oi.WRELU, 4, [i % 40 for i in range(280)]),
]


@pytest.mark.parametrize("dtype,heads,dim,mode,k,positions", INDEX_GRID_CASES)
def test_index_topk_exact_grid_bit_exact(dtype, heads, dim, mode, k, positions):
    """Exact-grid keys, queries and weights: every score is exact in fp32 in any order -> bit-exact sets and scores."""
    _log(f"index grid dtype={dtype} H={heads} D={dim} mode={mode} k={k} pos={positions}")
    import synth
    cfg = 11 + k + heads
    pc = si.paged_cache(cfg, 4, dim, dtype, positions, grid=True)
    g = synth.rng(cfg, synth.STREAM_QIDX)
    qv = synth.grid_values(g, (len(positions), heads, dim))
    w = (np.rint(synth.rng(cfg, synth.STREAM_HEADW).uniform(0, 16, (len(positions), heads))) / 16).astype(np.float32) \
        if mode == oi.WRELU else None
    q_dtype = "f32" if dtype == "f32" else "bf16"
    q_store = qv if q_dtype == "f32" else (qv.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    o_idx, o_cnt, o_sc = oi.index_topk(pc.oracle(), np.arange(len(positions)), positions,
                                       codecs.load_rows(q_store, q_dtype), w, mode, k)
    out, cnt, sc = _run_index(pc, positions, q_store, w, mode, k, q_dtype)
    assert np.array_equal(cnt, o_cnt)
    assert np.array_equal(out, o_idx)
    m = o_idx >= 0
    assert np.array_equal(sc[m].astype(np.float64), o_sc[m])
    assert np.all(np.isnan(sc[~m]))


@pytest.mark.parametrize("k,positions", [(512, [5000, 3000, 30000]), (2048, [5000, 3000, 30000]),
                                         (512, [300000, 70000, 2000]), (2048, [400000, 90000, 2000]),
                                         (2048, [1100000, 2000])])
def test_index_topk_all_ties_takes_lowest_indices(k, positions):
    """Every score equal: the lowest k indices win. 30000 tokens give 7498 tied candidates, more than
    the select kernel's LDS list holds, so its workspace overflow list takes part. With few queries of more
    than 2^16 entries the keys are scanned by the separate mark pass (every key a candidate), and one query
    there has fewer entries than k."""
    _log(f"index all ties k={k} pos={positions}")
    pc = si.paged_cache(3, 4, 128, "bf16", positions)
    pc.pages[:] = 0x3F80  # every key = 1.0
    q = np.full((3, 64, 128), 0x3F80, np.uint16)
    w = np.full((3, 64), 0.5, np.float32)
    out, cnt, sc = _run_index(pc, positions, q, w, oi.WRELU, k, "bf16")
    for b, p in enumerate(positions):
        n = min(k, paging.num_eligible(p, 4, 8))
        assert cnt[b] == n
        assert np.array_equal(out[b][:n], np.arange(n)) and np.all(out[b][n:] == -1)
        assert np.all(sc[b][:n] == 64 * 0.5 * 128.0) and np.all(np.isnan(sc[b][n:]))


def _run_index_one_seq(pc, positions, q, w, mode, k, q_dtype):
    """Every query on sequence 0 of `pc`."""
    B = len(positions)
    max_elig = max(paging.num_eligible(p, pc.ratio, pc.window) for p in positions)
    out = torch.full((B, k), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    sc = torch.zeros((B, k), dtype=torch.float32, device="cuda")
    qd = gu.dev_f32(q) if q_dtype == "f32" else gu.dev_bf16(q)
    csa.index_topk(_gpu_cache(pc), gu.dev_i32(np.zeros(B, np.int64)), gu.dev_i32(positions), max_elig, qd,
                   gu.dev_f32(w) if w is not None else None, mode, k, out, cnt, sc)
    torch.cuda.synchronize()
    return out.cpu().numpy(), cnt.cpu().numpy(), sc.cpu().numpy()


def test_index_topk_many_queries_long_bit_exact():
    """256 queries of one 600000-token sequence (up to 149999 eligible entries): the many-query select runs
    several key chunks per query and, as the launch's longest query has more than 131072 entries, keeps every
    query's chosen-entry bitmap in the workspace (shorter launches keep them in LDS; the other many-query tests
    cover those). Exact-grid keys and queries make every score exact and leave many equal
    scores, so ties at the boundary (lowest index first) and long candidate lists take part. A query's eligible
    entries are a prefix of the sequence's entry list, so the oracle's keys are taken once for the longest."""
    import synth
    P = 600000
    positions = np.unique(np.concatenate([np.linspace(9, P, 252).astype(np.int64), [P - 1, P, 524300, 524296, 7, 8]]))
    assert len(positions) >= 256
    _log(f"index many queries long: {len(positions)} queries up to {P}")
    pc = si.paged_cache(71, 4, 32, "f32", [P], grid=True)
    q = synth.grid_values(synth.rng(71, synth.STREAM_QIDX), (len(positions), 1, 32))
    k = 64
    out, cnt, sc = _run_index_one_seq(pc, positions, q, None, oi.DOT, k, "f32")
    keys = oi.eligible_keys(pc.oracle(), 0, P)
    for b, p in enumerate(positions):
        n = paging.num_eligible(int(p), 4, 8)
        o_idx, o_sc, o_cnt = oi.topk(oi.scores(keys[:n], q[b], None, oi.DOT), k)
        assert cnt[b] == o_cnt, (p, cnt[b], o_cnt)
        assert np.array_equal(out[b], o_idx), p
        assert np.array_equal(sc[b][:o_cnt].astype(np.float64), o_sc[:o_cnt]), p


def test_index_topk_long_queries_bitmap_in_workspace():
    """80 queries of one 1.1M-token sequence (up to 274999 eligible entries): more than 64 queries, so no mark pass;
    the 1024-thread select runs several key chunks per query and, as the launch's longest query has more than
    262144 entries, keeps every query's chosen-entry bitmap in the workspace. Exact-grid keys and queries as in the
    many-query test above."""
    import synth
    P = 1100000
    positions = np.unique(np.concatenate([np.linspace(9, P, 76).astype(np.int64), [P - 1, P, 1048576, 7]]))
    assert 64 < len(positions) < 256
    _log(f"index long queries, bitmap in the workspace: {len(positions)} queries up to {P}")
    pc = si.paged_cache(73, 4, 32, "f32", [P], grid=True)
    q = synth.grid_values(synth.rng(73, synth.STREAM_QIDX), (len(positions), 1, 32))
    k = 64
    out, cnt, sc = _run_index_one_seq(pc, positions, q, None, oi.DOT, k, "f32")
    keys = oi.eligible_keys(pc.oracle(), 0, P)
    for b, p in enumerate(positions):
        n = paging.num_eligible(int(p), 4, 8)
        o_idx, o_sc, o_cnt = oi.topk(oi.scores(keys[:n], q[b], None, oi.DOT), k)
        assert cnt[b] == o_cnt, (p, cnt[b], o_cnt)
        assert np.array_equal(out[b], o_idx), p
        assert np.array_equal(sc[b][:o_cnt].astype(np.float64), o_sc[:o_cnt]), p


def test_index_topk_many_queries_all_ties():
    """300 queries of one sequence, every score equal: each query's lowest k entries win. Up to 9999 tied
    candidates per query overflow the many-query select's LDS list into the workspace list."""
    positions = np.array([40000 - 131 * i for i in range(300)], np.int64)
    _log("index many queries all ties")
    pc = si.paged_cache(5, 4, 128, "bf16", [int(positions.max())])
    pc.pages[:] = 0x3F80  # every key = 1.0
    q = np.full((len(positions), 64, 128), 0x3F80, np.uint16)
    w = np.full((len(positions), 64), 0.5, np.float32)
    k = 512
    out, cnt, sc = _run_index_one_seq(pc, positions, q, w, oi.WRELU, k, "bf16")
    for b, p in enumerate(positions):
        n = min(k, paging.num_eligible(int(p), 4, 8))
        assert cnt[b] == n
        assert np.array_equal(out[b][:n], np.arange(n)) and np.all(out[b][n:] == -1)
        assert np.all(sc[b][:n] == 64 * 0.5 * 128.0) and np.all(np.isnan(sc[b][n:]))


@pytest.mark.parametrize("dtype,positions", [("bf16", [20000, 14011, 9001, 300, 7]), ("fp8", [30000, 2100]),
                                             ("bf16", [400000, 90001, 1500]), ("fp8", [1100000, 300])])
def test_index_topk_continuous_near_ties(dtype, positions):
    """N(0,1) keys and queries: the GPU set equals the oracle set up to swaps certified as fp32 near-ties."""
    _log(f"index continuous {dtype} {positions}")
    import synth
    pc = si.paged_cache(31, 4, 128, dtype, positions)
    if dtype == "fp8":  # per-entry scales that differ from entry to entry (a scale read from the wrong row shows)
        pc.scales = pc.scales * synth.uniform_f32(synth.rng(31, 41), pc.scales.shape, 0.25, 4.0)
    q = synth.normal_bf16_bits(synth.rng(31, synth.STREAM_QIDX), (len(positions), 64, 128))
    w = synth.uniform_f32(synth.rng(31, synth.STREAM_HEADW), (len(positions), 64))
    out, cnt, sc = _run_index(pc, positions, q, w, oi.WRELU, 512, "bf16")
    oc_ = pc.oracle()
    qf = codecs.load_rows(q, "bf16")
    swaps = 0
    for b, p in enumerate(positions):
        keys = oi.eligible_keys(oc_, b, p)
        s = oi.scores(keys, qf[b], w[b], oi.WRELU)
        mag = (np.abs(keys) @ np.abs(qf[b]).T) @ w[b].astype(np.float64)
        delta = 2.0 * (128 + 64 + 2) * 2.0 ** -24 * mag
        swaps += gu.check_topk_near_ties(out[b], cnt[b], s, 512, delta)
        kk = cnt[b]
        # returned scores are the GPU's fp32 scores of the returned entries
        assert np.all(np.abs(sc[b][:kk] - s[out[b][:kk]]) <= delta[out[b][:kk]])
    _log(f"certified near-tie swaps: {swaps}")


def test_index_topk_self_consistent_selection():
    """With k >= n_elig every entry comes back with its score; a smaller k picks exactly the top of those
    scores under (score desc, index asc) -- the selection itself is exact whatever the scores are."""
    _log("index self-consistency")
    import synth
    positions = [8150, 5003, 7, 4099]
    pc = si.paged_cache(21, 4, 128, "bf16", positions)
    q = synth.normal_bf16_bits(synth.rng(21, synth.STREAM_QIDX), (4, 64, 128))
    w = synth.uniform_f32(synth.rng(21, synth.STREAM_HEADW), (4, 64))
    all_idx, all_cnt, all_sc = _run_index(pc, positions, q, w, oi.WRELU, 2048, "bf16")
    for k in (1, 64, 512, 2047):
        out, cnt, _ = _run_index(pc, positions, q, w, oi.WRELU, k, "bf16")
        for b, p in enumerate(positions):
            n = paging.num_eligible(p, 4, 8)
            assert all_cnt[b] == n and np.array_equal(all_idx[b][:n], np.arange(n))
            s = all_sc[b][:n]
            order = np.lexsort((np.arange(n), -s.astype(np.float64)))
            want = np.sort(order[: min(k, n)])
            assert cnt[b] == min(k, n)
            assert np.array_equal(out[b][: cnt[b]], want) and np.all(out[b][cnt[b]:] == -1)


# ------------------------------------------------------------------ attend + inverse RoPE
ATTEND_CASES = [
    # ratio, dim, heads, dtype, top-k (0 = dense), positions
    (4, 128, 8, "f32", 64, [1024, 300]),
    (128, 512, 64, "bf16", 0, [4100, 1000, 130, 3]),
    (4, 512, 64, "bf16", 512, [9000, 3001, 40, 5]),
    (4, 512, 64, "fp8", 512, [7000, 2222]),
    (128, 512, 32, "fp8", 0, [3000, 127]),
    (4, 256, 4, "bf16", 100, [2000]),
    (4, 512, 16, "bf16", 2048, [9000]),
    # many queries: one key split per query, output written directly by the attention workgroup
    (4, 512, 64, "bf16", 64, [300 + (37 * i) % 400 for i in range(520)]),
    # 16 queries of 64 heads (key splits and their merge); short contexts leave top-k slots unfilled and windows
    # partly before position 0
    (4, 512, 64, "bf16", 512, [9000, 3001, 40, 5, 21000, 2059, 777, 20000, 12, 14000, 3, 4100, 9999, 2047, 700, 131]),
    (4, 512, 64, "fp8", 512, [7000, 2222, 17, 19000, 4095, 300, 15000, 1030, 8, 10000, 2500, 611, 12345, 77, 4000,
                              5555, 3001]),
    (128, 512, 64, "bf16", 0, [70000, 4100, 1000, 130, 3, 65535, 32768, 127, 128, 255, 9000, 50000, 20000, 700, 16000,
                               60000]),
    (4, 512, 128, "bf16", 2048, [12000, 9500, 30000, 100, 2060, 8191, 20000, 700]),  # 128 heads, top-2048 + window
]


@pytest.mark.parametrize("ratio,dim,heads,dtype,k,positions", ATTEND_CASES)
def test_attend_parity(ratio, dim, heads, dtype, k, positions):
    _log(f"attend ratio={ratio} dim={dim} H={heads} dtype={dtype} k={k} pos={positions}")
    import synth
    cfg = 41 + dim + k
    R = 64
    pc = si.paged_cache(cfg, ratio, dim, dtype, positions)
    n_phys = pc.bt.max() + 1 + 3
    swa_pages, swa_sc = si.window_rows(cfg, dim, dtype, n_phys)
    q_dtype = "f32" if dtype == "f32" else "bf16"
    g = synth.rng(cfg, synth.STREAM_Q)
    q = synth.normal_f32(g, (len(positions), heads, dim)) if q_dtype == "f32" else \
        synth.normal_bf16_bits(g, (len(positions), heads, dim))
    tk = si.topk_lists(cfg, positions, ratio, k) if k else None
    rows = max(positions) + 1
    scale = float(1.0 / np.sqrt(dim))
    # oracle
    ocache = pc.oracle(R)
    oswa = oc.Raw(dtype, dim, 0, swa_pages, None, swa_sc, pc.bt)
    qf = codecs.load_rows(q, q_dtype)
    table = orope.rope_table(rows, R)
    o_out, o_lse = oa.attend(ocache, oswa, 128, np.arange(len(positions)), positions, qf, tk, scale, True, table)
    o_raw, _ = oa.attend(ocache, oswa, 128, np.arange(len(positions)), positions, qf, tk, scale, False, table)
    # gpu
    gcache = csa.Cache(ratio, pc.window, dim, R, gu.dev_store(pc.pages, dtype), gu.dev_i32(pc.bt),
                       gu.dev_f32(pc.scales) if pc.scales is not None else None)
    gswa = csa.Raw(dim, 0, gu.dev_store(swa_pages, dtype), gu.dev_i32(pc.bt), None,
                   gu.dev_f32(swa_sc) if swa_sc is not None else None)
    grope = csa.rope_table(rows, R)
    qs, qp = gu.dev_i32(np.arange(len(positions))), gu.dev_i32(positions)
    qd = gu.dev_f32(q) if q_dtype == "f32" else gu.dev_bf16(q)
    gtk = gu.dev_i32(tk) if tk is not None else None
    max_elig = max(paging.num_eligible(p, ratio, pc.window) for p in positions)
    out = torch.full((len(positions), heads, dim), -7.0, device="cuda")
    lse = torch.full((len(positions), heads), -7.0, device="cuda")
    csa.attend(gcache, gswa, 128, qs, qp, qd, gtk, max_elig, scale, True, grope, out, lse)
    out2 = torch.full_like(out, -7.0)
    csa.attend(gcache, gswa, 128, qs, qp, qd, gtk, max_elig, scale, False, grope, out2)
    torch.cuda.synchronize()
    err = gu.rowwise_rel_err(out.cpu().numpy(), o_out)
    err_raw = gu.rowwise_rel_err(out2.cpu().numpy(), o_raw)
    _log(f"attend rowwise rel err fused {err:.3e} unfused {err_raw:.3e}")
    assert err <= TOL[dtype] and err_raw <= TOL[dtype]
    assert np.allclose(lse.cpu().numpy(), o_lse, rtol=0, atol=1e-4 if dtype != "f32" else 1e-5)
    # standalone inverse RoPE kernel on the unfused output reproduces the fused output
    csa.inv_rope(out2, qp, R, grope)
    torch.cuda.synchronize()
    assert gu.rowwise_rel_err(out2.cpu().numpy(), out.cpu().numpy()) <= 1e-6


@pytest.mark.parametrize("heads,k,window,dtype,positions", [(128, 512, 128, "bf16", [9000, 3001, 700]),
                                                             (64, 2048, 1024, "bf16", [12000, 9500]),
                                                             (64, 2048, 1024, "fp8", [12000]),
                                                             (128, 0, 1024, "bf16", [70000, 1100])])
def test_attend_maximum_sizes(heads, k, window, dtype, positions):
    """The largest shapes the ABI takes: 128 heads (two 64-head chunks per query), top-2048 plus a 1024-row window
    (the key-row table exactly full), and dense c128a with a 1024-row window."""
    _log(f"attend max heads={heads} k={k} window={window} dtype={dtype} pos={positions}")
    import synth
    ratio = 4 if k else 128
    dim, R = 512, 64
    cfg = 77 + heads + k + window
    pc = si.paged_cache(cfg, ratio, dim, dtype, positions)
    n_phys = pc.bt.max() + 1 + 3
    swa_pages, swa_sc = si.window_rows(cfg, dim, dtype, n_phys)
    q = synth.normal_bf16_bits(synth.rng(cfg, synth.STREAM_Q), (len(positions), heads, dim))
    tk = si.topk_lists(cfg, positions, ratio, k) if k else None
    rows = max(positions) + 1
    scale = float(1.0 / np.sqrt(dim))
    o_out, o_lse = oa.attend(pc.oracle(R), oc.Raw(dtype, dim, 0, swa_pages, None, swa_sc, pc.bt), window,
                             np.arange(len(positions)), positions, codecs.load_rows(q, "bf16"), tk, scale, True,
                             orope.rope_table(rows, R))
    gcache = csa.Cache(ratio, pc.window, dim, R, gu.dev_store(pc.pages, dtype), gu.dev_i32(pc.bt),
                       gu.dev_f32(pc.scales) if pc.scales is not None else None)
    gswa = csa.Raw(dim, 0, gu.dev_store(swa_pages, dtype), gu.dev_i32(pc.bt), None,
                   gu.dev_f32(swa_sc) if swa_sc is not None else None)
    max_elig = max(paging.num_eligible(p, ratio, pc.window) for p in positions)
    out = torch.full((len(positions), heads, dim), -7.0, device="cuda")
    lse = torch.full((len(positions), heads), -7.0, device="cuda")
    csa.attend(gcache, gswa, window, gu.dev_i32(np.arange(len(positions))), gu.dev_i32(positions), gu.dev_bf16(q),
               gu.dev_i32(tk) if tk is not None else None, max_elig, scale, True, csa.rope_table(rows, R), out, lse)
    torch.cuda.synchronize()
    err = gu.rowwise_rel_err(out.cpu().numpy(), o_out)
    _log(f"rowwise rel err {err:.3e}")
    assert err <= TOL[dtype]
    assert np.allclose(lse.cpu().numpy(), o_lse, rtol=0, atol=1e-4)


def test_inv_rope_parity():
    _log("inv_rope")
    import synth
    x = synth.normal_f32(synth.rng(61, 0), (5, 8, 512))
    pos = np.array([0, 1, 1000, 65536, 1048576], np.int32)
    table = orope.rope_table((1 << 20) + 1, 64)
    ref = orope.inv_rope_queries(x.astype(np.float64), pos, table, 64)
    t = gu.dev_f32(x)
    csa.inv_rope(t, gu.dev_i32(pos), 64, csa.rope_table((1 << 20) + 1, 64))
    torch.cuda.synchronize()
    assert gu.rowwise_rel_err(t.cpu().numpy(), ref) <= 1e-6


@pytest.mark.parametrize("heads,dim,rope,group", [(64, 512, 64, 128), (8, 128, 64, 32), (16, 512, 64, 512),
                                                  (4, 256, 0, 64), (3, 64, 32, 8)])
def test_inv_rope_quant_fp8_parity(heads, dim, rope, group):
    """Inverse RoPE + fp8 output quantisation against the oracle: scales within 2^-14, each dequantised element
    within one e4m3 step; an all-zero row stores zero codes with scale 1."""
    _log(f"inv_rope_quant_fp8 H={heads} D={dim} R={rope} G={group}")
    import synth
    from oracle import output_quant as oq
    pos = np.array([0, 1, 1000, 65536, 1 << 20, 7, 4095], np.int32)
    g = synth.rng(91, dim + group)
    x = synth.normal_f32(g, (len(pos), heads, dim)) * synth.uniform_f32(g, (len(pos), heads, 1), 0.01, 40.0)
    x[5, 0] = 0.0
    rows = (1 << 20) + 1
    table = orope.rope_table(rows, rope if rope else 64)
    ref_codes, ref_scales = oq.inv_rope_quant(x.astype(np.float64), pos, table, rope, group)
    codes, scales = csa.inv_rope_quant_fp8(gu.dev_f32(x), gu.dev_i32(pos), rope, csa.rope_table(rows, rope if rope else 64),
                                           group)
    torch.cuda.synchronize()
    codes, scales = codes.cpu().numpy(), scales.cpu().numpy()
    frac = gu.assert_fp8_rows(codes.reshape(-1, group), scales.reshape(-1), ref_codes.reshape(-1, group),
                              ref_scales.reshape(-1))
    assert np.all(codes[5, 0] == 0) and np.all(scales[5, 0] == 1.0)
    _log(f"identical codes {frac:.5f}")


@pytest.mark.parametrize("q_dtype,win_dtype,heads,dim,rope", [("bf16", "bf16", 64, 512, 64), ("bf16", "fp8", 64, 512, 64),
                                                                ("f32", "f32", 8, 128, 64), ("bf16", "bf16", 4, 32, 16)])
def test_prepare_qk_parity(q_dtype, win_dtype, heads, dim, rope):
    """Query norm + RoPE and window-key RoPE + insert against the oracle: queries within one bf16 ulp (fp32: 1e-6
    rowwise), written window rows within one storage step, every other row (and an unmapped block) untouched."""
    _log(f"prepare_qk q={q_dtype} window={win_dtype} H={heads} D={dim} R={rope}")
    import synth
    from oracle import prepare as op
    g = synth.rng(95, dim + heads)
    positions = np.array([0, 255, 256, 131071, 131072, 77, 5000, 300], np.int32)
    seqs = np.array([0, 0, 3, 2, 2, 3, 3, 1], np.int32)
    nb = 131072 // 256 + 1
    n_phys = 4 * nb
    bt = synth.random_block_table(synth.rng(95, synth.STREAM_BT), 4, nb, n_phys)
    bt[1, 300 // 256] = -1  # the last token's block is unmapped: it must be skipped
    n = len(positions)
    q = synth.normal_f32(g, (n, heads, dim)) * 3.0 if q_dtype == "f32" else synth.normal_bf16_bits(g, (n, heads, dim))
    kv = synth.normal_f32(g, (n, dim)) if q_dtype == "f32" else synth.normal_bf16_bits(g, (n, dim))
    gamma = synth.uniform_f32(g, (dim,), 0.5, 1.5)
    pages = gu.canary((n_phys * 256, dim), win_dtype)
    scales = np.full(n_phys * 256, np.nan, np.float32) if win_dtype == "fp8" else None
    rows = 131073
    table = orope.rope_table(rows, rope)
    oswa = oc.Raw(win_dtype, dim, 0, pages.copy(), None, None if scales is None else scales.copy(), bt)
    ref_q = op.prepare_qk(codecs.load_rows(q, q_dtype), q_dtype, codecs.load_rows(kv, q_dtype), seqs, positions, gamma,
                          1e-6, table, rope, oswa)
    gswa = csa.Raw(dim, 0, gu.dev_store(pages, win_dtype), gu.dev_i32(bt), None,
                   gu.dev_f32(scales) if scales is not None else None)
    qd = gu.dev_f32(q) if q_dtype == "f32" else gu.dev_bf16(q)
    kd = gu.dev_f32(kv) if q_dtype == "f32" else gu.dev_bf16(kv)
    out = csa.prepare_qk(qd, kd, gu.dev_i32(seqs), gu.dev_i32(positions), gu.dev_f32(gamma), 1e-6, gswa, rope,
                         csa.rope_table(rows, rope))
    torch.cuda.synchronize()
    got_q = gu.host_store(out)
    if q_dtype == "f32":
        assert gu.rowwise_rel_err(got_q, ref_q) <= 1e-6
    else:
        gu.assert_bf16_rows(got_q.reshape(-1, dim), ref_q.reshape(-1, dim))
    gp = gu.host_store(gswa.kv_pages)
    written = np.zeros(gp.shape[0], bool)
    for s_, p_ in zip(seqs, positions):
        if bt[s_, p_ // 256] >= 0:
            written[paging.raw_slot(bt[s_], int(p_))] = True
    assert written.sum() == n - 1
    if win_dtype == "fp8":
        gs = gswa.scales.cpu().numpy()
        gu.assert_fp8_rows(gp[written], gs[written], oswa.kv_pages[written], oswa.scales[written])
        assert np.array_equal(gp[~written], pages[~written]) and np.all(np.isnan(gs[~written]))
    elif win_dtype == "bf16":
        gu.assert_bf16_rows(gp[written], oswa.kv_pages[written])
        assert np.array_equal(gp[~written], pages[~written])
    else:
        assert gu.rowwise_rel_err(gp[written], oswa.kv_pages[written]) <= 1e-6
        assert np.all(np.isnan(gp[~written]))


def test_attend_deterministic():
    _log("attend determinism")
    cfg = StepConfig(seed=51, ratio=4, lens=[5000, 3000], dim=512, rope_dims=64, heads=64, cache_dtype="bf16",
                     in_dtype="bf16", indexer=True, idx_dim=128, idx_rope=64, idx_heads=64, idx_dtype="bf16",
                     mode=oi.WRELU, k=512)
    st = Step(cfg)
    st.run_gpu()
    first = st.g_out.clone()
    tk = st.g_topk.clone()
    for _ in range(5):
        csa.index_topk(st.g_icache, gu.dev_i32(st.q_seq), gu.dev_i32(st.q_pos), st.max_elig, gu.dev_bf16(st.q_idx),
                       gu.dev_f32(st.head_w), oi.WRELU, 512, st.g_topk)
        csa.attend(st.g_cache, st.g_swa, 128, gu.dev_i32(st.q_seq), gu.dev_i32(st.q_pos), gu.dev_bf16(st.q), st.g_topk,
                   st.max_elig, st.scale, True, st.g_rope, st.g_out)
        torch.cuda.synchronize()
        assert torch.equal(tk, st.g_topk)
        assert torch.equal(first, st.g_out)


# ------------------------------------------------------------------ whole decode steps, oracle end to end
def test_c1_chain_end_to_end():
    """c4a fp32 decode, batch 1, query at 1024, 8 heads, D 128 (R 64), indexer 1 head D 32 (DOT), top-64 + window 128."""
    _log("c1 chain")
    from tests import smoke_step
    smoke_step.run(verbose=True)


@pytest.mark.parametrize("cache_dtype", ["bf16", "fp8"])
def test_bf16_chain_end_to_end(cache_dtype):
    """c4a decode with bf16 raw tokens, D 512 / 64 heads, indexer 64 heads x 128 (WRELU), top-512 + window.

    Strict: counts and slots bit-exact; every eligible cache row within the rounding-aware storage bound; the
    top-k sets equal up to certified near-ties (scores differing by at most fp32 accumulation plus the bound
    on the stored keys); attention of every sequence within the benchmark spec's tolerance (2e-3 bf16, 5e-2 fp8)."""
    _log(f"bf16 chain cache={cache_dtype}")
    from tests.chain import verify
    cfg = StepConfig(seed=71, ratio=4, lens=[6000, 4093, 811], dim=512, rope_dims=64, heads=64, cache_dtype=cache_dtype,
                     in_dtype="bf16", indexer=True, idx_dim=128, idx_rope=64, idx_heads=64, idx_dtype=cache_dtype,
                     mode=oi.WRELU, k=512)
    st = Step(cfg)
    st.run_gpu()
    st.run_oracle()
    res = verify(st, TOL[cache_dtype], 1e-4, log=_log)
    _log(f"certified swaps {res['swaps']}, re-attended sequences {res['reattended']}")


# ------------------------------------------------------------------ attention with the fp8 output epilogue fused in
@pytest.mark.parametrize("ratio,heads,dtype,k,group,positions", [
    (4, 64, "bf16", 512, 128, [9000, 3001, 40, 5]),                      # several key splits: the merge kernel
    (4, 64, "fp8", 512, 64, [7000, 2222]),
    (4, 64, "bf16", 64, 32, [300 + (37 * i) % 400 for i in range(520)]),  # one split: the attention epilogue
    (128, 32, "bf16", 0, 16, [3000, 127, 1025]),                          # 16-head groups, dense c128a
    (4, 16, "fp8", 2048, 128, [9000]),
    # 16 queries x 64 heads: several key splits, the fp8 groups written by the merge
    (4, 64, "bf16", 512, 64, [9000, 3001, 40, 5, 21000, 2059, 777, 20000, 12, 14000, 3, 4100, 9999, 2047, 700, 131]),
    (128, 64, "fp8", 0, 16, [70000, 4100, 1000, 130, 3, 65535, 32768, 127, 128, 255, 9000, 50000, 20000, 700, 16000,
                             60000]),
    (4, 64, "bf16", 512, 128, [9000, 3001, 40, 5, 21000, 2059, 777, 20000, 12, 14000, 3, 4100, 9999, 2047, 700, 131]),
])
def test_attend_quant_fp8_parity(ratio, heads, dtype, k, group, positions):
    """csa_attend_quant_fp8 against the oracle's attention followed by its inverse RoPE + grouped fp8 rule (R23).

    The pre-quantisation output may differ from the oracle's by the attention tolerance yerr = TOL * max|row|, so
    each group's scale may differ by yerr / 448 and each dequantised element by one e4m3 step of the oracle's code
    (times its scale) plus 2 yerr; the codes must also agree with the unfused GPU path (csa_attend, then
    csa_inv_rope_quant_fp8) to the same bar."""
    _log(f"attend quant fp8 ratio={ratio} H={heads} dtype={dtype} k={k} G={group} n_q={len(positions)}")
    import synth
    from oracle import output_quant as oq
    dim, R = 512, 64
    cfg = 61 + heads + k + group
    pc = si.paged_cache(cfg, ratio, dim, dtype, positions)
    n_phys = pc.bt.max() + 1 + 3
    swa_pages, swa_sc = si.window_rows(cfg, dim, dtype, n_phys)
    q = synth.normal_bf16_bits(synth.rng(cfg, synth.STREAM_Q), (len(positions), heads, dim))
    tk = si.topk_lists(cfg, positions, ratio, k) if k else None
    rows = max(positions) + 1
    scale = float(1.0 / np.sqrt(dim))
    table = orope.rope_table(rows, R)
    o_raw, o_lse = oa.attend(pc.oracle(R), oc.Raw(dtype, dim, 0, swa_pages, None, swa_sc, pc.bt), 128,
                             np.arange(len(positions)), positions, codecs.load_rows(q, "bf16"), tk, scale, False, table)
    ref_codes, ref_scales = oq.inv_rope_quant(o_raw, np.asarray(positions), table, R, group)
    y_ref = orope.inv_rope_queries(o_raw, np.asarray(positions), table, R)
    gcache = csa.Cache(ratio, pc.window, dim, R, gu.dev_store(pc.pages, dtype), gu.dev_i32(pc.bt),
                       gu.dev_f32(pc.scales) if pc.scales is not None else None)
    gswa = csa.Raw(dim, 0, gu.dev_store(swa_pages, dtype), gu.dev_i32(pc.bt), None,
                   gu.dev_f32(swa_sc) if swa_sc is not None else None)
    grope = csa.rope_table(rows, R)
    qs, qp, qd = gu.dev_i32(np.arange(len(positions))), gu.dev_i32(positions), gu.dev_bf16(q)
    gtk = gu.dev_i32(tk) if tk is not None else None
    max_elig = max(paging.num_eligible(p, ratio, pc.window) for p in positions)
    n_q = len(positions)
    codes = torch.full((n_q, heads, dim), 0xA5, dtype=torch.uint8, device="cuda")
    scales = torch.full((n_q, heads, dim // group), -7.0, device="cuda")
    lse = torch.full((n_q, heads), -7.0, device="cuda")
    csa.attend_quant_fp8(gcache, gswa, 128, qs, qp, qd, gtk, max_elig, scale, grope, group, codes, scales, lse)
    raw = torch.full((n_q, heads, dim), -7.0, device="cuda")
    csa.attend(gcache, gswa, 128, qs, qp, qd, gtk, max_elig, scale, False, grope, raw)
    u_codes, u_scales = csa.inv_rope_quant_fp8(raw, qp, R, grope, group)
    torch.cuda.synchronize()
    gc, gs = codes.cpu().numpy(), scales.cpu().numpy()
    tol = TOL[dtype]
    yerr = tol * np.abs(y_ref).max(axis=-1, keepdims=True)           # [n_q][H][1]
    for label, cc, ss in (("oracle", ref_codes, ref_scales), ("unfused GPU", u_codes.cpu().numpy(),
                                                              u_scales.cpu().numpy())):
        rs = ss.astype(np.float64)
        assert np.all(np.abs(gs - rs) <= yerr / 448.0 + 2.0 ** -22 * rs), f"group scales differ from the {label}'s"
        gv = oq.dequant(gc, gs, group)
        rv = oq.dequant(cc, ss, group)
        mag = np.maximum(np.abs(codecs.e4m3_to_f64(cc)), 2.0 ** -6)
        step = np.ldexp(1.0, np.floor(np.log2(mag)).astype(int) - 3) * np.repeat(rs, group, axis=-1)
        assert np.all(np.abs(gv - rv) <= 1.01 * step + 2.0 * yerr), f"fp8 outputs differ from the {label}'s"
        _log(f"identical codes vs {label}: {np.mean(gc == cc):.5f}")
    assert np.allclose(lse.cpu().numpy(), o_lse, rtol=0, atol=1e-4)
