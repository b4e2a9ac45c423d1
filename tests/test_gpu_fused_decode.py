"""The fused decode launch (csa_compress_index_score) against the separate calls it stands for (needs an MI355X).

compress_index_score + index_select must leave exactly what compress_insert_pair + index_score + index_select
leave: main and indexer caches (codes, fp8 scales, MXFP4 exponents), both compressor states, and the selected
top-k lists with their counts and scores, bit for bit. The separate calls are themselves held to the oracle by
the compress and index parity tests. Each case runs several decode steps in a row, so that every sequence passes
through a position whose token completes an entry (read by the same step's query) and through positions that
complete none; sequences with no eligible entry at all (positions below 3) are included.
"""
import numpy as np
import pytest
import torch

import long_context_compressed_compress_amd as csa
import synth
from oracle import paging
import gpu_util as gu

pytestmark = pytest.mark.gpu

K = 512


def _log(msg):
    print(msg, flush=True)


def _make_cache(dtype, dim, n_rows, bt):
    if dtype == "fp4":
        pages = torch.full((n_rows, dim // 2), 0xA5, dtype=torch.uint8, device="cuda")
        scales = torch.full((n_rows, dim // 32), 0xA5, dtype=torch.uint8, device="cuda")
        return csa.Cache(4, 8, dim, 64, pages.view(torch.float4_e2m1fn_x2), bt, scales)
    if dtype == "fp8":
        return csa.Cache(4, 8, dim, 64, torch.zeros((n_rows, dim), dtype=torch.uint8, device="cuda"), bt,
                         torch.zeros(n_rows, device="cuda"))
    return csa.Cache(4, 8, dim, 64, torch.zeros((n_rows, dim), dtype=torch.bfloat16, device="cuda"), bt, None)


def _make_state(dim, n_phys, bt):
    return csa.Raw(dim, 2, torch.zeros((n_phys * 256, dim), dtype=torch.bfloat16, device="cuda"), bt,
                   torch.zeros((n_phys * 256, 2, dim), dtype=torch.bfloat16, device="cuda"))


def _state_bytes(cache, state):
    out = [cache.pages.view(torch.uint8), state.kv_pages.view(torch.uint8), state.logit_pages.view(torch.uint8)]
    if cache.scales is not None:
        out.append(cache.scales.view(torch.uint8))
    return out


FUSED_CASES = [
    # main dtype, indexer dtype, indexer heads, history lengths (the first decode token sits at that position)
    ("bf16", "bf16", 64, [700, 259, 300, 1031, 7, 64, 3, 0, 2, 20003]),
    ("fp8", "fp8", 64, [9000, 2051, 30, 7, 4095, 1]),
    ("fp8", "fp4", 64, [9000, 2051, 30, 7, 1, 12287]),
    ("fp8", "bf16", 64, [5000, 259, 6]),
    # configurations outside the one-launch form: the call runs the two launches
    ("bf16", "fp8", 64, [3000, 259, 6]),
    ("bf16", "bf16", 32, [3000, 259, 6]),
    # no query has an eligible entry at the first step (max_elig 0: the two launches and the empty-row select), the
    # first entries complete during the later steps
    ("bf16", "bf16", 64, [0, 1, 2]),
    ("fp8", "fp4", 64, [2, 0]),
]


@pytest.mark.parametrize("main_dt,idx_dt,heads,lens", FUSED_CASES)
def test_compress_index_score_matches_separate_calls(main_dt, idx_dt, heads, lens, steps=4):
    _log(f"fused decode main={main_dt} idx={idx_dt} heads={heads} lens={lens} steps={steps}")
    B = len(lens)
    nb = (max(lens) + steps) // 256 + 2
    n_phys = B * nb + 2
    bt = gu.dev_i32(synth.random_block_table(synth.rng(93, synth.STREAM_BT), B, nb, n_phys))
    g = synth.rng(93, heads + B)
    dims = (512, 128)
    gammas = [gu.dev_f32(synth.uniform_f32(g, (d,), 0.5, 1.5)) for d in dims]
    table = csa.rope_table(max(lens) + steps + 1, 64)
    hist = [(gu.dev_bf16(synth.normal_bf16_bits(g, (max(sum(lens), 1), d))),
             gu.dev_bf16(synth.normal_bf16_bits(g, (max(sum(lens), 1), 2, d)))) for d in dims]
    new = [[(gu.dev_bf16(synth.normal_bf16_bits(g, (B, d))), gu.dev_bf16(synth.normal_bf16_bits(g, (B, 2, d))))
            for d in dims] for _ in range(steps)]
    q_idx = [gu.dev_bf16(synth.normal_bf16_bits(g, (B, heads, 128))) for _ in range(steps)]
    head_w = [gu.dev_f32(synth.uniform_f32(g, (B, heads), -1.0, 1.0)) for _ in range(steps)]
    cu_h = gu.dev_i32(np.concatenate([[0], np.cumsum(lens)]))
    zero = gu.dev_i32(np.zeros(B))
    cu_n = gu.dev_i32(np.arange(B + 1))
    seq = gu.dev_i32(np.arange(B))
    max_elig = max(paging.num_eligible(p + steps - 1, 4, 8) for p in lens)
    sides = []
    for fused in (True, False):
        main = _make_cache(main_dt, 512, n_phys * 64, bt)
        idx = _make_cache(idx_dt, 128, n_phys * 64, bt)
        sm, sx = _make_state(512, n_phys, bt), _make_state(128, n_phys, bt)
        if max(lens) > 0:
            csa.compress_insert(main, sm, zero, cu_h, *hist[0], gammas[0], 1e-6, table, max(lens))
            csa.compress_insert(idx, sx, zero, cu_h, *hist[1], gammas[1], 1e-6, table, max(lens))
        ws = csa.index_workspace(B, max_elig, K, heads)
        outs = []
        for s in range(steps):
            pos = gu.dev_i32(np.asarray(lens) + s)
            elig = max(paging.num_eligible(p + s, 4, 8) for p in lens)
            (kva, lga), (kvb, lgb) = new[s]
            if fused:
                csa.compress_index_score(main, sm, kva, lga, gammas[0], table, idx, sx, kvb, lgb, gammas[1], table,
                                         pos, cu_n, 1e-6, seq, pos, elig, q_idx[s], head_w[s], csa.SCORE_WRELU, K, ws)
            else:
                csa.compress_insert_pair(main, sm, kva, lga, gammas[0], table, idx, sx, kvb, lgb, gammas[1], table,
                                         pos, cu_n, 1e-6, 1)
                csa.index_score(idx, seq, pos, elig, q_idx[s], head_w[s], csa.SCORE_WRELU, K, ws)
            o_idx = torch.full((B, K), -7, dtype=torch.int32, device="cuda")
            o_cnt = torch.full((B,), -7, dtype=torch.int32, device="cuda")
            o_sc = torch.zeros((B, K), dtype=torch.float32, device="cuda")
            csa.index_select(idx, seq, pos, elig, K, o_idx, ws, o_cnt, o_sc)
            outs.append((o_idx, o_cnt, o_sc))
        torch.cuda.synchronize()
        sides.append((_state_bytes(main, sm) + _state_bytes(idx, sx), outs))
    (st_f, out_f), (st_s, out_s) = sides
    for a, b in zip(st_f, st_s):
        assert torch.equal(a, b)
    for s, ((i0, c0, v0), (i1, c1, v1)) in enumerate(zip(out_f, out_s)):
        assert torch.equal(c0, c1), f"step {s}: counts differ"
        assert torch.equal(i0, i1), f"step {s}: selected entries differ"
        assert torch.equal(v0.view(torch.int32), v1.view(torch.int32)), f"step {s}: scores differ"
        want = [min(paging.num_eligible(p + s, 4, 8), K) for p in lens]
        assert c0.cpu().tolist() == want
