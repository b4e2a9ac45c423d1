"""One small c4a fp32 decode step on cuda:0 through libcsa, checked against the CPU oracle run end to end.

Configuration: batch 1, raw context 1024 with the query at position 1024; 8 query heads over one shared
K=V head of dim 128 with RoPE on the last 64 dims (theta 10000); kv, logits, q ~ N(0,1) fp32; indexer of one
head of dim 32 (its own compressor, RoPE on 16 dims), score q . k; top-64 of the 255 eligible entries plus
the 128-token window; 5 blocks of 256 positions at a random physical permutation; inverse RoPE at 1024.
Both sides start from the same synthetic raw tokens; no GPU result is handed to the oracle.
"""
from __future__ import annotations

import numpy as np

from oracle import codecs, index as oi, paging
from tests import gpu_util as gu
from tests.chain import Step, StepConfig

CACHE_TOL = 1e-5
OUT_TOL = 1e-5


def run(verbose: bool = False) -> dict:
    st = Step(StepConfig())
    st.run_gpu()
    st.run_oracle()
    c = st.cfg
    res = {}
    for (gs, gc), (os_, oc_) in ((st.g_prefill, st.o_prefill), (st.g_decode, st.o_decode)):
        assert np.array_equal(gc.cpu().numpy(), oc_)
        assert np.array_equal(gs.cpu().numpy()[:, : os_.shape[1]], os_[:, : gs.shape[1]])
    n_ent = paging.num_entries(c.lens[0] + 1, 4, 8)
    assert n_ent == 255
    rows = [paging.entry_slot(st.bt[0], i, 4) for i in range(n_ent)]
    res["compress_err"] = gu.rowwise_rel_err(gu.host_store(st.g_cache.pages)[rows], st.o_cache.pages[rows])
    res["idx_compress_err"] = gu.rowwise_rel_err(gu.host_store(st.g_icache.pages)[rows], st.o_icache.pages[rows])
    assert res["compress_err"] <= CACHE_TOL and res["idx_compress_err"] <= CACHE_TOL, res
    # top-k: the GPU scored its own indexer cache in fp32; certify any swap against the oracle's fp64 scores,
    # allowing for fp32 accumulation and for the cache tolerance above
    keys = oi.eligible_keys(st.o_icache, 0, c.lens[0])
    q = st.q_idx[0][0].astype(np.float64)
    s = keys @ q
    delta = 2.0 * (c.idx_dim + 3) * 2.0 ** -24 * (np.abs(keys) @ np.abs(q)) \
        + CACHE_TOL * np.abs(keys).max(axis=1) * np.abs(q).sum()
    gi, gc = st.g_topk.cpu().numpy(), st.g_cnt.cpu().numpy()
    res["topk_swaps"] = gu.check_topk_near_ties(gi[0], gc[0], s, c.k, delta)
    res["topk_equal"] = bool(np.array_equal(gi, st.o_topk))
    if res["topk_equal"]:
        res["attend_err"] = gu.rowwise_rel_err(st.g_out.cpu().numpy(), st.o_out)
        assert res["attend_err"] <= OUT_TOL, res
        assert np.allclose(st.g_lse.cpu().numpy(), st.o_lse, rtol=0, atol=1e-5)
    if verbose:
        print("smoke:", res, flush=True)
    return res


if __name__ == "__main__":
    run(verbose=True)
