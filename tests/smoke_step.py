"""One small c4a fp32 decode step on cuda:0 through libcsa, checked against the CPU oracle run end to end.

Configuration: batch 1, raw context 1024 with the query at position 1024; 8 query heads over one shared
K=V head of dim 128 with RoPE on the last 64 dims (theta 10000); kv, logits, q ~ N(0,1) fp32; indexer of one
head of dim 32 (its own compressor, RoPE on 16 dims), score q . k; top-64 of the 255 eligible entries plus
the 128-token window; 5 blocks of 256 positions at a random physical permutation; inverse RoPE at 1024.
Both sides start from the same synthetic raw tokens; no GPU result is handed to the oracle. Every check of
tests/chain.verify applies: counts and slots bit-exact, cache rows within 1e-5 of each row's largest value,
the top-k set equal up to certified near-ties, and the attention output within 1e-5 (max over rows of
max|d| / max|ref|) with lse within 1e-5.
"""
from __future__ import annotations

from oracle import paging
from tests.chain import Step, StepConfig, verify

OUT_TOL = 1e-5
LSE_TOL = 1e-5


def run(verbose: bool = False) -> dict:
    st = Step(StepConfig())
    st.run_gpu()
    st.run_oracle()
    c = st.cfg
    assert paging.num_entries(c.lens[0] + 1, 4, 8) == 255
    res = verify(st, OUT_TOL, LSE_TOL, log=(lambda m: print("smoke:", m, flush=True)) if verbose else None)
    return res


if __name__ == "__main__":
    run(verbose=True)
