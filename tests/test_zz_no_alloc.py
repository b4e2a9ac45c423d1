"""csa_index_topk_noalloc (the index stage on the library's fixed per-GPU scratch) against csa_index_topk with a
caller workspace, through the C ABI.

Three calls in a row on one stream, each compared bit for bit with csa_index_topk on a fresh workspace:
(1) 4 long queries (up to 249999 eligible entries: the mark-pass select), (2) a smaller input of 32 shorter
queries (the one-pass select; its histogram region overlaps what call 1 left in the scratch, which the call must
clear), (3) call 1 again. Top-k indices and counts are integer outputs and must be identical; the scores come from
the same kernels and must be identical too. A request larger than the scratch is rejected before any launch.
"""
import numpy as np
import pytest
import torch

import long_context_compressed_compress_amd as csa
import synth
from oracle import index as oi, paging
from tests import gpu_util as gu
from tests import stage_inputs as si

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def _case(cfg, positions, dtype, heads=64):
    pc = si.paged_cache(cfg, 4, 128, dtype, positions)
    g = synth.rng(cfg, synth.STREAM_QIDX)
    q = synth.normal_bf16_bits(g, (len(positions), heads, 128))
    w = synth.uniform_f32(synth.rng(cfg, synth.STREAM_HEADW), (len(positions), heads))
    cache = csa.Cache(4, 8, 128, 64, gu.dev_store(pc.pages, dtype), gu.dev_i32(pc.bt),
                      gu.dev_f32(pc.scales) if pc.scales is not None else None)
    max_elig = max(paging.num_eligible(int(p), 4, 8) for p in positions)
    return cache, gu.dev_i32(np.arange(len(positions))), gu.dev_i32(positions), max_elig, gu.dev_bf16(q), gu.dev_f32(w)


def _outputs(n_q, k):
    return (torch.full((n_q, k), -7, dtype=torch.int32, device="cuda"),
            torch.full((n_q,), -7, dtype=torch.int32, device="cuda"),
            torch.full((n_q, k), -7.0, dtype=torch.float32, device="cuda"))


def _compare(label, args, k):
    cache, qs, qp, max_elig, q, w = args
    n_q = q.shape[0]
    ref = _outputs(n_q, k)
    csa.index_topk(cache, qs, qp, max_elig, q, w, oi.WRELU, k, *ref)
    torch.cuda.synchronize()
    got = _outputs(n_q, k)
    _log(f"noalloc {label}: n_q={n_q} max_elig={max_elig} k={k} "
         f"needs {csa.index_topk_workspace(n_q, max_elig, k, q.shape[1])} B of {csa.NOALLOC_SCRATCH_BYTES}")
    csa.index_topk_noalloc(cache, qs, qp, max_elig, q, w, oi.WRELU, k, *got)
    torch.cuda.synchronize()
    for a, b in zip(got, ref):  # bit patterns (the NaN padding of the scores compares equal this way)
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), \
            f"{label}: csa_index_topk_noalloc differs from csa_index_topk"
    cnt = got[1].cpu().numpy()
    want = [min(k, paging.num_eligible(int(p), 4, 8)) for p in qp.cpu().numpy()]
    assert np.array_equal(cnt, want)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_index_topk_noalloc_matches_workspace_call(dtype):
    long_ = _case(601, np.array([1000000, 700001, 262147, 300]), dtype)
    short = _case(602, np.array([40000 - 997 * i for i in range(32)]), dtype)
    _compare("call 1 (long queries, mark pass)", long_, 512)
    _compare("call 2 (smaller input, 32 queries)", short, 512)
    _compare("call 3 (call 1 again)", long_, 512)


def test_index_topk_noalloc_rejects_oversized_request():
    cache, qs, qp, _, q, w = _case(603, np.array([5000, 3000]), "bf16")
    out, cnt, sc = _outputs(2, 512)
    with pytest.raises(csa.CsaError) as e:
        csa.index_topk_noalloc(cache, qs, qp, 0x7FFFFFFF, q, w, oi.WRELU, 512, out, cnt, sc)
    assert e.value.status == 5
    torch.cuda.synchronize()
    assert torch.all(out == -7), "a rejected call wrote its output"
