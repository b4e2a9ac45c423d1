"""The decode step captured in a HIP graph.

* test_partition_graph_matches_oracle: the whole decode step of one layer, the query / window-key preparation
  (csa_prepare_qk) included, captured with the two-stream partition of [P1] "GPU Compute Saturation" and
  [P2] "3.2 內核": on a c4a layer the indexer pipeline (indexer compress_insert, score, select) runs on a second
  stream beside main compress_insert + window insert; on a c128a layer main compress_insert runs beside the
  window insert; attention joins both. Inputs come from synth; every replay (after eager work elsewhere and with
  all outputs and written slots poisoned) is checked against the oracle run end to end with the rules of
  tests/chain.verify.
* test_graph_replay_matches_eager: the benchmark's capture (main compress on the side stream, bf16 or MXFP4
  indexer cache) replays to the eager result bit for bit.
* test_fused_layers_graph_replay_matches_eager: the fused decode step (both compresses inside the index-score
  launch) of two layers in one graph replays to the eager result bit for bit.

Shapes are the real ones (64 heads x K=V 512 bf16, indexer 64 heads x 128 WRELU in bf16 or MXFP4, top-512 +
window 128) at a few short contexts. Each replay runs after eager work of its own and a synchronisation; every replay's top-k lists,
attention output and written cache rows must equal the eager step's bit for bit (every kernel is
deterministic), and the eager step itself is checked against the oracle by the parity tests.
"""
import math

import numpy as np
import pytest
import torch

import long_context_compressed_compress_amd as csa
import synth
from oracle import index as oi, paging
from tests.chain import Step, StepConfig, verify

pytestmark = pytest.mark.gpu

B, H, D, R = 6, 64, 512, 64
H_IDX, D_IDX = 64, 128
K_TOP, SWA = 512, 128


def _log(msg):
    print(msg, flush=True)


class _Layer:
    def __init__(self, seed, fp4_idx=False):
        dev = "cuda"
        g = torch.Generator(device=dev)
        g.manual_seed(seed)
        self.lens = [int(x) for x in synth.lengths_uniform(synth.rng(seed, synth.STREAM_LEN), B, 9000, 20000)]
        nb = [L // 256 + 1 for L in self.lens]
        stride = max(nb)
        n_phys = sum(nb) + 5
        perm = torch.randperm(n_phys, generator=torch.Generator().manual_seed(seed))[: sum(nb)].to(torch.int32)
        bt = torch.full((B, stride), -1, dtype=torch.int32)
        o = 0
        for b, n in enumerate(nb):
            bt[b, :n] = perm[o:o + n]
            o += n
        self.bt = bt.to(dev)
        tail = torch.full((B, stride), -1, dtype=torch.int32)
        for b, L in enumerate(self.lens):
            tail[b, L // 256 - 1], tail[b, L // 256] = 2 * b, 2 * b + 1
        self.tail = tail.to(dev)
        bf = torch.bfloat16
        self.cache = csa.Cache(4, 8, D, R, torch.zeros((n_phys * 64, D), dtype=bf, device=dev), self.bt)
        if fp4_idx:  # MXFP4 indexer cache: packed codes and E8M0 block exponents
            ipages = torch.zeros((n_phys * 64, D_IDX // 2), dtype=torch.uint8, device=dev)
            self.iscales = torch.zeros((n_phys * 64, D_IDX // 32), dtype=torch.uint8, device=dev)
            self.icache = csa.Cache(4, 8, D_IDX, R, ipages.view(torch.float4_e2m1fn_x2), self.bt, self.iscales)
        else:
            ipages = torch.zeros((n_phys * 64, D_IDX), dtype=bf, device=dev)
            self.iscales = torch.zeros((1,), dtype=torch.uint8, device=dev)  # unused
            self.icache = csa.Cache(4, 8, D_IDX, R, ipages, self.bt)
        self.ipages_u8 = ipages.view(torch.uint8)
        z = lambda *s: torch.zeros(s, dtype=bf, device=dev)
        self.state = csa.Raw(D, 2, z(2 * B * 256, D), self.tail, z(2 * B * 256, 2, D))
        self.istate = csa.Raw(D_IDX, 2, z(2 * B * 256, D_IDX), self.tail, z(2 * B * 256, 2, D_IDX))
        self.swa = csa.Raw(D, 0, torch.randn((2 * B * 256, D), generator=g, device=dev, dtype=bf), self.tail)
        self.rope = csa.rope_table(max(self.lens) + 2, R)
        self.gamma, self.igamma = torch.ones(D, device=dev), torch.ones(D_IDX, device=dev)
        r = lambda *s: torch.randn(s, generator=g, device=dev, dtype=bf)
        n = self.lens
        cu = torch.tensor(np.concatenate([[0], np.cumsum(n)]), dtype=torch.int32, device=dev)
        start = torch.zeros(B, dtype=torch.int32, device=dev)
        csa.compress_insert(self.cache, self.state, start, cu, r(sum(n), D), r(sum(n), 2, D), self.gamma, 1e-6,
                            self.rope, max(n))
        csa.compress_insert(self.icache, self.istate, start, cu, r(sum(n), D_IDX), r(sum(n), 2, D_IDX), self.igamma,
                            1e-6, self.rope, max(n))
        self.pos = torch.tensor(self.lens, dtype=torch.int32, device=dev)
        self.seq = torch.arange(B, dtype=torch.int32, device=dev)
        self.cu1 = torch.arange(B + 1, dtype=torch.int32, device=dev)
        self.kv1, self.lg1, self.ikv1, self.ilg1 = r(B, D), r(B, 2, D), r(B, D_IDX), r(B, 2, D_IDX)
        self.q, self.q_idx = r(B, H, D), r(B, H_IDX, D_IDX)
        self.head_w = torch.rand((B, H_IDX), generator=g, device=dev)
        self.max_elig = max(csa.num_eligible(L, 4, 8) for L in self.lens)
        self.ws = csa.index_workspace(B, self.max_elig, K_TOP, H_IDX)
        self.att_ws = torch.empty(max(csa.attend_workspace(B, H, D, K_TOP + SWA), 1), dtype=torch.uint8, device=dev)
        self.topk = torch.full((B, K_TOP), -7, dtype=torch.int32, device=dev)
        self.out = torch.full((B, H, D), -7.0, device=dev)
        self.lse = torch.full((B, H), -7.0, device=dev)
        torch.cuda.synchronize()

    def step(self, side):
        cur = torch.cuda.current_stream()
        side.wait_stream(cur)
        with torch.cuda.stream(side):
            csa.compress_insert(self.cache, self.state, self.pos, self.cu1, self.kv1, self.lg1, self.gamma, 1e-6,
                                self.rope, 1)
        csa.compress_insert(self.icache, self.istate, self.pos, self.cu1, self.ikv1, self.ilg1, self.igamma, 1e-6,
                            self.rope, 1)
        csa.index_score(self.icache, self.seq, self.pos, self.max_elig, self.q_idx, self.head_w, csa.SCORE_WRELU,
                        K_TOP, self.ws)
        csa.index_select(self.icache, self.seq, self.pos, self.max_elig, K_TOP, self.topk, self.ws)
        cur.wait_stream(side)
        csa.attend(self.cache, self.swa, SWA, self.seq, self.pos, self.q, self.topk, self.max_elig,
                   1.0 / math.sqrt(D), True, self.rope, self.out, self.lse, workspace=self.att_ws)

    def step_fused(self):
        """The step with both caches' compress inside the index-score launch, every call on the current stream."""
        csa.compress_index_score(self.cache, self.state, self.kv1, self.lg1, self.gamma, self.rope, self.icache,
                                 self.istate, self.ikv1, self.ilg1, self.igamma, self.rope, self.pos, self.cu1, 1e-6,
                                 self.seq, self.pos, self.max_elig, self.q_idx, self.head_w, csa.SCORE_WRELU, K_TOP,
                                 self.ws)
        csa.index_select(self.icache, self.seq, self.pos, self.max_elig, K_TOP, self.topk, self.ws)
        csa.attend(self.cache, self.swa, SWA, self.seq, self.pos, self.q, self.topk, self.max_elig,
                   1.0 / math.sqrt(D), True, self.rope, self.out, self.lse, workspace=self.att_ws)

    def results(self):
        torch.cuda.synchronize()
        return [t.clone() for t in (self.topk, self.out, self.lse, self.cache.pages, self.ipages_u8, self.iscales,
                                    self.state.kv_pages, self.istate.kv_pages)]

    def poison(self):
        """Overwrite every output and every slot the step writes, so a replay that skips work shows."""
        self.topk.fill_(-7)
        self.out.fill_(-7.0)
        self.lse.fill_(-7.0)
        for L, b in zip(self.lens, range(B)):
            if L % 4 == 3:  # the decode token completes entry (L - 7) / 4
                i = (L - 7) // 4
                row = int(self.bt[b, i // 64]) * 64 + i % 64
                self.cache.pages[row].fill_(float("nan"))
                self.ipages_u8[row].fill_(0xA5)
                if self.iscales.shape[0] > row:
                    self.iscales[row].fill_(0xA5)


@pytest.mark.parametrize("fp4_idx", [False, True])
def test_graph_replay_matches_eager(fp4_idx):
    torch.cuda.synchronize()
    ly = _Layer(81, fp4_idx)
    other = _Layer(82, fp4_idx)
    side = torch.cuda.Stream()
    _log(f"graph replay: contexts {ly.lens}, fp4 indexer cache {fp4_idx}")
    ly.step(side)
    ref = ly.results()
    assert int((ref[0] >= 0).sum()) == B * K_TOP
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ly.step(side)
    torch.cuda.synchronize()
    for rep in range(3):
        other.step(side)          # eager work of the program between replays, on other buffers
        ly.poison()
        torch.cuda.synchronize()
        g.replay()
        got = ly.results()
        for name, a, b in zip(["topk", "out", "lse", "pages", "idx pages", "idx scales", "state", "idx state"], got, ref):
            assert torch.equal(a.view(torch.uint8) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.uint8) if b.dtype == torch.bfloat16 else b), f"replay {rep}: {name} differs"
        _log(f"replay {rep}: identical to the eager step")


NAMES = ["topk", "out", "lse", "pages", "idx pages", "idx scales", "state", "idx state"]


def _same(a, b):
    return torch.equal(a.view(torch.uint8) if a.dtype == torch.bfloat16 else a,
                       b.view(torch.uint8) if b.dtype == torch.bfloat16 else b)


@pytest.mark.parametrize("fp4_idx", [False, True])
def test_fused_layers_graph_replay_matches_eager(fp4_idx):
    """One graph holding the fused step (csa_compress_index_score, select, attention) of two layers in order, as the
    benchmark's multi-layer graphs do: every replay equals the eager fused step, which equals the unfused step."""
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    a, b = _Layer(83, fp4_idx), _Layer(84, fp4_idx)
    a2 = _Layer(83, fp4_idx)  # the same layer again, stepped with the separate calls
    other = _Layer(85, fp4_idx)
    _log(f"fused layers graph: contexts {a.lens} / {b.lens}, fp4 indexer cache {fp4_idx}")
    a.step_fused()
    b.step_fused()
    ref = [a.results(), b.results()]
    a2.step(side)
    for name, x, y in zip(NAMES, a2.results(), ref[0]):
        assert _same(x, y), f"fused eager step differs from the separate calls: {name}"
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        a.step_fused()
        b.step_fused()
    torch.cuda.synchronize()
    for rep in range(3):
        other.step_fused()        # eager work of the program between replays, on other buffers
        a.poison()
        b.poison()
        torch.cuda.synchronize()
        g.replay()
        for ly, r in zip((a, b), ref):
            for name, x, y in zip(NAMES, ly.results(), r):
                assert _same(x, y), f"replay {rep}: {name} differs"
        _log(f"replay {rep}: both layers identical to the eager fused step")


PARTITION_CASES = [
    ("c4a bf16", dict(ratio=4, lens=[3003, 4093, 811], cache_dtype="bf16", indexer=True, idx_dtype="bf16"), 2e-3),
    ("c4a fp8", dict(ratio=4, lens=[2999, 1603], cache_dtype="fp8", indexer=True, idx_dtype="fp8"), 5e-2),
    ("c128a bf16 dense", dict(ratio=128, lens=[4095, 3000, 511], cache_dtype="bf16", indexer=False), 2e-3),
]


def _poison(st: Step):
    """Overwrite every output of the step and every slot it writes, so a replay that skips work shows."""
    c = st.cfg
    st.g_out.fill_(-7.0)
    st.g_lse.fill_(-7.0)
    st.g_q.fill_(float("nan"))
    st.dec_args["slots"].fill_(-7)
    st.dec_args["cnt"].fill_(-7)
    pages = st.g_swa.kv_pages.view(torch.uint8).view(st.g_swa.kv_pages.shape[0], -1)
    for b, L in enumerate(c.lens):
        pages[paging.raw_slot(st.bt[b], L)].fill_(0x7F)  # NaN bf16 / fp8 bytes
        if (L + 1 - st.window) % c.ratio == 0:          # the decode token completes entry (L + 1 - w) / ratio
            row = paging.entry_slot(st.bt[b], (L + 1 - st.window) // c.ratio, c.ratio)
            st.g_cache.pages.view(torch.uint8).view(st.g_cache.pages.shape[0], -1)[row].fill_(0x7F)
            if c.indexer:
                st.g_icache.pages.view(torch.uint8).view(st.g_icache.pages.shape[0], -1)[row].fill_(0x7F)
    if c.indexer:
        st.g_topk.fill_(-7)
        st.g_cnt.fill_(-7)
        st.idec_args["slots"].fill_(-7)


@pytest.mark.parametrize("label,kw,tol", PARTITION_CASES, ids=[c[0] for c in PARTITION_CASES])
def test_partition_graph_matches_oracle(label, kw, tol):
    _log(f"partition graph: {label}")
    base = dict(seed=90, dim=512, rope_dims=64, heads=64, in_dtype="bf16", idx_dim=128, idx_rope=64, idx_heads=64,
                mode=oi.WRELU, k=512, prepare=True)
    st = Step(StepConfig(**{**base, **kw}))
    other = Step(StepConfig(**{**base, **kw, "seed": 91, "lens": [1500, 900]}))
    st.gpu_setup()
    other.gpu_setup()
    st.run_oracle()
    side = torch.cuda.Stream()
    st.gpu_decode_step(side)  # eager warm-up of exactly the captured work
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st.gpu_decode_step(side)
    torch.cuda.synchronize()
    for rep in range(3):
        other.gpu_decode_step(side)   # eager work of the program between replays, on other buffers
        _poison(st)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        res = verify(st, tol, 1e-4, log=_log)
        _log(f"{label} replay {rep}: matches the oracle (swaps {res['swaps']}, attention err {res['attend_err']:.2e})")
