"""A small decode step of one CSA layer built from synth draws, run on the GPU library and on the oracle.

Used by the GPU parity tests and by smoke(). Inputs for both sides come from `synth` only; the oracle
side receives host copies of exactly the arrays handed to the GPU.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
import torch

import long_context_compressed_compress_amd as csa
import synth
from oracle import attend as oa, codecs, compress as oc, index as oi, paging, rope as orope
from tests import gpu_util as gu


@dataclass
class StepConfig:
    seed: int = 1
    ratio: int = 4
    lens: List[int] = field(default_factory=lambda: [1024])  # query position p_b = L_b; raw tokens 0..L_b exist
    dim: int = 128
    rope_dims: int = 64
    heads: int = 8
    cache_dtype: str = "f32"   # main cache and window pages
    in_dtype: str = "f32"      # raw tokens / compressor state
    indexer: bool = True
    idx_dim: int = 32
    idx_rope: int = 16
    idx_heads: int = 1
    idx_dtype: str = "f32"
    mode: int = oi.DOT
    k: int = 64
    swa_window: int = 128
    theta: float = 10000.0
    eps: float = 1e-6
    random_gamma: bool = False


def _draw(g, shape, dtype):
    return synth.normal_f32(g, shape) if dtype == "f32" else synth.normal_bf16_bits(g, shape)


def _dev_in(arr, dtype):
    return gu.dev_f32(arr) if dtype == "f32" else gu.dev_bf16(arr)


class Step:
    """Inputs (host + device) of one decode step, with results of each side."""

    def __init__(self, cfg: StepConfig):
        self.cfg = c = cfg
        B = len(c.lens)
        self.B = B
        self.coff = 8 // 4 if c.ratio == 4 else 1
        self.window = 8 if c.ratio == 4 else 128
        n_blocks = max(c.lens) // 256 + 1
        self.n_blocks = n_blocks
        self.n_phys = B * n_blocks + 1
        g_bt = synth.rng(c.seed, synth.STREAM_BT)
        self.bt = synth.random_block_table(g_bt, B, n_blocks, self.n_phys)
        self.rows = max(c.lens) + 1
        # raw tokens (positions 0..L_b of every sequence)
        gk, gl = synth.rng(c.seed, synth.STREAM_KV), synth.rng(c.seed, synth.STREAM_LOGIT)
        self.kv = [_draw(gk, (L + 1, c.dim), c.in_dtype) for L in c.lens]
        self.lg = [_draw(gl, (L + 1, self.coff, c.dim), c.in_dtype) for L in c.lens]
        self.gamma = (synth.uniform_f32(synth.rng(c.seed, 20), (c.dim,), 0.5, 1.5) if c.random_gamma
                      else np.ones(c.dim, np.float32))
        if c.indexer:
            gik, gil = synth.rng(c.seed, synth.STREAM_IDX_KV), synth.rng(c.seed, synth.STREAM_IDX_LOGIT)
            self.ikv = [_draw(gik, (L + 1, c.idx_dim), c.in_dtype) for L in c.lens]
            self.ilg = [_draw(gil, (L + 1, 2, c.idx_dim), c.in_dtype) for L in c.lens]
            self.igamma = np.ones(c.idx_dim, np.float32)
        # window pages: every raw row drawn (iid N(0,1) rows stand for rows rotated upstream)
        gs = synth.rng(c.seed, synth.STREAM_SWA)
        if c.cache_dtype == "fp8":
            self.swa_pages, self.swa_scales = synth.e4m3_rows(gs, self.n_phys * 256, c.dim)
        elif c.cache_dtype == "bf16":
            self.swa_pages, self.swa_scales = synth.normal_bf16_bits(gs, (self.n_phys * 256, c.dim)), None
        else:
            self.swa_pages, self.swa_scales = synth.normal_f32(gs, (self.n_phys * 256, c.dim)), None
        # queries
        gq = synth.rng(c.seed, synth.STREAM_Q)
        qdt = "f32" if c.cache_dtype == "f32" else "bf16"
        self.q_dtype = qdt
        self.q = _draw(gq, (B, c.heads, c.dim), qdt)
        if c.indexer:
            gqi = synth.rng(c.seed, synth.STREAM_QIDX)
            self.qi_dtype = "f32" if c.idx_dtype == "f32" else "bf16"
            self.q_idx = _draw(gqi, (B, c.idx_heads, c.idx_dim), self.qi_dtype)
            self.head_w = (synth.uniform_f32(synth.rng(c.seed, synth.STREAM_HEADW), (B, c.idx_heads))
                           if c.mode == oi.WRELU else None)
        self.q_pos = np.array(c.lens, dtype=np.int32)
        self.q_seq = np.arange(B, dtype=np.int32)
        self.scale = float(1.0 / np.sqrt(c.dim))

    # ------------------------------------------------------------------ GPU side
    def _gpu_cache(self, dim, rdims, dtype):
        E = 256 // self.cfg.ratio
        pages = gu.dev_store(gu.canary((self.n_phys * E, dim), dtype), dtype)
        scales = gu.dev_f32(np.full(self.n_phys * E, np.nan, np.float32)) if dtype == "fp8" else None
        return csa.Cache(self.cfg.ratio, self.window, dim, rdims, pages, gu.dev_i32(self.bt), scales)

    def _gpu_state(self, dim, roles):
        c = self.cfg
        z = (lambda s: torch.zeros(s, dtype=torch.float32, device="cuda")) if c.in_dtype == "f32" else \
            (lambda s: torch.zeros(s, dtype=torch.bfloat16, device="cuda"))
        return csa.Raw(dim, roles, z((self.n_phys * 256, dim)), gu.dev_i32(self.bt), z((self.n_phys * 256, roles, dim)))

    def _gpu_compress(self, cache, state, kv, lg, gamma, rope_cs, lo, hi):
        """Insert positions lo[b] .. hi[b]-1 of every sequence."""
        c = self.cfg
        n = [h - l for l, h in zip(lo, hi)]
        cu = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
        kvn = np.concatenate([kv[b][lo[b]:hi[b]] for b in range(self.B)])
        lgn = np.concatenate([lg[b][lo[b]:hi[b]] for b in range(self.B)])
        mx = max(n)
        bound = (mx + c.ratio - 1) // c.ratio
        slots = torch.full((self.B, max(bound, 1)), -7, dtype=torch.int32, device="cuda")
        cnt = torch.full((self.B,), -7, dtype=torch.int32, device="cuda")
        csa.compress_insert(cache, state, gu.dev_i32(lo), gu.dev_i32(cu), _dev_in(kvn, c.in_dtype),
                            _dev_in(lgn, c.in_dtype), gu.dev_f32(gamma), c.eps, rope_cs, mx, slots, cnt)
        return slots, cnt

    def run_gpu(self):
        c = self.cfg
        self.g_rope = csa.rope_table(self.rows, max(c.rope_dims, 2), c.theta)
        self.g_cache = self._gpu_cache(c.dim, c.rope_dims, c.cache_dtype)
        self.g_state = self._gpu_state(c.dim, self.coff)
        zeros = [0] * self.B
        lens = list(c.lens)
        ends = [L + 1 for L in lens]
        self.g_prefill = self._gpu_compress(self.g_cache, self.g_state, self.kv, self.lg, self.gamma, self.g_rope, zeros, lens)
        self.g_decode = self._gpu_compress(self.g_cache, self.g_state, self.kv, self.lg, self.gamma, self.g_rope, lens, ends)
        swa_pages = gu.dev_store(self.swa_pages, c.cache_dtype)
        swa_sc = gu.dev_f32(self.swa_scales) if self.swa_scales is not None else None
        self.g_swa = csa.Raw(c.dim, 0, swa_pages, gu.dev_i32(self.bt), None, swa_sc)
        q_seq, q_pos = gu.dev_i32(self.q_seq), gu.dev_i32(self.q_pos)
        max_elig = max(paging.num_eligible(int(p), c.ratio, self.window) for p in self.q_pos)
        self.max_elig = max_elig
        self.g_topk = None
        if c.indexer:
            self.g_irope = csa.rope_table(self.rows, c.idx_rope, c.theta)
            self.g_icache = self._gpu_cache(c.idx_dim, c.idx_rope, c.idx_dtype)
            self.g_istate = self._gpu_state(c.idx_dim, 2)
            self._gpu_compress(self.g_icache, self.g_istate, self.ikv, self.ilg, self.igamma, self.g_irope, zeros, lens)
            self._gpu_compress(self.g_icache, self.g_istate, self.ikv, self.ilg, self.igamma, self.g_irope, lens, ends)
            self.g_topk = torch.full((self.B, c.k), -7, dtype=torch.int32, device="cuda")
            self.g_cnt = torch.full((self.B,), -7, dtype=torch.int32, device="cuda")
            self.g_tsc = torch.full((self.B, c.k), -7.0, dtype=torch.float32, device="cuda")
            hw = gu.dev_f32(self.head_w) if self.head_w is not None else None
            csa.index_topk(self.g_icache, q_seq, q_pos, max_elig, _dev_in(self.q_idx, self.qi_dtype), hw, c.mode, c.k,
                           self.g_topk, self.g_cnt, self.g_tsc)
        self.g_out = torch.full((self.B, c.heads, c.dim), -7.0, dtype=torch.float32, device="cuda")
        self.g_lse = torch.full((self.B, c.heads), -7.0, dtype=torch.float32, device="cuda")
        csa.attend(self.g_cache, self.g_swa, c.swa_window, q_seq, q_pos, _dev_in(self.q, self.q_dtype), self.g_topk,
                   max_elig, self.scale, True, self.g_rope, self.g_out, self.g_lse)
        torch.cuda.synchronize()

    # ------------------------------------------------------------------ oracle side
    def _o_cache(self, dim, rdims, dtype):
        E = 256 // self.cfg.ratio
        return oc.Cache(self.cfg.ratio, self.window, dim, rdims, dtype, gu.canary((self.n_phys * E, dim), dtype),
                        np.full(self.n_phys * E, np.nan, np.float32) if dtype == "fp8" else None, self.bt.copy())

    def _o_state(self, dim, roles):
        c = self.cfg
        if c.in_dtype == "f32":
            kv = np.zeros((self.n_phys * 256, dim), np.float32)
            lg = np.zeros((self.n_phys * 256, roles, dim), np.float32)
        else:
            kv = np.zeros((self.n_phys * 256, dim), np.uint16)
            lg = np.zeros((self.n_phys * 256, roles, dim), np.uint16)
        return oc.Raw(c.in_dtype, dim, roles, kv, lg, None, self.bt.copy())

    def _o_compress(self, cache, state, kv, lg, gamma, table, lo, hi):
        c = self.cfg
        n = [h - l for l, h in zip(lo, hi)]
        cu = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
        kvn = np.concatenate([kv[b][lo[b]:hi[b]] for b in range(self.B)])
        lgn = np.concatenate([lg[b][lo[b]:hi[b]] for b in range(self.B)])
        bound = max((max(n) + c.ratio - 1) // c.ratio, 1)
        return oc.compress_insert(cache, state, np.array(lo), cu, kvn, lgn, gamma, c.eps, table, bound)

    def run_oracle_compress(self):
        c = self.cfg
        self.o_rope = orope.rope_table(self.rows, c.rope_dims, c.theta)
        self.o_cache = self._o_cache(c.dim, c.rope_dims, c.cache_dtype)
        self.o_state = self._o_state(c.dim, self.coff)
        zeros, lens = [0] * self.B, list(c.lens)
        ends = [L + 1 for L in lens]
        self.o_prefill = self._o_compress(self.o_cache, self.o_state, self.kv, self.lg, self.gamma, self.o_rope, zeros, lens)
        self.o_decode = self._o_compress(self.o_cache, self.o_state, self.kv, self.lg, self.gamma, self.o_rope, lens, ends)
        if c.indexer:
            self.o_irope = orope.rope_table(self.rows, c.idx_rope, c.theta)
            self.o_icache = self._o_cache(c.idx_dim, c.idx_rope, c.idx_dtype)
            self.o_istate = self._o_state(c.idx_dim, 2)
            self._o_compress(self.o_icache, self.o_istate, self.ikv, self.ilg, self.igamma, self.o_irope, zeros, lens)
            self._o_compress(self.o_icache, self.o_istate, self.ikv, self.ilg, self.igamma, self.o_irope, lens, ends)

    def run_oracle(self):
        """The whole step on the oracle from the raw inputs: compress, index (if any), attend with inverse RoPE."""
        c = self.cfg
        self.run_oracle_compress()
        qf = self.q_f64(self.q, self.q_dtype)
        self.o_topk = None
        if c.indexer:
            qi = self.q_f64(self.q_idx, self.qi_dtype)
            self.o_topk, self.o_cnt, self.o_tsc = oi.index_topk(self.o_icache, self.q_seq, self.q_pos, qi, self.head_w,
                                                               c.mode, c.k)
        self.o_out, self.o_lse = oa.attend(self.o_cache, self.oracle_swa(), c.swa_window, self.q_seq, self.q_pos, qf,
                                           self.o_topk, self.scale, True, self.o_rope)

    def oracle_swa(self) -> oc.Raw:
        return oc.Raw(self.cfg.cache_dtype, self.cfg.dim, 0, self.swa_pages, None, self.swa_scales, self.bt.copy())

    def q_f64(self, arr, dtype):
        return codecs.load_rows(arr, "f32" if dtype == "f32" else "bf16")

    # ------------------------------------------------------------------ unrounded oracle rows
    def run_oracle_unrounded(self):
        """The oracle's compressed rows before storage rounding (an fp32 cache fed the same raw tokens)."""
        c = self.cfg
        zeros, lens = [0] * self.B, list(c.lens)
        ends = [L + 1 for L in lens]
        self.o_cache32 = self._o_cache(c.dim, c.rope_dims, "f32")
        st = self._o_state(c.dim, self.coff)
        self._o_compress(self.o_cache32, st, self.kv, self.lg, self.gamma, self.o_rope, zeros, lens)
        self._o_compress(self.o_cache32, st, self.kv, self.lg, self.gamma, self.o_rope, lens, ends)
        if c.indexer:
            self.o_icache32 = self._o_cache(c.idx_dim, c.idx_rope, "f32")
            st = self._o_state(c.idx_dim, 2)
            self._o_compress(self.o_icache32, st, self.ikv, self.ilg, self.igamma, self.o_irope, zeros, lens)
            self._o_compress(self.o_icache32, st, self.ikv, self.ilg, self.igamma, self.o_irope, lens, ends)

    def gpu_attend_with(self, topk: np.ndarray) -> np.ndarray:
        """GPU attention of every query over a given top-k list (the oracle's), on the GPU-built caches."""
        c = self.cfg
        out = torch.full((self.B, c.heads, c.dim), -7.0, dtype=torch.float32, device="cuda")
        lse = torch.full((self.B, c.heads), -7.0, dtype=torch.float32, device="cuda")
        csa.attend(self.g_cache, self.g_swa, c.swa_window, gu.dev_i32(self.q_seq), gu.dev_i32(self.q_pos),
                   _dev_in(self.q, self.q_dtype), gu.dev_i32(topk), self.max_elig, self.scale, True, self.g_rope, out,
                   lse)
        torch.cuda.synchronize()
        return out.cpu().numpy(), lse.cpu().numpy()


def _stored(cache, rows):
    return cache.pages[rows], (cache.scales[rows] if cache.scales is not None else None)


def verify(st: Step, out_tol: float, lse_tol: float, log=None) -> dict:
    """Check a whole decode step of the GPU library against the oracle run from the same raw tokens.

    * entry counts and slots of both compress calls: bit-exact;
    * every eligible row of the main and indexer caches: within the rounding-aware element bound of
      gpu_util.stored_elem_bound (codes equal except where the unrounded value sits at a rounding midpoint);
    * top-k sets: equal to the oracle's except for swaps certified as near-ties, where each score may differ
      by the fp32 accumulation bound plus the storage bound of the indexer rows (any other difference fails);
    * attention output of every sequence within out_tol (max over rows of max|d| / max|ref|) and its lse:
      sequences whose GPU set equals the oracle's are compared as they came out of the GPU chain; a sequence
      whose set differs by certified swaps is re-attended on the GPU over the oracle's set (an oracle
      output fed to the GPU, never the reverse) and compared the same way.
    """
    c = st.cfg
    log = log or (lambda m: None)
    res = {"swaps": 0, "reattended": []}
    window = st.window
    for (gs, gc), (os_, oc_) in ((st.g_prefill, st.o_prefill), (st.g_decode, st.o_decode)):
        assert np.array_equal(gc.cpu().numpy(), oc_)
        assert np.array_equal(gs.cpu().numpy()[:, : os_.shape[1]], os_[:, : gs.shape[1]])
    st.run_oracle_unrounded()
    gmain = (gu.host_store(st.g_cache.pages), st.g_cache.scales.cpu().numpy() if st.g_cache.scales is not None else None)
    if c.indexer:
        gidx = (gu.host_store(st.g_icache.pages),
                st.g_icache.scales.cpu().numpy() if st.g_icache.scales is not None else None)
    gi = st.g_topk.cpu().numpy() if c.indexer else None
    gcnt = st.g_cnt.cpu().numpy() if c.indexer else None
    g_out = st.g_out.cpu().numpy()
    g_lse = st.g_lse.cpu().numpy()
    differing = []
    for b in range(st.B):
        p = int(st.q_pos[b])
        n = paging.num_eligible(p, c.ratio, window)
        rows = np.array([paging.entry_slot(st.bt[b], i, c.ratio) for i in range(n)], np.int64)
        if n:
            rp, rs = _stored(st.o_cache, rows)
            gu.stored_elem_bound(c.cache_dtype, st.o_cache32.pages[rows], rp, rs, gmain[0][rows],
                                 None if gmain[1] is None else gmain[1][rows])
        if not c.indexer:
            continue
        if n:
            rp, rs = _stored(st.o_icache, rows)
            u = gu.stored_elem_bound(c.idx_dtype, st.o_icache32.pages[rows], rp, rs, gidx[0][rows],
                                     None if gidx[1] is None else gidx[1][rows])
            keys = codecs.load_rows(rp, c.idx_dtype, rs)
        else:
            u = keys = np.zeros((0, c.idx_dim))
        qi = st.q_f64(st.q_idx, st.qi_dtype)[b]
        w = None if st.head_w is None else st.head_w[b].astype(np.float64)
        s = oi.scores(keys, qi, w, c.mode)
        delta = gu.wrelu_score_delta(keys, u, qi, w, c.mode, c.idx_dim, c.idx_heads)
        swaps = gu.check_topk_near_ties(gi[b], gcnt[b], s, c.k, delta)
        res["swaps"] += swaps
        if not np.array_equal(gi[b], st.o_topk[b]):
            differing.append(b)
    res["attend_err"] = gu.rowwise_rel_err(np.delete(g_out, differing, axis=0), np.delete(st.o_out, differing, axis=0)) \
        if len(differing) < st.B else 0.0
    lse_ok = [b for b in range(st.B) if b not in differing]
    assert np.allclose(g_lse[lse_ok], st.o_lse[lse_ok], rtol=0, atol=lse_tol), "lse differs from the oracle's"
    if differing:
        re, re_lse = st.gpu_attend_with(st.o_topk)
        res["reattended"] = differing
        res["reattend_err"] = gu.rowwise_rel_err(re[differing], st.o_out[differing])
        assert res["reattend_err"] <= out_tol, res
        assert np.allclose(re_lse[differing], st.o_lse[differing], rtol=0, atol=lse_tol)
    log(f"chain: {res}")
    assert res["attend_err"] <= out_tol, res
    return res
