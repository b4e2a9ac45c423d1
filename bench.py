#!/usr/bin/env python3
"""Decode-step benchmark of one c4a compressed-sparse-attention layer on one MI355X.

Workload (the 128K bf16 decode configuration): batch 32, per-sequence context L_b ~ U{98304..131072}
with the query at position L_b; main cache bf16, one shared K=V head of dim 512 with RoPE on the last
64 dims; indexer cache bf16 of dim 128 (RoPE 64), 64 indexer heads with weights ~U(0,1),
score = sum_h w_h ReLU(q_h . k); top-512 compressed entries + 128-token raw window; 64 query heads;
256-position blocks at random physical pages. Inputs are synthetic (seeded), resident in HBM.

A step is one pass of the whole path for the batch: compress_insert of the decode token into the main
and the indexer cache (one paired call), index score, top-k select, attention with fused inverse RoPE. Steps rotate over
--layers independently built layer caches (placed at random in their own pools) so repeated steps do
not run out of the 256 MB Infinity Cache.

Prints one JSON line (see README of the driver contract): value = queries/s of the whole step.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "decode queries/s and achieved HBM GB/s (% peak) for c4a/c128a CSA at 128K-1M ctx"

B, H, D, R = 32, 64, 512, 64
H_IDX, D_IDX, R_IDX = 64, 128, 64
K_TOP, SWA = 512, 128
LEN_LO, LEN_HI = 98304, 131072
CONFIG_ID = 3

# HBM bytes per launch of the index score kernel on the 128K bf16 (c3), 1M fp8 (c4) and 1M fp8 with MXFP4 indexer
# (c4f) decode workloads, from one
# FETCH_SIZE and one WRITE_SIZE counter run (FETCH_SIZE x 2.0, WRITE_SIZE x 1.0 as calibrated on a 1 GiB device
# copy). The figures hold only for the kernel source they were measured on; for any other source the traffic is
# reported as unknown.
SCORE_TRAFFIC = {"source": "long_context_compressed_compress_amd/csrc/index_topk.hip",
                 "sha256": "d4353ac71a5daed1db3ffcbd72964d1a3d37b3c386e35fc4201d30cfbc191e4c",
                 "bytes": {"c3": 245275871, "c4": 143762077, "c4f": 76344249}}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def score_traffic(workload):
    with open(os.path.join(ROOT, SCORE_TRAFFIC["source"]), "rb") as f:
        same = hashlib.sha256(f.read()).hexdigest() == SCORE_TRAFFIC["sha256"]
    return SCORE_TRAFFIC["bytes"].get(workload) if same else None


def workload_lengths():
    import synth
    return synth.lengths_uniform(synth.rng(CONFIG_ID, synth.STREAM_LEN), B, LEN_LO, LEN_HI)


# ------------------------------------------------------------------ GPU workload
class Layer:
    """Caches, state, window pages and per-step inputs of one layer, built on the device."""

    def __init__(self, l, lens, torch, csa, rope_main, rope_idx):
        self.l = l
        dev = "cuda"
        gen = torch.Generator(device=dev)
        gen.manual_seed(1000 * CONFIG_ID + 100 * (l + 1))
        cpu_gen = torch.Generator()
        cpu_gen.manual_seed(1000 * CONFIG_ID + 7 + 100 * (l + 1))
        n_blocks = [int(L) // 256 + 1 for L in lens]
        self.bt_stride = max(n_blocks)
        need = sum(n_blocks)
        n_phys = int(math.ceil(1.25 * need))
        perm = torch.randperm(n_phys, generator=cpu_gen)[:need].to(torch.int32)
        bt = torch.full((B, self.bt_stride), -1, dtype=torch.int32)
        o = 0
        for b, nb in enumerate(n_blocks):
            bt[b, :nb] = perm[o:o + nb]
            o += nb
        self.bt = bt.to(dev)
        # state / window pages: only the last two logical blocks of each sequence are mapped
        tail = torch.full((B, self.bt_stride), -1, dtype=torch.int32)
        tperm = torch.randperm(2 * B, generator=cpu_gen).to(torch.int32)
        for b, L in enumerate(lens):
            last = int(L) // 256
            tail[b, last - 1] = tperm[2 * b]
            tail[b, last] = tperm[2 * b + 1]
        self.tail_bt = tail.to(dev)
        bf = torch.bfloat16
        self.cache = csa.Cache(4, 8, D, R, torch.empty((n_phys * 64, D), dtype=bf, device=dev), self.bt)
        self.icache = csa.Cache(4, 8, D_IDX, R_IDX, torch.empty((n_phys * 64, D_IDX), dtype=bf, device=dev), self.bt)
        self.state = csa.Raw(D, 2, torch.zeros((2 * B * 256, D), dtype=bf, device=dev), self.tail_bt,
                             torch.zeros((2 * B * 256, 2, D), dtype=bf, device=dev))
        self.istate = csa.Raw(D_IDX, 2, torch.zeros((2 * B * 256, D_IDX), dtype=bf, device=dev), self.tail_bt,
                              torch.zeros((2 * B * 256, 2, D_IDX), dtype=bf, device=dev))
        self.swa = csa.Raw(D, 0, torch.randn((2 * B * 256, D), generator=gen, device=dev).to(bf), self.tail_bt)
        self.gamma = torch.ones(D, device=dev)
        self.igamma = torch.ones(D_IDX, device=dev)
        # prefix build: all tokens 0..L_b-1, four sequences per call (the others append nothing)
        lens_t = [int(L) for L in lens]
        for c0 in range(0, B, 4):
            n = [lens_t[b] if c0 <= b < c0 + 4 else 0 for b in range(B)]
            cu = torch.tensor(np.concatenate([[0], np.cumsum(n)]), dtype=torch.int32, device=dev)
            start = torch.zeros(B, dtype=torch.int32, device=dev)
            tot = int(sum(n))
            kv = torch.randn((tot, D), generator=gen, device=dev).to(bf)
            lg = torch.randn((tot, 2, D), generator=gen, device=dev).to(bf)
            csa.compress_insert(self.cache, self.state, start, cu, kv, lg, self.gamma, 1e-6, rope_main, max(n))
            del kv, lg
            ikv = torch.randn((tot, D_IDX), generator=gen, device=dev).to(bf)
            ilg = torch.randn((tot, 2, D_IDX), generator=gen, device=dev).to(bf)
            csa.compress_insert(self.icache, self.istate, start, cu, ikv, ilg, self.igamma, 1e-6, rope_idx, max(n))
            del ikv, ilg
        # decode-step inputs
        self.pos = torch.tensor(lens_t, dtype=torch.int32, device=dev)
        self.seq = torch.arange(B, dtype=torch.int32, device=dev)
        self.cu1 = torch.arange(B + 1, dtype=torch.int32, device=dev)
        self.kv1 = torch.randn((B, D), generator=gen, device=dev).to(bf)
        self.lg1 = torch.randn((B, 2, D), generator=gen, device=dev).to(bf)
        self.ikv1 = torch.randn((B, D_IDX), generator=gen, device=dev).to(bf)
        self.ilg1 = torch.randn((B, 2, D_IDX), generator=gen, device=dev).to(bf)
        self.q = torch.randn((B, H, D), generator=gen, device=dev).to(bf)
        self.q_idx = torch.randn((B, H_IDX, D_IDX), generator=gen, device=dev).to(bf)
        self.head_w = torch.rand((B, H_IDX), generator=gen, device=dev)


def algorithmic_bytes(lens):
    """Bytes the method must move per step: every eligible indexer key once, q_idx and head weights per query; the
    top-k indices; the selected entries and window rows once, q and the fp32 output per query; the decode-step
    compression's raw rows and new entries."""
    from long_context_compressed_compress_amd import num_eligible
    score = sel = att = comp = 0
    for L in lens:
        n = num_eligible(int(L), 4, 8)
        score += n * D_IDX * 2 + H_IDX * D_IDX * 2 + 4 * H_IDX          # eligible indexer keys + q_idx + weights
        sel += 4 * K_TOP                                               # top-k indices out
        att += min(K_TOP, n) * D * 2 + min(SWA, int(L) + 1) * D * 2 + 4 * K_TOP + H * D * 2 + 4 * H * D
        new = 1 if int(L) % 4 == 3 else 0                              # decode token completes an entry?
        comp += 3 * (D + D_IDX) * 2 * 2 + new * (7 * 3 * (D + D_IDX) * 2 + (D + D_IDX) * 2)
    return {"score": score, "select": sel, "attend": att, "compress": comp}


def time_steps(torch, step, layers, steps, warmup, n_stages):
    """Warm up, then time `steps` calls of step(layer, events) with HIP events on torch's current stream (the
    stream every library call runs on). Returns (total ms, mean ms of each stage between consecutive events)."""
    for i in range(warmup):
        step(layers[i % len(layers)], None)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n_stages + 1)] for _ in range(steps)]
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for i in range(steps):
        step(layers[i % len(layers)], evs[i])
    t1.record()
    torch.cuda.synchronize()
    stage = [float(np.mean([e[j].elapsed_time(e[j + 1]) for e in evs])) for j in range(n_stages)]
    return t0.elapsed_time(t1), stage


EAGER_ONLY = False
STEP_MODES = {"eager": "eager launches on one stream with an event between stages",
              "graph": "one HIP graph per layer, every call on one stream",
              "graph_2stream": "one HIP graph per layer, main-cache compress_insert on a second stream beside the "
                               "indexer pipeline",
              "graph_partition": "one HIP graph per layer, the indexer pipeline (its compress_insert, score, select) on "
                                 "a second stream beside the main-cache compress_insert",
              "graph_fused": "one HIP graph per layer, every call on one stream, both caches' compress_insert inside "
                             "the index-score launch (csa_compress_index_score)",
              "graph_layers": "HIP graphs that each hold one step of several consecutive layers in order (as a "
                              "whole-model decode graph holds every layer), every call on one stream",
              "graph_fused_layers": "HIP graphs that each hold one step of several consecutive layers in order (as a "
                                    "whole-model decode graph holds every layer), every call on one stream, both "
                                    "caches' compress_insert inside the index-score launch (csa_compress_index_score)"}


def capture_graphs(torch, layers, fn):
    """One HIP graph per layer holding one whole step (fn(layer) issued on the capturing stream)."""
    graphs = []
    for ly in layers:
        fn(ly)  # eager warm-up of exactly the captured work
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn(ly)
        graphs.append(g)
    torch.cuda.synchronize()
    return graphs


def capture_layers_graph(torch, layers, fn):
    """One HIP graph holding one step of every layer, in layer order (fn(layer) for each, on the capturing stream)."""
    for ly in layers:
        fn(ly)  # eager warm-up of exactly the captured work
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for ly in layers:
            fn(ly)
    torch.cuda.synchronize()
    return g


def time_graphs(torch, graphs, steps, warmup, per=1):
    """Replay the step graphs in rotation (each replay runs `per` steps); ms for `steps` steps between two events."""
    for i in range(max(1, warmup // per)):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(steps // per):
        graphs[i % len(graphs)].replay()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1)


def replay_percentiles(torch, graphs, steps, per=1):
    """Each replay between its own pair of events (a separate pass after the timed region): p10 / median / p90 of
    the per-step time in microseconds (a replay's time over its `per` steps)."""
    ev = []
    for i in range(steps // per):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        graphs[i % len(graphs)].replay()
        b.record()
        ev.append((a, b))
    torch.cuda.synchronize()
    v = np.array([a.elapsed_time(b) * 1e3 / per for a, b in ev])
    return {"p10": round(float(np.percentile(v, 10)), 2), "median": round(float(np.median(v)), 2),
            "p90": round(float(np.percentile(v, 90)), 2), "n": int(len(v))}


LAST_PERCENTILES = {}


def best_graph_mode(torch, layers, steps, warmup, sequential, two_stream, partitioned=None, fused=None):
    """Time the step as one HIP graph per layer in each stream arrangement given (all on one stream; main-cache
    compress on a second stream; the indexer pipeline on a second stream; all on one stream with the compress inside
    the index-score launch), and as graphs that each hold one step of gcd(steps, layers) consecutive layers in order
    (the fused step where given, else the one-stream step), replayed in rotation so that exactly `steps` steps run
    and every layer as often; returns (ms of the fastest, its name, ms of each). The per-step percentiles of the fastest are left in LAST_PERCENTILES. With --eager-only (profiler
    runs) no graph is built and (None, "eager", {}) comes back."""
    LAST_PERCENTILES.clear()
    if EAGER_ONLY:
        return None, "eager", {}
    modes, kept = {}, {}
    for name, fn in (("graph", sequential), ("graph_2stream", two_stream), ("graph_partition", partitioned),
                     ("graph_fused", fused)):
        if fn is None:
            continue
        graphs = capture_graphs(torch, layers, fn)
        modes[name] = time_graphs(torch, graphs, steps, warmup)
        kept[name] = (graphs, 1)
    per = math.gcd(steps, len(layers))  # layers per graph: exactly `steps` steps, every layer equally often
    if per > 1:
        name = "graph_fused_layers" if fused is not None else "graph_layers"
        graphs = [capture_layers_graph(torch, layers[i:i + per], fused if fused is not None else sequential)
                  for i in range(0, len(layers), per)]
        modes[name] = time_graphs(torch, graphs, steps, warmup, per=per)
        kept[name] = (graphs, per)
    best = min(modes, key=modes.get)
    LAST_PERCENTILES.update(replay_percentiles(torch, kept[best][0], steps, per=kept[best][1]))
    LAST_PERCENTILES["steps_per_replay"] = kept[best][1]
    del kept
    return modes[best], best, modes


def partition_modes(torch, layers, steps, warmup, prepare, main_compress, index_path, attend, pair=None, fused=None):
    """The step with the query / window-key preparation in front (csa_prepare_qk), captured two ways: every call on
    one stream (the indexer and main compress as one paired launch when `pair` is given), and the pages' two-stream
    partition -- on a c4a layer the indexer pipeline (its compress, score, select) on a second stream beside main
    compress + window insert, on a c128a layer (index_path None) main compress beside the window insert; attention
    joins; with `fused` (both compresses, score and select in csa_compress_index_score + csa_index_select) also that
    on one stream. Returns ms per step of each, or {} without graphs."""
    if EAGER_ONLY:
        return {}
    side = torch.cuda.Stream()

    def single(ly):
        prepare(ly)
        if pair is not None:
            pair(ly)
        else:
            main_compress(ly)
        if index_path is not None:
            index_path(ly)
        attend(ly)

    def split(ly):
        cur = torch.cuda.current_stream()
        side.wait_stream(cur)
        with torch.cuda.stream(side):
            if index_path is not None:
                index_path(ly)
            else:
                main_compress(ly)
        if index_path is not None:
            main_compress(ly)
        prepare(ly)
        cur.wait_stream(side)
        attend(ly)

    def single_fused(ly):
        prepare(ly)
        fused(ly)
        attend(ly)

    out = {}
    for name, fn in (("single_stream", single), ("partition_2stream", split),
                     ("single_stream_fused", single_fused if fused is not None else None)):
        if fn is None:
            continue
        graphs = capture_graphs(torch, layers, fn)
        out[name] = time_graphs(torch, graphs, steps, warmup) / steps
        del graphs
    return {k: round(v, 5) for k, v in out.items()}


def partitioned(torch, side, main_compress, index_path, attend):
    """The decode step with the indexer pipeline on a second stream beside the main-cache compress ([P1] "GPU Compute
    Saturation", [P2] "3.2 內核"); attention joins both."""
    def fn(ly):
        cur = torch.cuda.current_stream()
        side.wait_stream(cur)
        with torch.cuda.stream(side):
            index_path(ly)
        main_compress(ly)
        cur.wait_stream(side)
        attend(ly)
    return fn


def overlapped(torch, side, main_compress, index_path, attend):
    """The decode step with the main-cache compress on a second stream beside the indexer pipeline: only the
    attention needs the main cache, so it joins there (both streams at the default priority)."""
    def fn(ly):
        cur = torch.cuda.current_stream()
        side.wait_stream(cur)
        with torch.cuda.stream(side):
            main_compress(ly)
        index_path(ly)
        cur.wait_stream(side)
        attend(ly)
    return fn


def run_gpu(args, lens):
    import torch
    import long_context_compressed_compress_amd as csa
    torch.cuda.init()
    max_rows = LEN_HI + 2
    rope_main = csa.rope_table(max_rows, R)
    rope_idx = csa.rope_table(max_rows, R_IDX)
    layers = []
    for l in range(args.layers):
        t0 = time.time()
        layers.append(Layer(l, lens, torch, csa, rope_main, rope_idx))
        torch.cuda.synchronize()
        log(f"layer {l} built in {time.time() - t0:.1f}s")
    max_elig = max(csa.num_eligible(int(L), 4, 8) for L in lens)
    ws = csa.index_workspace(B, max_elig, K_TOP, H_IDX)
    topk = torch.empty((B, K_TOP), dtype=torch.int32, device="cuda")
    out = torch.empty((B, H, D), dtype=torch.float32, device="cuda")
    scale = 1.0 / math.sqrt(D)
    att_ws_bytes = csa.attend_workspace(B, H, D, K_TOP + SWA)
    att_ws = torch.empty(max(att_ws_bytes, 1), dtype=torch.uint8, device="cuda")

    def step(ly, ev=None):
        if ev: ev[0].record()
        csa.compress_insert_pair(ly.cache, ly.state, ly.kv1, ly.lg1, ly.gamma, rope_main, ly.icache, ly.istate, ly.ikv1,
                                 ly.ilg1, ly.igamma, rope_idx, ly.pos, ly.cu1, 1e-6, 1)
        if ev: ev[1].record()
        csa.index_score(ly.icache, ly.seq, ly.pos, max_elig, ly.q_idx, ly.head_w, csa.SCORE_WRELU, K_TOP, ws)
        if ev: ev[2].record()
        csa.index_select(ly.icache, ly.seq, ly.pos, max_elig, K_TOP, topk, ws)
        if ev: ev[3].record()
        csa.attend(ly.cache, ly.swa, SWA, ly.seq, ly.pos, ly.q, topk, max_elig, scale, True, rope_main, out,
                   workspace=att_ws)
        if ev: ev[4].record()

    # achievable copy bandwidth of this device (1 GiB device-to-device, read + write counted)
    src = torch.empty(1 << 29, dtype=torch.int16, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(5):
        dst.copy_(src)
    c1.record()
    torch.cuda.synchronize()
    copy_gbs = 5 * 2 * (1 << 30) / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()

    for i in range(args.warmup):
        step(layers[i % len(layers)])
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.time()
    t_start.record()
    for i in range(args.steps):
        step(layers[i % len(layers)], evs[i])
    t_end.record()
    torch.cuda.synchronize()
    wall = time.time() - wall0
    eager_ms = t_start.elapsed_time(t_end)
    names = ["compress", "score", "select", "attend"]
    stage_ms = {n: float(np.mean([e[j].elapsed_time(e[j + 1]) for e in evs])) for j, n in enumerate(names)}

    # the step as deployed: one HIP graph per layer, main-cache compress overlapped with the indexer pipeline
    side = torch.cuda.Stream()
    parts = (
        lambda ly: csa.compress_insert(ly.cache, ly.state, ly.pos, ly.cu1, ly.kv1, ly.lg1, ly.gamma, 1e-6, rope_main, 1),
        lambda ly: (csa.compress_insert(ly.icache, ly.istate, ly.pos, ly.cu1, ly.ikv1, ly.ilg1, ly.igamma, 1e-6,
                                        rope_idx, 1),
                    csa.index_score(ly.icache, ly.seq, ly.pos, max_elig, ly.q_idx, ly.head_w, csa.SCORE_WRELU, K_TOP,
                                    ws),
                    csa.index_select(ly.icache, ly.seq, ly.pos, max_elig, K_TOP, topk, ws)),
        lambda ly: csa.attend(ly.cache, ly.swa, SWA, ly.seq, ly.pos, ly.q, topk, max_elig, scale, True, rope_main, out,
                              workspace=att_ws))
    fused_index = lambda ly: (
        csa.compress_index_score(ly.cache, ly.state, ly.kv1, ly.lg1, ly.gamma, rope_main, ly.icache, ly.istate, ly.ikv1,
                                 ly.ilg1, ly.igamma, rope_idx, ly.pos, ly.cu1, 1e-6, ly.seq, ly.pos, max_elig,
                                 ly.q_idx, ly.head_w, csa.SCORE_WRELU, K_TOP, ws),
        csa.index_select(ly.icache, ly.seq, ly.pos, max_elig, K_TOP, topk, ws))
    wall0 = time.time()
    fn = overlapped(torch, side, *parts)
    fn_p = partitioned(torch, torch.cuda.Stream(), *parts)
    total_ms, mode, modes = best_graph_mode(torch, layers, args.steps, args.warmup, lambda ly: step(ly, None), fn,
                                            fn_p, lambda ly: (fused_index(ly), parts[2](ly)))
    wall = time.time() - wall0
    pct = dict(LAST_PERCENTILES)
    for ly in layers:
        ly.q_raw = ly.q.clone()          # synthetic un-normed queries; prepare writes the attention's query
        ly.q_gamma = torch.ones(D, device="cuda")
    f4 = partition_modes(
        torch, layers, args.steps, args.warmup,
        lambda ly: csa.prepare_qk(ly.q_raw, ly.kv1, ly.seq, ly.pos, ly.q_gamma, 1e-6, ly.swa, R, rope_main, ly.q),
        lambda ly: csa.compress_insert(ly.cache, ly.state, ly.pos, ly.cu1, ly.kv1, ly.lg1, ly.gamma, 1e-6, rope_main, 1),
        lambda ly: (csa.compress_insert(ly.icache, ly.istate, ly.pos, ly.cu1, ly.ikv1, ly.ilg1, ly.igamma, 1e-6,
                                        rope_idx, 1),
                    csa.index_score(ly.icache, ly.seq, ly.pos, max_elig, ly.q_idx, ly.head_w, csa.SCORE_WRELU, K_TOP,
                                    ws),
                    csa.index_select(ly.icache, ly.seq, ly.pos, max_elig, K_TOP, topk, ws)),
        lambda ly: csa.attend(ly.cache, ly.swa, SWA, ly.seq, ly.pos, ly.q, topk, max_elig, scale, True, rope_main, out,
                              workspace=att_ws),
        pair=lambda ly: csa.compress_insert_pair(ly.cache, ly.state, ly.kv1, ly.lg1, ly.gamma, rope_main, ly.icache,
                                                 ly.istate, ly.ikv1, ly.ilg1, ly.igamma, rope_idx, ly.pos, ly.cu1, 1e-6,
                                                 1),
        fused=fused_index)
    epilogue = time_output_epilogue(torch, csa, layers, step, out, topk, max_elig, scale, rope_main, att_ws)
    epilogue["step_with_prepare_ms"] = f4
    epilogue["step_us_percentiles"] = pct
    epilogue["upstream_prepare"] = time_prepare(torch, csa, layers[-1], rope_main)
    return total_ms, eager_ms, wall, stage_ms, copy_gbs, mode, modes, epilogue


def time_prepare(torch, csa, ly, rope, iters=100):
    """The fused step in front of this path (query RMSNorm + RoPE for 64 heads, window-key RoPE + insert) for the
    batch's 32 decode tokens, timed alone (it rewrites the window row of each query position of this layer).
    Algorithmic bytes: q read and written once (bf16), the key row read and its window row written."""
    q_out = torch.empty_like(ly.q)
    gamma = torch.ones(D, device="cuda")
    for _ in range(5):
        csa.prepare_qk(ly.q, ly.kv1, ly.seq, ly.pos, gamma, 1e-6, ly.swa, R, rope, q_out)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        csa.prepare_qk(ly.q, ly.kv1, ly.seq, ly.pos, gamma, 1e-6, ly.swa, R, rope, q_out)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / iters
    alg = 2 * ly.q.numel() * 2 + 2 * ly.kv1.numel() * 2 + D * 4
    return {"kernel": "prepare_qk_kernel", "us": round(us, 2), "alg_bytes": alg, "gbs": round(alg / (us * 1e-6) / 1e9, 1),
            "frac_peak": round(alg / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}


def time_output_epilogue(torch, csa, layers, step, out, topk, max_elig, scale, rope, att_ws, group=128, iters=100):
    """The fused inverse RoPE + fp8 quantisation of the attention output (the step after this path, in front of an
    fp8 output projection) on this workload's real outputs: attention without its fused rotation, then the
    epilogue kernel timed alone. Algorithmic bytes: the fp32 output read once, codes and group scales written."""
    ly = layers[0]
    step(ly, None)
    raw = torch.empty_like(out)
    csa.attend(ly.cache, ly.swa, SWA, ly.seq, ly.pos, ly.q, topk, max_elig, scale, False, rope, raw, workspace=att_ws)
    codes = torch.empty(raw.shape, dtype=torch.uint8, device="cuda")
    scales = torch.empty((B, H, D // group), dtype=torch.float32, device="cuda")
    for _ in range(5):
        csa.inv_rope_quant_fp8(raw, ly.pos, R, rope, group, codes, scales)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        csa.inv_rope_quant_fp8(raw, ly.pos, R, rope, group, codes, scales)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / iters
    alg = raw.numel() * 4 + codes.numel() + scales.numel() * 4

    # the same output produced by the attention itself (csa_attend_quant_fp8: the fp32 output never reaches HBM),
    # against the attention with an fp32 output (fused inverse RoPE), both over the rotated layers
    def attn_us(fn):
        for i in range(5):
            fn(layers[i % len(layers)])
        torch.cuda.synchronize()
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record()
        for i in range(iters):
            fn(layers[i % len(layers)])
        a1.record()
        torch.cuda.synchronize()
        return a0.elapsed_time(a1) * 1e3 / iters
    fused = attn_us(lambda l: csa.attend_quant_fp8(l.cache, l.swa, SWA, l.seq, l.pos, l.q, topk, max_elig, scale, rope,
                                                   group, codes, scales, workspace=att_ws))
    fp32 = attn_us(lambda l: csa.attend(l.cache, l.swa, SWA, l.seq, l.pos, l.q, topk, max_elig, scale, True, rope, out,
                                        workspace=att_ws))
    return {"kernel": "inv_rope_quant_kernel (separate pass over the fp32 output)", "group": group, "us": round(us, 2),
            "alg_bytes": alg, "gbs": round(alg / (us * 1e-6) / 1e9, 1),
            "frac_peak": round(alg / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "fused": {"call": "csa_attend_quant_fp8 (attention with the inverse RoPE + fp8 epilogue fused in)",
                      "attend_fp8_out_us": round(fused, 2), "attend_fp32_out_us": round(fp32, 2),
                      "unfused_attend_plus_pass_us": round(fp32 + us, 2),
                      "topk_note": "the top-k of the last timed step is reused for every layer"}}


# ------------------------------------------------------------------ side workloads, measured in the same run
POOL_BYTES = 200 * 10 ** 9
MFMA_BF16_PEAK_TFLOPS = 2500.0


def _gen(torch, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return g


def _tail(torch, lens, bt_stride, first_rel, last_rel, cpu_gen):
    """Table mapping only logical blocks L//256+first_rel .. L//256+last_rel of each sequence (window and
    compressor-state pages) onto a pool of its own; returns (device table, pages)."""
    per = last_rel - first_rel + 1
    perm = torch.randperm(len(lens) * per, generator=cpu_gen).to(torch.int32)
    t = torch.full((len(lens), bt_stride), -1, dtype=torch.int32)
    for b, L in enumerate(lens):
        for j, rel in enumerate(range(first_rel, last_rel + 1)):
            t[b, int(L) // 256 + rel] = perm[b * per + j]
    return t.to("cuda"), len(lens) * per


def _fp8_rows(torch, gen, rows, dim):
    """fp8 window rows: N(0,1) x 112 clamped to the e4m3fn range and cast by torch, one fp32 scale 4/448 per row."""
    x = (torch.randn((rows, dim), generator=gen, device="cuda") * 112.0).clamp_(-448.0, 448.0)  # e4m3fn has no inf
    return x.to(torch.float8_e4m3fn).view(torch.uint8), torch.full((rows,), 4.0 / 448.0, device="cuda")


def _build_prefix(torch, csa, cache, state, B, lens, dim, roles, gen, rope, per_call=1):
    """Append tokens 0..L_b-1 of every sequence (N(0,1) bf16 raw rows and logits) with compress_insert."""
    for c0 in range(0, B, per_call):
        n = [int(lens[b]) if c0 <= b < c0 + per_call else 0 for b in range(B)]
        cu = torch.tensor(np.concatenate([[0], np.cumsum(n)]), dtype=torch.int32, device="cuda")
        start = torch.zeros(B, dtype=torch.int32, device="cuda")
        tot = int(sum(n))
        kv = torch.randn((tot, dim), generator=gen, device="cuda", dtype=torch.bfloat16)
        lg = torch.randn((tot, roles, dim), generator=gen, device="cuda", dtype=torch.bfloat16)
        csa.compress_insert(cache, state, start, cu, kv, lg, torch.ones(dim, device="cuda"), 1e-6, rope, max(n))
        del kv, lg


def _decode_bytes(n_elig, p, e_main, e_idx, k, with_index):
    """Algorithmic bytes of one decode query: (index score, top-k out, attention) -- eligible indexer keys once plus
    q_idx and head weights; k indices; the selected entries and window rows once plus q and the fp32 output."""
    sel = min(k, n_elig) if with_index else n_elig
    score = n_elig * e_idx + H_IDX * D_IDX * 2 + 4 * H_IDX if with_index else 0
    att = sel * e_main + min(SWA, p + 1) * e_main + (4 * k if with_index else 0) + H * D * 2 + 4 * H * D
    return score, (4 * k if with_index else 0), att


def run_c4(args, torch, csa, fp4_idx=False):
    """c4a decode at 1M: batch 4, query at 2^20, fp8 main / indexer / window caches with per-entry scales, pages of
    every layer drawn uniformly from one 200 GB pool; top-512 + window 128. fp4_idx: the indexer cache is MXFP4
    (64 B of e2m1 codes + 4 E8M0 block exponents per entry) instead of fp8."""
    B, P = 4, 1 << 20
    nb = P // 256 + 1
    n_layers = args.layers_c4
    row_i = D_IDX // 2 if fp4_idx else D_IDX
    per_page = 64 * D + 64 * row_i + 2 * 64 * 4
    n_phys = POOL_BYTES // per_page
    cpu_gen = torch.Generator()
    cpu_gen.manual_seed(4007)
    gen = _gen(torch, 4100)
    pool_m = torch.empty((n_phys * 64, D), dtype=torch.uint8, device="cuda")
    pool_ms = torch.empty((n_phys * 64,), dtype=torch.float32, device="cuda")
    if fp4_idx:
        pool_i = torch.empty((n_phys * 64, row_i), dtype=torch.uint8, device="cuda").view(torch.float4_e2m1fn_x2)
        pool_is = torch.empty((n_phys * 64, D_IDX // 32), dtype=torch.uint8, device="cuda")
    else:
        pool_i = torch.empty((n_phys * 64, D_IDX), dtype=torch.uint8, device="cuda")
        pool_is = torch.empty((n_phys * 64,), dtype=torch.float32, device="cuda")
    ids = torch.randperm(n_phys, generator=cpu_gen)[: n_layers * B * nb].to(torch.int32)
    rope = csa.rope_table(P + 2, R)
    lens = [P] * B
    layers = []
    for l in range(n_layers):
        t0 = time.time()
        ly = type("C4Layer", (), {})()
        ly.bt = ids[l * B * nb:(l + 1) * B * nb].view(B, nb).contiguous().to("cuda")
        ly.cache = csa.Cache(4, 8, D, R, pool_m, ly.bt, pool_ms)
        ly.icache = csa.Cache(4, 8, D_IDX, R_IDX, pool_i, ly.bt, pool_is)
        tail, n_tail = _tail(torch, [P - 1] * B, nb, -1, 1, cpu_gen)
        ly.state = csa.Raw(D, 2, torch.zeros((n_tail * 256, D), dtype=torch.bfloat16, device="cuda"), tail,
                           torch.zeros((n_tail * 256, 2, D), dtype=torch.bfloat16, device="cuda"))
        ly.istate = csa.Raw(D_IDX, 2, torch.zeros((n_tail * 256, D_IDX), dtype=torch.bfloat16, device="cuda"), tail,
                            torch.zeros((n_tail * 256, 2, D_IDX), dtype=torch.bfloat16, device="cuda"))
        codes, sc = _fp8_rows(torch, gen, n_tail * 256, D)
        ly.swa = csa.Raw(D, 0, codes, tail, None, sc)
        _build_prefix(torch, csa, ly.cache, ly.state, B, lens, D, 2, gen, rope)
        _build_prefix(torch, csa, ly.icache, ly.istate, B, lens, D_IDX, 2, gen, rope)
        ly.pos = torch.full((B,), P, dtype=torch.int32, device="cuda")
        ly.seq = torch.arange(B, dtype=torch.int32, device="cuda")
        ly.cu1 = torch.arange(B + 1, dtype=torch.int32, device="cuda")
        ly.kv1 = torch.randn((B, D), generator=gen, device="cuda").to(torch.bfloat16)
        ly.lg1 = torch.randn((B, 2, D), generator=gen, device="cuda").to(torch.bfloat16)
        ly.ikv1 = torch.randn((B, D_IDX), generator=gen, device="cuda").to(torch.bfloat16)
        ly.ilg1 = torch.randn((B, 2, D_IDX), generator=gen, device="cuda").to(torch.bfloat16)
        ly.q = torch.randn((B, H, D), generator=gen, device="cuda").to(torch.bfloat16)
        ly.q_idx = torch.randn((B, H_IDX, D_IDX), generator=gen, device="cuda").to(torch.bfloat16)
        ly.head_w = torch.rand((B, H_IDX), generator=gen, device="cuda")
        ly.gamma, ly.igamma = torch.ones(D, device="cuda"), torch.ones(D_IDX, device="cuda")
        layers.append(ly)
        torch.cuda.synchronize()
        log(f"c4 layer {l} built in {time.time() - t0:.1f}s")
    max_elig = csa.num_eligible(P, 4, 8)
    ws = csa.index_workspace(B, max_elig, K_TOP, H_IDX)
    topk = torch.empty((B, K_TOP), dtype=torch.int32, device="cuda")
    out = torch.empty((B, H, D), dtype=torch.float32, device="cuda")
    att_ws = torch.empty(max(csa.attend_workspace(B, H, D, K_TOP + SWA), 1), dtype=torch.uint8, device="cuda")

    def step(ly, ev):
        if ev: ev[0].record()
        csa.compress_insert_pair(ly.cache, ly.state, ly.kv1, ly.lg1, ly.gamma, rope, ly.icache, ly.istate, ly.ikv1,
                                 ly.ilg1, ly.igamma, rope, ly.pos, ly.cu1, 1e-6, 1)
        if ev: ev[1].record()
        csa.index_score(ly.icache, ly.seq, ly.pos, max_elig, ly.q_idx, ly.head_w, csa.SCORE_WRELU, K_TOP, ws)
        if ev: ev[2].record()
        csa.index_select(ly.icache, ly.seq, ly.pos, max_elig, K_TOP, topk, ws)
        if ev: ev[3].record()
        csa.attend(ly.cache, ly.swa, SWA, ly.seq, ly.pos, ly.q, topk, max_elig, 1.0 / math.sqrt(D), True, rope, out,
                   workspace=att_ws)
        if ev: ev[4].record()

    log(f"c4: timing {args.steps} steps")
    eager_ms, st = time_steps(torch, step, layers, args.steps, args.warmup, 4)
    stage = dict(zip(["compress", "score", "select", "attend"], st))
    side = torch.cuda.Stream()
    parts = (
        lambda ly: csa.compress_insert(ly.cache, ly.state, ly.pos, ly.cu1, ly.kv1, ly.lg1, ly.gamma, 1e-6, rope, 1),
        lambda ly: (csa.compress_insert(ly.icache, ly.istate, ly.pos, ly.cu1, ly.ikv1, ly.ilg1, ly.igamma, 1e-6, rope, 1),
                    csa.index_score(ly.icache, ly.seq, ly.pos, max_elig, ly.q_idx, ly.head_w, csa.SCORE_WRELU, K_TOP,
                                    ws),
                    csa.index_select(ly.icache, ly.seq, ly.pos, max_elig, K_TOP, topk, ws)),
        lambda ly: csa.attend(ly.cache, ly.swa, SWA, ly.seq, ly.pos, ly.q, topk, max_elig, 1.0 / math.sqrt(D), True,
                              rope, out, workspace=att_ws))
    fused_index = lambda ly: (
        csa.compress_index_score(ly.cache, ly.state, ly.kv1, ly.lg1, ly.gamma, rope, ly.icache, ly.istate, ly.ikv1,
                                 ly.ilg1, ly.igamma, rope, ly.pos, ly.cu1, 1e-6, ly.seq, ly.pos, max_elig, ly.q_idx,
                                 ly.head_w, csa.SCORE_WRELU, K_TOP, ws),
        csa.index_select(ly.icache, ly.seq, ly.pos, max_elig, K_TOP, topk, ws))
    fn = overlapped(torch, side, *parts)
    fn_p = partitioned(torch, torch.cuda.Stream(), *parts)
    total_ms, mode, modes = best_graph_mode(torch, layers, args.steps, args.warmup, lambda ly: step(ly, None), fn,
                                            fn_p, lambda ly: (fused_index(ly), parts[2](ly)))
    total_ms = eager_ms if total_ms is None else total_ms
    pct = dict(LAST_PERCENTILES)
    for ly in layers:
        ly.q_raw, ly.q_gamma = ly.q.clone(), torch.ones(D, device="cuda")
    f4 = partition_modes(
        torch, layers, args.steps, args.warmup,
        lambda ly: csa.prepare_qk(ly.q_raw, ly.kv1, ly.seq, ly.pos, ly.q_gamma, 1e-6, ly.swa, R, rope, ly.q),
        lambda ly: csa.compress_insert(ly.cache, ly.state, ly.pos, ly.cu1, ly.kv1, ly.lg1, ly.gamma, 1e-6, rope, 1),
        lambda ly: (csa.compress_insert(ly.icache, ly.istate, ly.pos, ly.cu1, ly.ikv1, ly.ilg1, ly.igamma, 1e-6, rope, 1),
                    csa.index_score(ly.icache, ly.seq, ly.pos, max_elig, ly.q_idx, ly.head_w, csa.SCORE_WRELU, K_TOP,
                                    ws),
                    csa.index_select(ly.icache, ly.seq, ly.pos, max_elig, K_TOP, topk, ws)),
        lambda ly: csa.attend(ly.cache, ly.swa, SWA, ly.seq, ly.pos, ly.q, topk, max_elig, 1.0 / math.sqrt(D), True,
                              rope, out, workspace=att_ws),
        pair=lambda ly: csa.compress_insert_pair(ly.cache, ly.state, ly.kv1, ly.lg1, ly.gamma, rope, ly.icache,
                                                 ly.istate, ly.ikv1, ly.ilg1, ly.igamma, rope, ly.pos, ly.cu1, 1e-6, 1),
        fused=fused_index)
    sb, kb, ab = (B * x for x in _decode_bytes(max_elig, P, D + 4, row_i + 4, K_TOP, True))
    del layers, pool_m, pool_ms, pool_i, pool_is, ws
    torch.cuda.empty_cache()
    path_ms = stage["score"] + stage["select"] + stage["attend"]
    score_gbs = sb / (stage["score"] * 1e-3) / 1e9
    idx_desc = ("MXFP4 (e2m1 + E8M0 per 32 channels)" if fp4_idx else "fp8")
    return {
        "workload": f"c4a fp8 decode, batch {B}, context 2^20 (262143 compressed entries), query at 2^20, 64 heads x "
                    f"K=V 512 fp8 e4m3 + per-entry fp32 scale, indexer 64 heads x 128 {idx_desc} WRELU, top-512 + "
                    f"window 128, pages uniform over a 200 GB pool ({n_phys} 256-position pages), {n_layers} layers "
                    "rotated",
        "value": round(B * args.steps / (total_ms * 1e-3), 1), "unit": "queries/s",
        "ms_per_step": round(total_ms / args.steps, 5), "step_mode": STEP_MODES[mode],
        "modes_ms_per_step": {"eager_with_stage_events": round(eager_ms / args.steps, 5),
                              **{k: round(v / args.steps, 5) for k, v in modes.items()}},
        "dtype": ("fp8 e4m3 main cache, MXFP4 indexer cache" if fp4_idx else "fp8 e4m3 caches") +
                 ", bf16 queries, fp32 accumulate",
        "step_us_percentiles": pct,
        "stages_us": {k: round(v * 1e3, 2) for k, v in stage.items()},
        "step_with_prepare_ms": f4,
        "roofline": {"bound": "hbm", "kernel": f"{'score_mfma_kernel<fp4>' if fp4_idx else 'score_lt_kernel<fp8>'} "
                                               "(index score)",
                     "achieved": round(score_gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(score_gbs / HBM_PEAK_GBS, 4),
                     "traffic": score_traffic("c4f" if fp4_idx else "c4"),
                     "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE/WRITE_SIZE, copy-calibrated)",
                     "alg_bytes_per_launch": sb, "avg_launch_us": round(stage["score"] * 1e3, 2)},
        "gathered_path": {"hbm_gbs": round((sb + kb + ab) / (path_ms * 1e-3) / 1e9, 1),
                          "frac_peak": round((sb + kb + ab) / (path_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                          "alg_bytes": sb + kb + ab, "us": round(path_ms * 1e3, 2)},
    }


def run_c2(args, torch, csa):
    """c128a bf16 decode, batch 16 at position 65536: dense attention over all 512 eligible entries + window 128."""
    B, P = 16, 65536
    nb = P // 256 + 1
    n_layers = args.layers_c2
    cpu_gen = torch.Generator()
    cpu_gen.manual_seed(2007)
    gen = _gen(torch, 2100)
    rope = csa.rope_table(P + 2, R)
    layers = []
    t0 = time.time()
    for l in range(n_layers):
        ly = type("C2Layer", (), {})()
        n_phys = 2 * B * nb
        ly.bt = torch.randperm(n_phys, generator=cpu_gen)[: B * nb].to(torch.int32).view(B, nb).contiguous().to("cuda")
        ly.cache = csa.Cache(128, 128, D, R, torch.empty((n_phys * 2, D), dtype=torch.bfloat16, device="cuda"), ly.bt)
        tail, n_tail = _tail(torch, [P] * B, nb, -1, 0, cpu_gen)
        ly.state = csa.Raw(D, 1, torch.zeros((n_tail * 256, D), dtype=torch.bfloat16, device="cuda"), tail,
                           torch.zeros((n_tail * 256, 1, D), dtype=torch.bfloat16, device="cuda"))
        ly.swa = csa.Raw(D, 0, torch.randn((n_tail * 256, D), generator=gen, device="cuda", dtype=torch.bfloat16), tail)
        _build_prefix(torch, csa, ly.cache, ly.state, B, [P] * B, D, 1, gen, rope, per_call=B)
        ly.pos = torch.full((B,), P, dtype=torch.int32, device="cuda")
        ly.seq = torch.arange(B, dtype=torch.int32, device="cuda")
        ly.cu1 = torch.arange(B + 1, dtype=torch.int32, device="cuda")
        ly.kv1 = torch.randn((B, D), generator=gen, device="cuda", dtype=torch.bfloat16)
        ly.lg1 = torch.randn((B, 1, D), generator=gen, device="cuda", dtype=torch.bfloat16)
        ly.q = torch.randn((B, H, D), generator=gen, device="cuda", dtype=torch.bfloat16)
        layers.append(ly)
    gamma = torch.ones(D, device="cuda")
    torch.cuda.synchronize()
    log(f"c2: {n_layers} layers built in {time.time() - t0:.1f}s")
    n_elig = csa.num_eligible(P, 128, 128)
    out = torch.empty((B, H, D), dtype=torch.float32, device="cuda")
    att_ws = torch.empty(max(csa.attend_workspace(B, H, D, n_elig + SWA), 1), dtype=torch.uint8, device="cuda")

    def step(ly, ev):
        if ev: ev[0].record()
        csa.compress_insert(ly.cache, ly.state, ly.pos, ly.cu1, ly.kv1, ly.lg1, gamma, 1e-6, rope, 1)
        if ev: ev[1].record()
        csa.attend(ly.cache, ly.swa, SWA, ly.seq, ly.pos, ly.q, None, n_elig, 1.0 / math.sqrt(D), True, rope, out,
                   workspace=att_ws)
        if ev: ev[2].record()

    log(f"c2: timing {args.steps} steps")
    eager_ms, st = time_steps(torch, step, layers, args.steps, args.warmup, 2)
    stage = dict(zip(["compress", "attend"], st))
    total_ms, mode, modes = best_graph_mode(torch, layers, args.steps, args.warmup, lambda ly: step(ly, None), None)
    total_ms = eager_ms if total_ms is None else total_ms
    pct = dict(LAST_PERCENTILES)
    for ly in layers:
        ly.q_raw, ly.q_gamma = ly.q.clone(), torch.ones(D, device="cuda")
    f4 = partition_modes(
        torch, layers, args.steps, args.warmup,
        lambda ly: csa.prepare_qk(ly.q_raw, ly.kv1, ly.seq, ly.pos, ly.q_gamma, 1e-6, ly.swa, R, rope, ly.q),
        lambda ly: csa.compress_insert(ly.cache, ly.state, ly.pos, ly.cu1, ly.kv1, ly.lg1, gamma, 1e-6, rope, 1),
        None,
        lambda ly: csa.attend(ly.cache, ly.swa, SWA, ly.seq, ly.pos, ly.q, None, n_elig, 1.0 / math.sqrt(D), True,
                              rope, out, workspace=att_ws))
    _, _, ab = (B * x for x in _decode_bytes(n_elig, P, 2 * D, 0, 0, False))
    del layers
    torch.cuda.empty_cache()
    gbs = ab / (stage["attend"] * 1e-3) / 1e9
    return {
        "workload": f"c128a bf16 decode, batch {B}, context 65536 (512 compressed entries), query at 65536, 64 heads x "
                    f"K=V 512, dense over every eligible entry + window 128, {n_layers} layers rotated",
        "value": round(B * args.steps / (total_ms * 1e-3), 1), "unit": "queries/s",
        "ms_per_step": round(total_ms / args.steps, 5), "step_mode": STEP_MODES[mode],
        "modes_ms_per_step": {"eager_with_stage_events": round(eager_ms / args.steps, 5),
                              **{k: round(v / args.steps, 5) for k, v in modes.items()}},
        "dtype": "bf16",
        "step_us_percentiles": pct,
        "stages_us": {k: round(v * 1e3, 2) for k, v in stage.items()},
        "step_with_prepare_ms": dict(f4, note="main compress beside the window insert on c128a layers"),
        "roofline": {"bound": "hbm", "kernel": "attend_split_kernel + attend_combine_kernel (dense)",
                     "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "alg_bytes_per_launch": ab,
                     "avg_launch_us": round(stage["attend"] * 1e3, 2)},
    }


def run_c5(args, torch, csa):
    """Prefill chunk on one c4a + c128a layer pair: 2 sequences x 2048 new tokens at context 262144. compress_insert of
    the chunk into the c4a main, indexer and c128a caches, index + top-512 for all 4096 queries, causal top-512 +
    window attention (c4a), dense attention over the 2048-2064 eligible c128a entries + window."""
    B, CTX, CH = 2, 262144, 2048
    nb = (CTX + CH - 1) // 256 + 1
    n_layers = args.layers_c5
    cpu_gen = torch.Generator()
    cpu_gen.manual_seed(5007)
    gen = _gen(torch, 5100)
    rows = CTX + CH + 1
    rope = csa.rope_table(rows, R)
    n_q = B * CH
    q_pos = torch.arange(CTX, CTX + CH, dtype=torch.int32).repeat(B).to("cuda")
    q_seq = torch.arange(B, dtype=torch.int32).repeat_interleave(CH).to("cuda")
    start = torch.full((B,), CTX, dtype=torch.int32, device="cuda")
    cu = (torch.arange(B + 1, dtype=torch.int32) * CH).to("cuda")
    layers = []
    t0 = time.time()
    for l in range(n_layers):
        ly = type("C5Layer", (), {})()
        n_phys = B * nb + 8
        ly.bt = torch.randperm(n_phys, generator=cpu_gen)[: B * nb].to(torch.int32).view(B, nb).contiguous().to("cuda")
        bf = torch.bfloat16
        ly.cache = csa.Cache(4, 8, D, R, torch.empty((n_phys * 64, D), dtype=bf, device="cuda"), ly.bt)
        ly.icache = csa.Cache(4, 8, D_IDX, R_IDX, torch.empty((n_phys * 64, D_IDX), dtype=bf, device="cuda"), ly.bt)
        ly.hcache = csa.Cache(128, 128, D, R, torch.empty((n_phys * 2, D), dtype=bf, device="cuda"), ly.bt)
        tail, n_tail = _tail(torch, [CTX] * B, nb, -1, (CH - 1) // 256, cpu_gen)
        z = lambda *shape: torch.zeros(shape, dtype=bf, device="cuda")
        ly.state = csa.Raw(D, 2, z(n_tail * 256, D), tail, z(n_tail * 256, 2, D))
        ly.istate = csa.Raw(D_IDX, 2, z(n_tail * 256, D_IDX), tail, z(n_tail * 256, 2, D_IDX))
        ly.hstate = csa.Raw(D, 1, z(n_tail * 256, D), tail, z(n_tail * 256, 1, D))
        ly.swa = csa.Raw(D, 0, torch.randn((n_tail * 256, D), generator=gen, device="cuda", dtype=bf), tail)
        _build_prefix(torch, csa, ly.cache, ly.state, B, [CTX] * B, D, 2, gen, rope, per_call=B)
        _build_prefix(torch, csa, ly.icache, ly.istate, B, [CTX] * B, D_IDX, 2, gen, rope, per_call=B)
        _build_prefix(torch, csa, ly.hcache, ly.hstate, B, [CTX] * B, D, 1, gen, rope, per_call=B)
        r = lambda *shape: torch.randn(shape, generator=gen, device="cuda", dtype=bf)
        ly.kv, ly.lg, ly.ikv, ly.ilg = r(n_q, D), r(n_q, 2, D), r(n_q, D_IDX), r(n_q, 2, D_IDX)
        ly.hkv, ly.hlg = r(n_q, D), r(n_q, 1, D)
        ly.q, ly.q_idx = r(n_q, H, D), r(n_q, H_IDX, D_IDX)
        ly.head_w = torch.rand((n_q, H_IDX), generator=gen, device="cuda")
        layers.append(ly)
    g1, gi = torch.ones(D, device="cuda"), torch.ones(D_IDX, device="cuda")
    torch.cuda.synchronize()
    log(f"c5: {n_layers} layers built in {time.time() - t0:.1f}s")
    max_elig = csa.num_eligible(CTX + CH - 1, 4, 8)
    max_elig_h = csa.num_eligible(CTX + CH - 1, 128, 128)
    ws = csa.index_workspace(n_q, max_elig, K_TOP, H_IDX)
    topk = torch.empty((n_q, K_TOP), dtype=torch.int32, device="cuda")
    out = torch.empty((n_q, H, D), dtype=torch.float32, device="cuda")
    out_h = torch.empty((n_q, H, D), dtype=torch.float32, device="cuda")
    scale = 1.0 / math.sqrt(D)

    def step(ly, ev):
        if ev: ev[0].record()
        csa.compress_insert_pair(ly.cache, ly.state, ly.kv, ly.lg, g1, rope, ly.icache, ly.istate, ly.ikv, ly.ilg, gi,
                                 rope, start, cu, 1e-6, CH)
        csa.compress_insert(ly.hcache, ly.hstate, start, cu, ly.hkv, ly.hlg, g1, 1e-6, rope, CH)
        if ev: ev[1].record()
        csa.index_score(ly.icache, q_seq, q_pos, max_elig, ly.q_idx, ly.head_w, csa.SCORE_WRELU, K_TOP, ws)
        if ev: ev[2].record()
        csa.index_select(ly.icache, q_seq, q_pos, max_elig, K_TOP, topk, ws)
        if ev: ev[3].record()
        csa.attend(ly.cache, ly.swa, SWA, q_seq, q_pos, ly.q, topk, max_elig, scale, True, rope, out)
        if ev: ev[4].record()
        csa.attend(ly.hcache, ly.swa, SWA, q_seq, q_pos, ly.q, None, max_elig_h, scale, True, rope, out_h)
        if ev: ev[5].record()

    steps = max(1, min(args.steps, args.steps_c5))
    log(f"c5: timing {steps} steps")
    total_ms, st = time_steps(torch, step, layers, steps, min(args.warmup, 2), 5)
    stage = dict(zip(["compress", "score", "select", "attend_c4a", "attend_c128a"], st))
    del layers, ws
    torch.cuda.empty_cache()
    pos = np.arange(CTX, CTX + CH)
    ne = np.array([(p + 1 - 8) // 4 + 1 for p in pos], np.int64)        # eligible c4a entries at each position
    ne_h = np.array([(p + 1 - 128) // 128 + 1 for p in pos], np.int64)   # eligible c128a entries
    score_fl = B * int(np.sum(2 * H_IDX * D_IDX * ne))
    att_fl = B * int(np.sum(4 * H * D * (np.minimum(K_TOP, ne) + SWA)))
    atth_fl = B * int(np.sum(4 * H * D * (ne_h + SWA)))
    tf = lambda fl, ms: fl / (ms * 1e-3) / 1e12
    mf = {"score": (score_fl, stage["score"]), "attend_c4a": (att_fl, stage["attend_c4a"]),
          "attend_c128a": (atth_fl, stage["attend_c128a"])}
    return {
        "workload": f"prefill chunk, batch {B} x {CH} new tokens at context {CTX}: compress_insert (c4a main + indexer, "
                    "c128a), index + top-512 for every new query, causal top-512 + window 128 attention (c4a), dense "
                    "c128a attention over 2048-2064 entries + window 128; 64 heads x K=V 512 bf16, indexer 64 x 128 "
                    f"WRELU, one shared block table, {n_layers} layers rotated",
        "value": round(n_q * steps / (total_ms * 1e-3), 1), "unit": "tokens/s",
        "ms_per_step": round(total_ms / steps, 4), "steps": steps, "dtype": "bf16",
        "stages_us": {k: round(v * 1e3, 1) for k, v in stage.items()},
        "mfma": {k: {"flop": fl, "tflops": round(tf(fl, ms), 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "frac": round(tf(fl, ms) / MFMA_BF16_PEAK_TFLOPS, 4)} for k, (fl, ms) in mf.items()},
        "roofline": {"bound": "mfma", "kernel": "score_shared_kernel (index score, 4096 queries)",
                     "achieved": round(tf(score_fl, stage["score"]), 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tf(score_fl, stage["score"]) / MFMA_BF16_PEAK_TFLOPS, 4),
                     "avg_launch_us": round(stage["score"] * 1e3, 1)},
    }


SIDE = {"c4": ("c4a_fp8_1m", run_c4),
        "c4f": ("c4a_fp8_fp4idx_1m", lambda args, torch, csa: run_c4(args, torch, csa, fp4_idx=True)),
        "c2": ("c128a_dense_64k", run_c2), "c5": ("prefill_chunk_256k", run_c5)}


# ------------------------------------------------------------------ CPU baseline: the oracle, untuned
def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        return os.cpu_count() or 1


def _time_units(fn, min_seconds):
    """Call fn() (one unit of work each) until min_seconds have passed; (units, seconds)."""
    n, t0 = 0, time.time()
    while True:
        fn(n)
        n += 1
        if time.time() - t0 >= min_seconds:
            return n, time.time() - t0


def _timed_both(fn, min_seconds, unit, sample):
    """The oracle at the BLAS library's default thread count and at one thread."""
    from threadpoolctl import threadpool_limits
    threads = _blas_threads()
    n, dt = _time_units(fn, min_seconds)
    with threadpool_limits(limits=1):
        n1, dt1 = _time_units(fn, min_seconds)
    return {"value": n / dt, "unit": unit, "cores": int(threads), "kind": "oracle",
            "value_1_thread": n1 / dt1, "cpu_model": cpu_model(), "nproc": os.cpu_count(),
            "sample": sample + f"; {n} units in {dt:.1f} s at {threads} BLAS threads, {n1} in {dt1:.1f} s at 1 thread"}


def _host_decode_layer(g, L, ratio, main_dt, idx_dt, dim_i, fp4_idx=False):
    """Oracle host caches of one sequence at position L: identity block table, every entry drawn (bf16 N(0,1) rows
    or the per-row e4m3 rows of synth), window / compressor-state pages for the last two blocks only."""
    import synth
    from oracle import codecs, compress as oc
    nb = L // 256 + 1
    E = 256 // ratio
    window = 8 if ratio == 4 else 128
    bt = np.arange(nb, dtype=np.int32)[None]
    tail = np.full((1, nb), -1, np.int32)
    tail[0, nb - 2], tail[0, nb - 1] = 0, 1

    def cache(dim, dt, rope):
        if dt == "bf16":
            return oc.Cache(ratio, window, dim, rope, "bf16", synth.normal_bf16_bits(g, (nb * E, dim)), None, bt)
        if dt == "fp8":
            codes, sc = synth.e4m3_rows(g, nb * E, dim)
            return oc.Cache(ratio, window, dim, rope, "fp8", codes, sc, bt)
        # MXFP4: random e2m1 codes and block exponents around 2^-2
        pk = g.integers(0, 256, size=(nb * E, dim // 2), dtype=np.uint8)
        ex = (125 + g.integers(0, 3, size=(nb * E, dim // 32))).astype(np.uint8)
        return oc.Cache(ratio, window, dim, rope, "fp4", pk, ex, bt)

    mc = cache(D, main_dt, R)
    ic = cache(dim_i, idx_dt, R_IDX) if dim_i else None
    if main_dt == "fp8":
        wp, ws_ = synth.e4m3_rows(g, 512, D)
        swa = oc.Raw("fp8", D, 0, wp, None, ws_, tail)
    else:
        swa = oc.Raw("bf16", D, 0, synth.normal_bf16_bits(g, (512, D)), None, None, tail)
    roles = window // ratio
    st = oc.Raw("bf16", D, roles, synth.normal_bf16_bits(g, (512, D)), synth.normal_bf16_bits(g, (512, roles, D)), None,
                tail)
    ist = oc.Raw("bf16", dim_i, 2, synth.normal_bf16_bits(g, (512, dim_i)),
                 synth.normal_bf16_bits(g, (512, 2, dim_i)), None, tail) if dim_i else None
    return mc, ic, swa, st, ist


def _decode_unit(L, layer, g, tables, with_index):
    """One decode query through the oracle: compress_insert of the token (main and, with an index, indexer),
    index_topk, attention with inverse RoPE."""
    import synth
    from oracle import attend as oa, codecs, compress as oc, index as oi
    mc, ic, swa, st, ist = layer
    table, itable = tables
    roles = st.roles
    new = (synth.normal_bf16_bits(g, (1, D)), synth.normal_bf16_bits(g, (1, roles, D)))
    q = codecs.load_rows(synth.normal_bf16_bits(g, (1, H, D)), "bf16")
    one = np.array([0, 1], np.int32)

    def run(_):
        oc.compress_insert(mc, st, [L], one, new[0], new[1], np.ones(D), 1e-6, table, 1)
        idx = None
        if with_index:
            inew = (synth.normal_bf16_bits(g, (1, D_IDX)), synth.normal_bf16_bits(g, (1, 2, D_IDX)))
            oc.compress_insert(ic, ist, [L], one, inew[0], inew[1], np.ones(D_IDX), 1e-6, itable, 1)
            qi = codecs.load_rows(synth.normal_bf16_bits(g, (1, H_IDX, D_IDX)), "bf16")
            idx, _, _ = oi.index_topk(ic, [0], [L], qi, synth.uniform_f32(g, (1, H_IDX)), oi.WRELU, K_TOP)
        oa.attend(mc, swa, SWA, [0], [L], q, idx, 1.0 / math.sqrt(D), True, table)
    return run


def cpu_baseline(lens, min_seconds=10.0, n_seq=8):
    """128K bf16 decode: the full step for 8 sequences of the workload, repeated."""
    import synth
    from oracle import rope as orope
    g = synth.rng(CONFIG_ID, 40)
    tables = (orope.rope_table(LEN_HI + 2, R), orope.rope_table(LEN_HI + 2, R_IDX))
    units = [_decode_unit(int(lens[b]), _host_decode_layer(g, int(lens[b]), 4, "bf16", "bf16", D_IDX), g, tables, True)
             for b in range(n_seq)]
    return _timed_both(lambda n: units[n % n_seq](n), min_seconds, "queries/s",
                       f"decode queries of {n_seq} sequences of the workload (contexts {int(min(lens[:n_seq]))}-"
                       f"{int(max(lens[:n_seq]))}) through the numpy fp64 oracle: compress_insert x2, index_topk, "
                       "attend with inverse RoPE")


def cpu_baseline_c4(min_seconds, fp4_idx=False):
    """1M fp8 decode (fp8 or MXFP4 indexer cache): the full step of one sequence at 2^20, repeated."""
    import synth
    from oracle import rope as orope
    P = 1 << 20
    g = synth.rng(4, 40)
    tables = (orope.rope_table(P + 2, R), orope.rope_table(P + 2, R_IDX))
    unit = _decode_unit(P, _host_decode_layer(g, P, 4, "fp8", "fp4" if fp4_idx else "fp8", D_IDX), g, tables, True)
    return _timed_both(unit, min_seconds, "queries/s",
                       "decode queries at 2^20 (262143 eligible entries, fp8 main cache, "
                       f"{'MXFP4' if fp4_idx else 'fp8'} indexer cache) through the numpy fp64 oracle: compress_insert "
                       "x2, index_topk, attend with inverse RoPE")


def cpu_baseline_c2(min_seconds):
    """c128a dense 64K decode: compress_insert of the token and dense attention, repeated."""
    import synth
    from oracle import rope as orope
    P = 65536
    g = synth.rng(2, 40)
    tables = (orope.rope_table(P + 2, R), None)
    unit = _decode_unit(P, _host_decode_layer(g, P, 128, "bf16", None, 0), g, tables, False)
    return _timed_both(unit, min_seconds, "queries/s",
                       "decode queries at 65536 (512 c128a entries, dense + window 128) through the numpy fp64 oracle: "
                       "compress_insert, attend with inverse RoPE")


def cpu_baseline_c5(min_seconds, n_sample=8):
    """Prefill chunk at 262144: per-token oracle work on a deterministic sample of the chunk's queries (index_topk +
    c4a attention + dense c128a attention each) plus the chunk's compression (three caches) of one sequence, timed
    separately and charged per token."""
    import synth
    from oracle import attend as oa, codecs, compress as oc, index as oi, rope as orope
    CTX, CH = 262144, 2048
    g = synth.rng(5, 40)
    table, itable = orope.rope_table(CTX + CH + 2, R), orope.rope_table(CTX + CH + 2, R_IDX)
    L = CTX + CH - 1
    mc, ic, swa, st, ist = _host_decode_layer(g, L, 4, "bf16", "bf16", D_IDX)
    hc, _, _, hst, _ = _host_decode_layer(g, L, 128, "bf16", None, 0)
    pos = [CTX + int(i * (CH - 1) / (n_sample - 1)) for i in range(n_sample)]   # first, last and evenly between
    qs = [codecs.load_rows(synth.normal_bf16_bits(g, (1, H, D)), "bf16") for _ in pos]
    qis = [codecs.load_rows(synth.normal_bf16_bits(g, (1, H_IDX, D_IDX)), "bf16") for _ in pos]
    w = synth.uniform_f32(g, (1, H_IDX))

    def per_query(n):
        i = n % n_sample
        idx, _, _ = oi.index_topk(ic, [0], [pos[i]], qis[i], w, oi.WRELU, K_TOP)
        oa.attend(mc, swa, SWA, [0], [pos[i]], qs[i], idx, 1.0 / math.sqrt(D), True, table)
        oa.attend(hc, swa, SWA, [0], [pos[i]], qs[i], None, 1.0 / math.sqrt(D), True, table)

    n_tok = 256  # compression of the chunk's first 256 tokens of one sequence into all three caches
    kv = synth.normal_bf16_bits(g, (n_tok, D))
    lg2, lg1 = synth.normal_bf16_bits(g, (n_tok, 2, D)), synth.normal_bf16_bits(g, (n_tok, 1, D))
    ikv, ilg = synth.normal_bf16_bits(g, (n_tok, D_IDX)), synth.normal_bf16_bits(g, (n_tok, 2, D_IDX))
    cu = np.array([0, n_tok], np.int32)
    # window / state pages of the oracle layer map only the last two blocks: give the compressor the chunk's blocks
    for raw in (st, ist, hst):
        raw.block_table = np.full_like(raw.block_table, -1)
        raw.block_table[0, CTX // 256 - 1], raw.block_table[0, CTX // 256] = 0, 1

    def compress(_):
        oc.compress_insert(mc, st, [CTX], cu, kv, lg2, np.ones(D), 1e-6, table, 0)
        oc.compress_insert(ic, ist, [CTX], cu, ikv, ilg, np.ones(D_IDX), 1e-6, itable, 0)
        oc.compress_insert(hc, hst, [CTX], cu, kv, lg1, np.ones(D), 1e-6, table, 0)

    from threadpoolctl import threadpool_limits
    threads = _blas_threads()
    res = {}
    for label, limit in (("", None), ("_1_thread", 1)):
        with threadpool_limits(limits=limit):
            nq, tq = _time_units(per_query, min_seconds)
            nc, tc = _time_units(compress, min(min_seconds, 5.0))
        per_tok = tq / nq + tc / (nc * n_tok)
        res["value" + label] = 1.0 / per_tok
        res["detail" + label] = f"{nq} queries in {tq:.1f} s, chunk compression {nc} x {n_tok} tokens in {tc:.1f} s"
    return {"value": res["value"], "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "value_1_thread": res["value_1_thread"], "cpu_model": cpu_model(), "nproc": os.cpu_count(),
            "sample": f"prefill chunk at {CTX}: per token = oracle index_topk + c4a attention + dense c128a attention "
                      f"of one of {n_sample} sampled queries (positions {pos[0]}..{pos[-1]}, evenly spaced) plus the "
                      f"oracle compression of the chunk into the three caches per token (measured on {n_tok} tokens "
                      f"of one sequence); {res['detail']} at {threads} BLAS threads; {res['detail_1_thread']} at 1 "
                      "thread"}


CPU_SIDE = {"c4a_fp8_1m": lambda sec: cpu_baseline_c4(sec), "c4a_fp8_fp4idx_1m": lambda sec: cpu_baseline_c4(sec, True),
            "c128a_dense_64k": cpu_baseline_c2, "prefill_chunk_256k": cpu_baseline_c5}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--layers", type=int, default=5)
    ap.add_argument("--workloads", default="c3,c4,c4f,c2,c5",
                    help="c3 = the headline 128K bf16 decode (always run); side workloads c4 = 1M fp8 decode, "
                         "c4f = the same with an MXFP4 indexer cache, c2 = c128a dense 64K decode, "
                         "c5 = 2048-token prefill chunk at 256K")
    ap.add_argument("--layers-c4", type=int, default=4)
    ap.add_argument("--layers-c2", type=int, default=32)
    ap.add_argument("--layers-c5", type=int, default=2)
    ap.add_argument("--steps-c5", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager-only", action="store_true", help="no HIP graphs (for profiler counter runs)")
    ap.add_argument("--cpu-seconds", type=float, default=5.0,
                    help="seconds of oracle work per workload and thread setting")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this path runs per GPU with no exchange (sequences shard by data "
              f"parallelism), and multi-GPU runs are not measured here; got --gpus {args.gpus}.", file=sys.stderr)
        sys.exit(2)
    global EAGER_ONLY
    EAGER_ONLY = args.eager_only
    lens = workload_lengths()
    total_ms, eager_ms, wall, stage_ms, copy_gbs, mode, modes, epilogue = run_gpu(args, lens)
    if total_ms is None:
        total_ms = eager_ms
    ms_step = total_ms / args.steps
    qps = B * args.steps / (total_ms / 1e3)
    ab = algorithmic_bytes(lens)
    path_bytes = ab["score"] + ab["select"] + ab["attend"]
    path_ms = stage_ms["score"] + stage_ms["select"] + stage_ms["attend"]
    score_gbs = ab["score"] / (stage_ms["score"] * 1e-3) / 1e9
    res = {
        "metric": METRIC,
        "value": round(qps, 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "step_mode": STEP_MODES[mode] + " (stage times below come from an eager pass with an event between stages)",
        "modes_ms_per_step": {"eager_with_stage_events": round(eager_ms / args.steps, 5),
                              **{k: round(v / args.steps, 5) for k, v in modes.items()}},
        "step_us_percentiles": epilogue.pop("step_us_percentiles"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "c4a bf16 decode, batch 32, context U[98304,131072], query at L, 64 heads x K=V 512 "
                               "(RoPE 64), indexer 64 heads x 128 WRELU, top-512 + window 128, 256-position pages",
                   "batch": B, "context_lo": LEN_LO, "context_hi": LEN_HI, "heads": H, "dim": D, "top_k": K_TOP,
                   "window": SWA, "layers_rotated": args.layers, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "kernel": "score_lt_kernel (index score)",
                     "achieved": round(score_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(score_gbs / HBM_PEAK_GBS, 4), "traffic": score_traffic("c3"),
                     "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE/WRITE_SIZE, copy-calibrated)",
                     "alg_bytes_per_launch": ab["score"], "avg_launch_us": round(stage_ms["score"] * 1e3, 2),
                     "frac_of_copy_bw": round(score_gbs / copy_gbs, 4)},
        "gathered_path": {"hbm_gbs": round(path_bytes / (path_ms * 1e-3) / 1e9, 1),
                          "frac_peak": round(path_bytes / (path_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                          "alg_bytes": path_bytes, "us": round(path_ms * 1e3, 2)},
        "stages_us": {k: round(v * 1e3, 2) for k, v in stage_ms.items()},
        "upstream_prepare": epilogue.pop("upstream_prepare"),
        "step_with_prepare_ms": dict(epilogue.pop("step_with_prepare_ms"),
                                     note="prepare_qk + compress + index + attend as one graph per layer: all on one "
                                          "stream, or the indexer pipeline on a second stream beside main compress + "
                                          "window insert"),
        "fp8_output_epilogue": epilogue,
        "copy_gbs": round(copy_gbs, 1),
        "wall_s_timed": round(wall, 3),
    }
    side = [w for w in args.workloads.split(",") if w and w != "c3"]
    if side:
        import torch
        import long_context_compressed_compress_amd as csa
        torch.cuda.empty_cache()
        res["workloads"] = {}
        for w in side:
            name, fn = SIDE[w]
            log(f"side workload {name}")
            t0 = time.time()
            try:
                res["workloads"][name] = fn(args, torch, csa)
            except torch.cuda.OutOfMemoryError as e:  # a device without room for the 200 GB pool; any other error
                res["workloads"][name] = {"error": f"{type(e).__name__}: {e}"}  # (a device fault above all) propagates
            torch.cuda.empty_cache()
            log(f"side workload {name} done in {time.time() - t0:.1f}s")
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        res["cpu_baseline"] = cpu_baseline(lens, args.cpu_seconds)
        for name, w in res.get("workloads", {}).items():
            if name in CPU_SIDE and "error" not in w:
                log(f"timing the CPU oracle on {name}")
                w["cpu_baseline"] = CPU_SIDE[name](args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
