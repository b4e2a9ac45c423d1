#!/usr/bin/env python3
"""Decode-step benchmark of one c4a compressed-sparse-attention layer on one MI355X.

Workload (the 128K bf16 decode configuration): batch 32, per-sequence context L_b ~ U{98304..131072}
with the query at position L_b; main cache bf16, one shared K=V head of dim 512 with RoPE on the last
64 dims; indexer cache bf16 of dim 128 (RoPE 64), 64 indexer heads with weights ~U(0,1),
score = sum_h w_h ReLU(q_h . k); top-512 compressed entries + 128-token raw window; 64 query heads;
256-position blocks at random physical pages. Inputs are synthetic (seeded), resident in HBM.

A step is one pass of the whole path for the batch: compress_insert of the decode token into the main
and the indexer cache, index score, top-k select, attention with fused inverse RoPE. Steps rotate over
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

# HBM bytes per launch of the index score kernel on this workload, from one FETCH_SIZE and one WRITE_SIZE
# counter run (FETCH_SIZE x 2.0, WRITE_SIZE x 1.0 as calibrated on a 1 GiB device copy). The figure holds only
# for the kernel source it was measured on; for any other source the traffic is reported as unknown.
SCORE_TRAFFIC = {"source": "long_context_compressed_compress_amd/csrc/index_topk.hip",
                 "sha256": "e985d1858f777b718e6b0dd3ac17f1793bcf0650d2d7850a419904cfff0e9f6c",
                 "bytes": 245996850}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def score_traffic():
    with open(os.path.join(ROOT, SCORE_TRAFFIC["source"]), "rb") as f:
        same = hashlib.sha256(f.read()).hexdigest() == SCORE_TRAFFIC["sha256"]
    return SCORE_TRAFFIC["bytes"] if same else None


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
    """Bytes the method must move per step (SURVEY-style accounting)."""
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
        csa.compress_insert(ly.cache, ly.state, ly.pos, ly.cu1, ly.kv1, ly.lg1, ly.gamma, 1e-6, rope_main, 1)
        csa.compress_insert(ly.icache, ly.istate, ly.pos, ly.cu1, ly.ikv1, ly.ilg1, ly.igamma, 1e-6, rope_idx, 1)
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
    total_ms = t_start.elapsed_time(t_end)
    names = ["compress", "score", "select", "attend"]
    stage_ms = {n: float(np.mean([e[j].elapsed_time(e[j + 1]) for e in evs])) for j, n in enumerate(names)}
    return total_ms, wall, stage_ms, copy_gbs


# ------------------------------------------------------------------ CPU baseline: the oracle, untuned
def cpu_baseline(lens, min_seconds=10.0, n_seq=8):
    import synth
    from oracle import attend as oa, codecs, compress as oc, index as oi, paging, rope as orope
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    g = synth.rng(CONFIG_ID, 40)
    seqs = []
    for b in range(n_seq):
        L = int(lens[b])
        nb = L // 256 + 1
        bt = np.arange(nb, dtype=np.int32)[None]
        tail = np.full((1, nb), -1, np.int32)  # window / state pages: only the last two blocks are mapped
        tail[0, nb - 2], tail[0, nb - 1] = 0, 1
        mc = oc.Cache(4, 8, D, R, "bf16", synth.normal_bf16_bits(g, (nb * 64, D)), None, bt)
        ic = oc.Cache(4, 8, D_IDX, R_IDX, "bf16", synth.normal_bf16_bits(g, (nb * 64, D_IDX)), None, bt)
        swa = oc.Raw("bf16", D, 0, synth.normal_bf16_bits(g, (512, D)), None, None, tail)
        st = oc.Raw("bf16", D, 2, synth.normal_bf16_bits(g, (512, D)), synth.normal_bf16_bits(g, (512, 2, D)), None, tail)
        ist = oc.Raw("bf16", D_IDX, 2, synth.normal_bf16_bits(g, (512, D_IDX)),
                     synth.normal_bf16_bits(g, (512, 2, D_IDX)), None, tail)
        new = (synth.normal_bf16_bits(g, (1, D)), synth.normal_bf16_bits(g, (1, 2, D)),
               synth.normal_bf16_bits(g, (1, D_IDX)), synth.normal_bf16_bits(g, (1, 2, D_IDX)))
        q = codecs.load_rows(synth.normal_bf16_bits(g, (1, H, D)), "bf16")
        qi = codecs.load_rows(synth.normal_bf16_bits(g, (1, H_IDX, D_IDX)), "bf16")
        w = synth.uniform_f32(g, (1, H_IDX))
        seqs.append((L, mc, ic, swa, st, ist, new, q, qi, w))
    table = orope.rope_table(LEN_HI + 2, R)
    itable = orope.rope_table(LEN_HI + 2, R_IDX)
    one = np.array([0, 1], np.int32)
    queries, t0 = 0, time.time()
    while True:
        for (L, mc, ic, swa, st, ist, new, q, qi, w) in seqs:
            oc.compress_insert(mc, st, [L], one, new[0], new[1], np.ones(D), 1e-6, table, 1)
            oc.compress_insert(ic, ist, [L], one, new[2], new[3], np.ones(D_IDX), 1e-6, itable, 1)
            idx, _, _ = oi.index_topk(ic, [0], [L], qi, w, oi.WRELU, K_TOP)
            oa.attend(mc, swa, SWA, [0], [L], q, idx, 1.0 / math.sqrt(D), True, table)
            queries += 1
        if time.time() - t0 >= min_seconds:
            break
    dt = time.time() - t0
    return {"value": queries / dt, "unit": "queries/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{queries} decode queries ({n_seq} sequences of the workload, contexts "
                      f"{int(min(lens[:n_seq]))}-{int(max(lens[:n_seq]))}, repeated) through the numpy fp64 oracle: "
                      f"compress_insert x2, index_topk, attend with inverse RoPE; {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--layers", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this path runs per GPU with no exchange (sequences shard by data "
              f"parallelism), and multi-GPU runs are not part of this build; got --gpus {args.gpus}.", file=sys.stderr)
        sys.exit(2)
    lens = workload_lengths()
    total_ms, wall, stage_ms, copy_gbs = run_gpu(args, lens)
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
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "c4a bf16 decode, batch 32, context U[98304,131072], query at L, 64 heads x K=V 512 "
                               "(RoPE 64), indexer 64 heads x 128 WRELU, top-512 + window 128, 256-position pages",
                   "batch": B, "context_lo": LEN_LO, "context_hi": LEN_HI, "heads": H, "dim": D, "top_k": K_TOP,
                   "window": SWA, "layers_rotated": args.layers, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "kernel": "score_mfma_kernel (index score)",
                     "achieved": round(score_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(score_gbs / HBM_PEAK_GBS, 4), "traffic": score_traffic(),
                     "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE/WRITE_SIZE, copy-calibrated)",
                     "alg_bytes_per_launch": ab["score"], "avg_launch_us": round(stage_ms["score"] * 1e3, 2),
                     "frac_of_copy_bw": round(score_gbs / copy_gbs, 4)},
        "gathered_path": {"hbm_gbs": round(path_bytes / (path_ms * 1e-3) / 1e9, 1),
                          "frac_peak": round(path_bytes / (path_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                          "alg_bytes": path_bytes, "us": round(path_ms * 1e3, 2)},
        "stages_us": {k: round(v * 1e3, 2) for k, v in stage_ms.items()},
        "copy_gbs": round(copy_gbs, 1),
        "wall_s_timed": round(wall, 3),
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        res["cpu_baseline"] = cpu_baseline(lens, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
