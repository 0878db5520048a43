#!/usr/bin/env python
"""Benchmark of two-stage GQA block-sparse attention on one MI355X.

Headline: sparse decode at 1M-token context (batch 1, 32 query / 8 KV heads, head_dim 128,
64-token blocks, top-64 blocks, bf16 paged KV cache with permuted pages). One step = one full
decode step: append the new token and refresh its block summary, score every block, top-k,
gather-attend over the selected blocks, merge. Also reported: selected-KV bandwidth of the
attend stage against HBM peak, the stage-1 scan bandwidth, sparse prefill TFLOP/s (4096 new
tokens on a 262,144-token cache, top-32 + diagonal per 64-query tile), and the CPU oracle's
rate on a bounded sample of the same decode workload.

Timing: inputs are resident in HBM before the timed region; steps rotate over --layers
independent caches (4 x 4 GiB by default, far beyond the 256 MB infinity cache) and over fresh
queries; the steps are captured once in a HIP graph and replayed; HIP events on the launch
stream bracket exactly --steps steps, with a device synchronisation on both sides.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse decode tokens/s + KV GB/s (% HBM peak) at 1M ctx; prefill TFLOP/s"
HBM_PEAK_GBPS = 8000.0
BF16_PEAK_TFLOPS = 2500.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def selected_kv_bytes(idx, lens, P=64, D=128, elem=2):
    """K+V bytes the attend stage must read: valid tokens of every selected block."""
    import numpy as np
    idx = idx.cpu().numpy()
    total = 0
    for b in range(idx.shape[0]):
        n = int(lens[b])
        nb = (n + P - 1) // P
        for g in range(idx.shape[1]):
            for j in idx[b, g]:
                if 0 <= j < nb:
                    total += min(P, n - j * P) * D * elem * 2
    return total


def timed_graph(fn_steps, nsteps_graph, torch, eager_first=True):
    """Capture nsteps_graph calls of fn_steps(i) in a HIP graph; with eager_first, one eager call
    on the capture stream first (so every kernel's code object is loaded before the capture)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    if eager_first:
        with torch.cuda.stream(s):
            fn_steps(0)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(nsteps_graph):
            fn_steps(i)
    torch.cuda.synchronize()
    return g


def single_steps(fn_steps, nsteps, torch, scrub_bytes=1 << 30):
    """Median times of single steps, each a one-step HIP graph timed alone (so the graph's own
    launch is inside the interval): (warm, cold). Warm steps follow each other; each cold step
    follows a write of scrub_bytes to an unrelated buffer, outside the timed interval, so no
    input of the step is left in the infinity cache or an L2 by the step before."""
    graphs = [timed_graph(lambda i, j=j: fn_steps(j), 1, torch) for j in range(nsteps)]
    scrub = torch.empty(scrub_bytes, dtype=torch.uint8, device="cuda")
    res = []
    for cold in (False, True):
        times = []
        for rep in range(3):
            for j, g in enumerate(graphs):
                if cold:
                    scrub.fill_((rep + j) & 0xff)
                start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                start.record()
                g.replay()
                end.record()
                torch.cuda.synchronize()
                times.append(start.elapsed_time(end) / 1e3)
        res.append(float(sorted(times)[len(times) // 2]))
    del graphs, scrub
    return res[0], res[1]


def measured_peaks(torch, msa, read_bytes=4 << 30, mfma_workgroups=1024, mfma_iters=4000):
    """The GPU's achievable HBM read rate (msa_probe_hbm_read over a read_bytes buffer, far beyond
    the infinity cache) and bf16 MFMA rate (msa_probe_mfma_bf16: register operands, no memory
    traffic), each the best of five launches timed with HIP events on the launch stream."""
    dev = torch.device("cuda")

    def best(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            start.record()
            fn()
            end.record()
            torch.cuda.synchronize()
            ts.append(start.elapsed_time(end) / 1e3)
        return min(ts)
    buf = torch.empty(read_bytes, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    sink = torch.empty(msa.PROBE_READ_SINK_FLOATS, dtype=torch.float32, device=dev)
    t_read = best(lambda: msa.msa_probe_hbm_read(buf, sink))
    del buf, sink
    msink = torch.empty(4 * mfma_workgroups, dtype=torch.float32, device=dev)
    t_mfma = best(lambda: msa.msa_probe_mfma_bf16(msink, mfma_workgroups, mfma_iters))
    flops = float(mfma_workgroups) * 4 * mfma_iters * 4 * 32768
    hbm, mf = read_bytes / t_read / 1e9, flops / t_mfma / 1e12
    log("measured peaks: HBM read %.0f GB/s (%.0f %% of %.0f), bf16 MFMA %.0f TFLOP/s (%.0f %% of %.0f)"
        % (hbm, 100 * hbm / HBM_PEAK_GBPS, HBM_PEAK_GBPS, mf, 100 * mf / BF16_PEAK_TFLOPS, BF16_PEAK_TFLOPS))
    return {"hbm_read_GBps": hbm, "hbm_read_frac_of_published": hbm / HBM_PEAK_GBPS,
            "bf16_mfma_TFLOPs": mf, "bf16_mfma_frac_of_published": mf / BF16_PEAK_TFLOPS,
            "method": "msa_probe_hbm_read: %d MiB streamed once per launch, 16 B loads, 8 in flight per thread; "
                      "msa_probe_mfma_bf16: %d workgroups x 4 waves x %d rounds of 4 independent "
                      "32x32x16 bf16 MFMAs; best of 5 launches each" % (read_bytes >> 20, mfma_workgroups,
                                                                         mfma_iters)}


GRAPH_MAX_STEPS = 200


def time_exact_steps(fn, steps, warmup, torch):
    """Seconds per step over exactly `steps` calls fn(0), fn(1), ... replayed from HIP graphs of at
    most GRAPH_MAX_STEPS calls (a full graph replayed steps // per times, then a graph of the
    remainder), after exactly `warmup` untimed calls fn(0) .. fn(warmup - 1) on the same stream.
    HIP events on the launch stream bracket the replays, with a device synchronisation on both
    sides, so the launch of each graph is inside the timed interval."""
    per = max(1, min(GRAPH_MAX_STEPS, steps))
    full, rem = divmod(steps, per)
    g_full = timed_graph(fn, per, torch)
    g_rem = timed_graph(fn, rem, torch, eager_first=False) if rem else None
    torch.cuda.synchronize()
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(full):
        g_full.replay()
    if g_rem is not None:
        g_rem.replay()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / 1e3 / steps


def run_graph(g, replays, torch):
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(replays):
        g.replay()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / 1e3


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--layers", type=int, default=16,
                    help="independent caches rotated over the steps (16 x 4 GiB of K/V at 1M tokens; the "
                         "summaries and selected K/V the steps read total about 1.3 GB, about five times "
                         "the 256 MB infinity cache)")
    ap.add_argument("--workload", default="decode_bf16_1m_paged")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-batched", action="store_true", help="skip the batch-8 x 131072-token decode line")
    ap.add_argument("--no-mixed", action="store_true", help="skip the batch-32 mixed-length decode line")
    ap.add_argument("--no-large-k", action="store_true", help="skip the 1M-token k=1024 operating-point line")
    ap.add_argument("--no-index", action="store_true", help="skip the 1M-token index-branch select line")
    ap.add_argument("--no-bf16-summaries", action="store_true", help="skip the 1M-token bf16 summary-pool line")
    ap.add_argument("--no-forced", action="store_true", help="skip the 1M-token forced sink / local block line")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--counters", action="store_true",
                    help="counter pass: eager launches of the scoring kernel over the rotating caches, of the "
                         "k = 1024 attend and of the index-branch select, then of a 256 MiB device copy (the "
                         "byte-count calibration), for rocprofv3 --pmc; no timing")
    ap.add_argument("--prefill-only", action="store_true",
                    help="only the prefill chunk line (its own JSON object), then a 256 MiB device copy (the "
                         "byte-count calibration), e.g. for rocprofv3 --pmc passes over the MFMA attend")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (use --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import long_context_sparse_select_amd as msa
    from synth import make_decode_case_torch, make_prefill_case_torch, workload

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    if args.prefill_only:
        rec = {"prefill": bench_prefill(args, torch, np, msa, make_prefill_case_torch, workload, dev)}
        calibration_copies(torch, dev)   # after the timing: the byte-count calibration of counter passes
        rec["copy_launches"], rec["copy_bytes"] = 4, COPY_BYTES
        print(json.dumps(rec), flush=True)
        return
    kw = workload(args.workload, seed=args.seed)
    L = max(1, args.layers)
    log("generating %d caches of %s" % (L, args.workload))
    caches, cases = [], []
    for layer in range(L):
        kwl = dict(kw, seed=args.seed + 1000 * layer)
        c = make_decode_case_torch(device=dev, **kwl)
        table = torch.from_numpy(c.block_table).to(dev)
        lens = torch.from_numpy(c.seq_lens).to(dev)
        S = torch.empty((c.num_pages, c.Hkv, c.D), dtype=torch.float32, device=dev)
        cache = msa.KVCache(c.k_pool, c.v_pool, S, table, lens)
        cfg = msa.make_config(c.Hq, c.Hkv, c.top_k, dtype=c.dtype, softmax_scale=c.scale)
        msa.msa_build_summaries(cfg, cache, c.B, c.max_seq_len)
        caches.append(cache)
        cases.append(c)
    c0 = cases[0]
    B, Hq, Hkv, D, k = c0.B, c0.Hq, c0.Hkv, c0.D, c0.top_k
    max_len = c0.max_seq_len
    tdt = torch.bfloat16 if c0.dtype == "bf16" else torch.float32
    R = 8
    gen = torch.Generator(device=dev)
    gen.manual_seed(args.seed + 77)
    q_ring = [torch.randn((B, Hq, D), generator=gen, device=dev).to(tdt) for _ in range(R)]
    kn_ring = [torch.randn((B, Hkv, D), generator=gen, device=dev).to(tdt) for _ in range(R)]
    vn_ring = [torch.randn((B, Hkv, D), generator=gen, device=dev).to(tdt) for _ in range(R)]
    out = torch.empty((B, Hq, D), dtype=tdt, device=dev)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    idx_bufs = [torch.empty((B, Hkv, k), dtype=torch.int32, device=dev) for _ in range(L)]
    ws = torch.empty(msa.msa_workspace_size(cfg, msa.MSA_OP_DECODE, B, max_len), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def decode(i):
        layer = i % L
        msa.msa_decode_step(cfg, q_ring[i % R], caches[layer], B, max_len, out, k_new=kn_ring[i % R],
                            v_new=vn_ring[i % R], idx_out=idx_bufs[layer], lse_out=lse, workspace=ws)

    def select(i):
        layer = i % L
        msa.msa_select(cfg, q_ring[i % R], caches[layer], B, max_len, idx_bufs[layer], workspace=ws)

    def attend(i):
        layer = i % L
        msa.msa_attend(cfg, q_ring[i % R], caches[layer], B, max_len, idx_bufs[layer], out, lse_out=lse,
                       workspace=ws)

    mb = (max_len + 63) // 64
    sc_buf = torch.empty((B, Hkv, mb), dtype=torch.float32, device=dev)
    if args.counters:
        counter_pass(args, torch, msa, cfg, q_ring, caches, B, max_len, sc_buf, dev)
        return

    # exactly --steps steps (step i: cache i % L, query i % R) from graphs of up to 200 steps, so the
    # launch of a graph (~9 us, see single_step_warm) is spread over many steps, after exactly
    # --warmup untimed steps
    rot = L * R // math.gcd(L, R) if L * R <= 64 else L
    steps, warmup = max(1, args.steps), max(0, args.warmup)
    per_graph = min(GRAPH_MAX_STEPS, steps)

    def timed(fn):
        """seconds per call of fn(i) over the same schedule as the timed steps"""
        return time_exact_steps(fn, steps, warmup, torch)

    t_step = timed(decode)
    log("decode step: %.2f us (%d steps timed after %d warmup steps, %d caches rotated)"
        % (t_step * 1e6, steps, warmup, L))
    t_warm1, t_cold = single_steps(decode, rot, torch)
    log("single decode steps timed alone (graph launch included): %.2f us warm, %.2f us after a 1 GiB "
        "scrub write" % (t_warm1 * 1e6, t_cold * 1e6))
    # stage timings: Step 1 scoring alone (one kernel), Step 1 (score + top-k), Step 2 (attend + merge)
    # the scoring kernel alone streams summaries only: it rotates over SCORE_POOLS summary pools (the
    # caches' own plus copies), ~1 GB at 1M tokens, so no pool can stay in the 256 MB infinity cache
    # from one launch to its next use and the rate is HBM's
    score_caches = list(caches)
    while len(score_caches) < SCORE_POOLS:
        base = caches[len(score_caches) % L]
        score_caches.append(msa.KVCache(base.k_pages, base.v_pages, base.summaries.clone(), base.block_table,
                                        base.seq_lens))
    P = len(score_caches)
    g_score = timed_graph(lambda i: msa.msa_score(cfg, q_ring[i % R], score_caches[i % P], B, max_len, sc_buf),
                          P, torch)
    run_graph(g_score, 2, torch)
    n_score = max(2, steps // P)
    t_score = run_graph(g_score, n_score, torch) / (n_score * P)
    del g_score, score_caches
    t_sel = timed(select)
    # Step 2 alone: one selected list per (cache, query) pair, L * R lists (512 MiB of selected K/V
    # at 1M tokens, beyond the infinity cache), attended in rotation
    att_idx = [[torch.empty_like(idx_bufs[0]) for _ in range(R)] for _ in range(L)]
    for l in range(L):
        for r in range(R):
            msa.msa_select(cfg, q_ring[r], caches[l], B, max_len, att_idx[l][r], workspace=ws)
    PA = L * R
    g_att = timed_graph(lambda i: msa.msa_attend(cfg, q_ring[(i // L) % R], caches[i % L], B, max_len,
                                                 att_idx[i % L][(i // L) % R], out, lse_out=lse, workspace=ws),
                        PA, torch)
    run_graph(g_att, 2, torch)
    n_att = max(2, steps // PA)
    t_att = run_graph(g_att, n_att, torch) / (n_att * PA)
    del g_att
    torch.cuda.synchronize()
    elem = 2 if c0.dtype == "bf16" else 4
    kv_bytes = float(np.mean([selected_kv_bytes(att_idx[l][r], cases[l].seq_lens, elem=elem)
                              for l in range(L) for r in range(R)]))
    nb_tot = sum((int(n) + 63) // 64 for n in c0.seq_lens)
    # algorithmic bytes of one scoring launch: summaries + block-table entries read, scores written
    score_bytes = nb_tot * Hkv * D * 4 + nb_tot * 4 + nb_tot * Hkv * 4 + B * Hq * D * elem
    kv_gbps = kv_bytes / t_att / 1e9
    step_bytes = score_bytes + kv_bytes + 2 * B * Hq * D * elem + B * Hkv * k * 4
    working_set = L * step_bytes   # what the rotation of the timed steps reads, in distinct bytes
    score_gbps = score_bytes / t_score / 1e9
    log("score %.2f us (%.0f GB/s); select %.2f us; attend %.2f us (%.0f GB/s of selected KV)"
        % (t_score * 1e6, score_gbps, t_sel * 1e6, t_att * 1e6, kv_gbps))

    rec = {
        "metric": METRIC,
        "value": B / t_step,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": t_step * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": c0.dtype,
        "data": "synthetic (seeded N(0,1) q/K/V, planted blocks, permuted 64-token pages)",
        "config": {"workload": args.workload, "batch": B, "context": int(max_len), "q_heads": Hq,
                   "kv_heads": Hkv, "head_dim": D, "block": 64, "top_k": k,
                   "caches_rotated": L, "step_working_set_bytes": working_set,
                   "graph_steps": per_graph},
        "kv_GBps": kv_gbps,
        "kv_hbm_frac": kv_gbps / HBM_PEAK_GBPS,
        # the whole step's algorithmic bytes (summaries, table, scores, selected K/V, q twice, o, the
        # index lists) over the step time, beside the selected-KV rate so Step 1's cost is not hidden
        "step_GBps": step_bytes / t_step / 1e9,
        "step_hbm_frac": step_bytes / t_step / 1e9 / HBM_PEAK_GBPS,
        "step_bytes": step_bytes,
        "roofline": {"bound": "hbm", "kernel": "k_score_decode (msa_score): Step 1 block scoring",
                     "achieved": score_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": score_gbps / HBM_PEAK_GBPS, "traffic": None, "traffic_detail": None,
                     "bytes_per_launch": score_bytes, "us_per_launch": t_score * 1e6},
        "stages_us": {"score": t_score * 1e6, "select": t_sel * 1e6, "attend_merge": t_att * 1e6,
                      "step": t_step * 1e6, "single_step_warm": t_warm1 * 1e6,
                      "single_step_cold": t_cold * 1e6},
        "attend_roofline": {"bound": "hbm", "kernel": "k_attend_decode + k_merge (msa_attend)",
                            "achieved": kv_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                            "frac": kv_gbps / HBM_PEAK_GBPS, "bytes_per_launch": kv_bytes},
    }
    if not args.no_large_k:
        rec["large_k"] = bench_large_k(args, torch, np, msa, caches, cases, q_ring, kn_ring, vn_ring, L, R, rot)
    if not args.no_bf16_summaries:
        rec["bf16_summaries"] = bench_bf16_summaries(args, torch, np, msa, caches, cases, q_ring, kn_ring, vn_ring, L,
                                                     R, rot)
    if not args.no_forced:
        rec["forced_blocks"] = bench_forced(args, torch, np, msa, caches, cases, q_ring, kn_ring, vn_ring, L, R, rot)
    tr = recorded_traffic(score_bytes)
    if tr is not None:
        rec["roofline"]["traffic"] = tr["bytes_per_launch"]
        rec["roofline"]["traffic_detail"] = tr
    del caches, cases, q_ring, kn_ring, vn_ring, idx_bufs, ws
    torch.cuda.empty_cache()
    if not args.no_batched:
        rec["batched_decode"] = bench_batched(args, torch, np, msa, make_decode_case_torch, workload, dev)
        torch.cuda.empty_cache()
    if not args.no_mixed:
        rec["mixed_batch"] = bench_mixed(args, torch, np, msa, make_decode_case_torch, workload, dev)
        torch.cuda.empty_cache()
    if not args.no_index:
        rec["index_select"] = bench_index(args, torch, np, msa, dev)
        torch.cuda.empty_cache()

    # ---- prefill
    if not args.no_prefill:
        try:
            rec["prefill"] = bench_prefill(args, torch, np, msa, make_prefill_case_torch, workload, dev)
        except msa.MsaError as e:
            log("prefill skipped: %s" % e)
            rec["prefill"] = None
    # ---- the GPU's own denominators, measured beside the published ones
    peaks = measured_peaks(torch, msa)
    rec["measured_peaks"] = peaks
    rec["roofline"]["frac_of_measured"] = rec["roofline"]["achieved"] / peaks["hbm_read_GBps"]
    rec["attend_roofline"]["frac_of_measured"] = rec["attend_roofline"]["achieved"] / peaks["hbm_read_GBps"]
    if rec.get("prefill"):
        rec["prefill"]["bf16_mfma_frac_of_measured"] = rec["prefill"]["TFLOPs"] / peaks["bf16_mfma_TFLOPs"]
        pr = rec["prefill"]["roofline"]
        pr["frac_of_measured"] = pr["achieved"] / (peaks["hbm_read_GBps"] if pr["bound"] == "hbm"
                                                   else peaks["bf16_mfma_TFLOPs"])
    # ---- CPU oracle baseline (regenerates the first cache of the workload: same seed, same data)
    if not args.no_cpu_baseline:
        c = make_decode_case_torch(device=dev, **dict(kw, seed=args.seed))
        rec["cpu_baseline"] = cpu_baseline(args, c, torch, np)
        del c
    print(json.dumps(rec), flush=True)


COPY_BYTES = 256 << 20
SCORE_POOLS = 16
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "k_score_decode_1m_hbm_traffic.md")
SCORE_SOURCES = ("long_context_sparse_select_amd/csrc/score.hip", "long_context_sparse_select_amd/csrc/common.h")


def counter_pass(args, torch, msa, cfg, q_ring, caches, B, max_len, sc_buf, dev):
    """Eager launches for rocprofv3 --pmc: msa_score (one k_score_decode dispatch each) over the
    rotating caches, then a device copy of COPY_BYTES (its FETCH_SIZE / WRITE_SIZE per dispatch
    calibrate the counters against a known byte count)."""
    L, R = len(caches), len(q_ring)
    n = max(8, args.steps // 10)
    for i in range(2 * L):
        msa.msa_score(cfg, q_ring[i % R], caches[i % L], B, max_len, sc_buf)
    for i in range(n):
        msa.msa_score(cfg, q_ring[i % R], caches[i % L], B, max_len, sc_buf)
    # whole decode steps without a new token (k_score_decode, k_decode_select_attend, k_merge
    # dispatches): the selected K/V of each step, counted from its lists
    import numpy as np
    Hq0, Hkv0 = int(cfg.num_q_heads), int(cfg.num_kv_heads)
    dout = torch.empty((B, Hq0, 128), dtype=q_ring[0].dtype, device=dev)
    dws = torch.empty(msa.msa_workspace_size(cfg, msa.MSA_OP_DECODE, B, max_len), dtype=torch.uint8, device=dev)
    didx = [torch.empty((B, Hkv0, int(cfg.top_k)), dtype=torch.int32, device=dev) for _ in range(L)]
    for i in range(n):
        msa.msa_decode_step(cfg, q_ring[i % R], caches[i % L], B, max_len, dout, idx_out=didx[i % L], workspace=dws)
    torch.cuda.synchronize()
    step_kv_bytes = float(np.mean([selected_kv_bytes(didx[l], caches[l].seq_lens.cpu().numpy(),
                                                     elem=2 if int(cfg.q_dtype) == msa.MSA_BF16 else 4)
                                   for l in range(min(L, n))]))
    # the k = 1024 operating point: one selection per cache, then eager attends over those lists
    # (k_attend_decode_mfma + k_merge dispatches; the selections add k_score_decode dispatches
    # of the same work)
    bf16 = int(cfg.q_dtype) == msa.MSA_BF16
    cfg_k = msa.make_config(int(cfg.num_q_heads), int(cfg.num_kv_heads), 1024, dtype="bf16" if bf16 else "f32",
                            softmax_scale=float(cfg.softmax_scale))
    Hq, Hkv = int(cfg.num_q_heads), int(cfg.num_kv_heads)
    idx = [torch.empty((B, Hkv, 1024), dtype=torch.int32, device=dev) for _ in range(L)]
    for l in range(L):
        msa.msa_select(cfg_k, q_ring[l % R], caches[l], B, max_len, idx[l])
    out = torch.empty((B, Hq, 128), dtype=q_ring[0].dtype, device=dev)
    for i in range(n):
        msa.msa_attend(cfg_k, q_ring[i % R], caches[i % L], B, max_len, idx[i % L], out)
    torch.cuda.synchronize()
    attend_bytes = float(np.mean([selected_kv_bytes(idx[l], caches[l].seq_lens.cpu().numpy(), elem=2 if bf16 else 4)
                                  for l in range(L)]))
    # the index branch on two 1M-token index-key caches (k_score_index dispatches)
    from synth import make_index_case_torch
    icases = [make_index_case_torch(B=1, Hkv=8, lens=[1 << 20], top_k=64, dtype="bf16", permute=True,
                                    plant=("count", 16), seed=args.seed + 1000 * l, device=dev) for l in range(2)]
    icfg = msa.make_config(8, 8, 64, dtype="bf16")
    itabs = [(torch.from_numpy(c.block_table).to(dev), torch.from_numpy(c.seq_lens).to(dev)) for c in icases]
    iidx = torch.empty((1, 8, 64), dtype=torch.int32, device=dev)
    for i in range(n):
        c = icases[i % 2]
        msa.msa_select_index(icfg, c.q_idx, c.index_keys, itabs[i % 2][0], itabs[i % 2][1], 1, c.max_seq_len, iidx)
    torch.cuda.synchronize()
    nbi = (icases[0].max_seq_len + 63) // 64
    index_bytes = nbi * 64 * 128 * 2 + nbi * 4 + 8 * 128 * 2 + 8 * nbi * 4
    del icases
    calibration_copies(torch, dev)
    print(json.dumps({"counter_pass": args.workload, "score_launches": n + 2 * L + L + n,
                      "decode_step_launches": n, "decode_step_selected_kv_bytes": step_kv_bytes,
                      "attend_launches": n,
                      "attend_bytes_per_launch": attend_bytes, "index_launches": n,
                      "index_score_bytes_per_launch": index_bytes, "copy_launches": 4,
                      "copy_bytes": COPY_BYTES}), flush=True)


def calibration_copies(torch, dev, n=4):
    """n device copies of COPY_BYTES: a kernel of known traffic, which scales the FETCH_SIZE /
    WRITE_SIZE counts of the same rocprofv3 pass to bytes"""
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
    src.fill_(1)
    dst = torch.empty_like(src)
    for _ in range(n):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def sources_digest(paths):
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic(algorithmic_bytes):
    """HBM bytes per k_score_decode launch from the committed rocprofv3 --pmc record, or None when
    there is no record or the kernel's sources changed since the counters were taken."""
    try:
        with open(TRAFFIC_RECORD) as f:
            for line in f:
                if line.startswith("traffic-json: "):
                    rec = json.loads(line[len("traffic-json: "):])
                    if rec.get("sources_digest") != sources_digest(SCORE_SOURCES):
                        return None
                    return {"bytes_per_launch": rec["bytes_per_launch"],
                            "vs_algorithmic": rec["bytes_per_launch"] / algorithmic_bytes,
                            "fetch_bytes": rec["fetch_bytes"], "write_bytes": rec["write_bytes"],
                            "record": os.path.relpath(TRAFFIC_RECORD, ROOT)}
    except (OSError, ValueError, KeyError):
        return None
    return None


def bench_prefill(args, torch, np, msa, make_prefill_case_torch, workload, dev):
    kw = workload("prefill_bf16_4k_on_256k", seed=args.seed)
    p = make_prefill_case_torch(device=dev, **kw)
    table = torch.from_numpy(p.block_table).to(dev)
    S = torch.empty((p.num_pages, p.Hkv, p.D), dtype=torch.float32, device=dev)
    cache = msa.KVCache(p.k_pool, p.v_pool, S, table, torch.tensor([p.past_len], dtype=torch.int32, device=dev))
    cfg = msa.make_config(p.Hq, p.Hkv, p.top_k, dtype="bf16", softmax_scale=p.scale)
    msa.msa_build_summaries(cfg, cache, 1, p.past_len)
    out = torch.empty_like(p.q)
    ntiles = (p.T + 63) // 64
    idx = torch.empty((ntiles, p.Hkv, p.top_k + 1), dtype=torch.int32, device=dev)
    ws = torch.empty(msa.msa_workspace_size(cfg, msa.MSA_OP_PREFILL, 1, p.past_len + p.T, p.T),
                     dtype=torch.uint8, device=dev)

    def chunk(i):
        msa.msa_prefill_chunk(cfg, p.q, p.k_new, p.v_new, cache, p.past_len, p.T, out, idx_out=idx, workspace=ws)

    chunk(0)
    torch.cuda.synchronize()
    # four chunks per graph (the chunk is idempotent: the same tokens appended at the same positions),
    # so the launch of the graph itself is amortised as for the decode steps
    per = 4
    g = timed_graph(chunk, per, torch)
    run_graph(g, 2, torch)
    n = 6
    t = run_graph(g, n, torch) / (n * per)
    # Step 2 alone (msa_prefill_attend: one k_attend_prefill launch) over the chunk's own lists
    ga = timed_graph(lambda i: msa.msa_prefill_attend(cfg, p.q, cache, p.past_len, p.T, idx, out), per, torch)
    run_graph(ga, 2, torch)
    t_att = run_graph(ga, n, torch) / (n * per)
    del g, ga
    pairs = 0
    for tau in range(ntiles):
        rows = min(64, p.T - tau * 64)
        keff = min(p.top_k, p.past_len // 64 + tau)
        pairs += rows * 64 * keff + rows * (rows + 1) // 2
    flops = 4.0 * p.D * p.Hq * pairs
    # every (tile, group) reads the K and V of its diagonal block and of its selected blocks; the
    # launch also reads the chunk's queries and writes its outputs (bf16)
    blocks = p.Hkv * sum(1 + min(p.top_k, p.past_len // 64 + tau) for tau in range(ntiles))
    kv_bytes = blocks * 2 * 64 * p.D * 2
    hbm_bytes = kv_bytes + 2 * p.T * p.Hq * p.D * 2
    tf = flops / t / 1e12
    tfa = flops / t_att / 1e12
    kv_gbps = kv_bytes / t_att / 1e9
    hbm_gbps = hbm_bytes / t_att / 1e9
    log("prefill chunk: %.1f us, %.1f TFLOP/s (causal-visible, whole chunk); attend alone %.1f us, %.1f TFLOP/s, "
        "%.0f GB/s (selected K/V, queries, outputs)" % (t * 1e6, tf, t_att * 1e6, tfa, hbm_gbps))
    # the kernel's two floors: its FLOPs at the bf16 MFMA peak and its K/V bytes at the HBM peak;
    # the larger one is the bound
    views = {"mfma": {"achieved": tfa, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": tfa / BF16_PEAK_TFLOPS,
                      "floor_us": flops / (BF16_PEAK_TFLOPS * 1e12) * 1e6},
             "hbm": {"achieved": hbm_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": hbm_gbps / HBM_PEAK_GBPS,
                     "floor_us": hbm_bytes / (HBM_PEAK_GBPS * 1e9) * 1e6}}
    bound = max(views, key=lambda v: views[v]["floor_us"])
    roof = {"bound": bound, "kernel": "k_attend_prefill (msa_prefill_attend): Step 2 of the chunk"}
    roof.update({k: views[bound][k] for k in ("achieved", "peak", "unit", "frac")})
    roof.update({"flops_per_launch": flops, "hbm_bytes_per_launch": hbm_bytes, "kv_bytes_per_launch": kv_bytes,
                 "us_per_launch": t_att * 1e6,
                 "flops_rule": "4 * 128 * Hq * (causal-visible query-key pairs of the selected blocks)",
                 "hbm_bytes_rule": "Hkv * sum over tiles of (1 + k_eff) blocks * (K + V) * 64 tokens * 128 dims * 2 B"
                                   " + queries read + outputs written (T * Hq * 128 * 2 B each)",
                 "views": views})
    return {"workload": "prefill_bf16_4k_on_256k", "chunk_us": t * 1e6, "TFLOPs": tf,
            "bf16_mfma_frac": tf / BF16_PEAK_TFLOPS, "flops": flops,
            "note": "whole chunk: append + summaries + tile query + score + top-k + MFMA attend",
            "roofline": roof}


def bench_batched(args, torch, np, msa, make_decode_case_torch, workload, dev, L=8, R=8):
    """The batch-8, 131,072-token workload (32 q / 8 kv heads, k = 32, in-order pages): whole decode
    steps (append + score + top-k + attend + merge), the scoring kernel alone and the attend stage
    alone. L caches (4 GiB of K/V each) rotated with R fresh queries: a step reads 64 MiB of
    summaries and 64 MiB of selected K/V, so the rotation of each stage reads several times the
    256 MB infinity cache."""
    kw = workload("decode_bf16_b8_128k", seed=args.seed)
    caches, cases = [], []
    for layer in range(L):
        c = make_decode_case_torch(device=dev, **dict(kw, seed=args.seed + 1000 * layer))
        table = torch.from_numpy(c.block_table).to(dev)
        lens = torch.from_numpy(c.seq_lens).to(dev)
        S = torch.empty((c.num_pages, c.Hkv, c.D), dtype=torch.float32, device=dev)
        cache = msa.KVCache(c.k_pool, c.v_pool, S, table, lens)
        cfg = msa.make_config(c.Hq, c.Hkv, c.top_k, dtype="bf16", softmax_scale=c.scale)
        msa.msa_build_summaries(cfg, cache, c.B, c.max_seq_len)
        caches.append(cache)
        cases.append(c)
    c0 = cases[0]
    B, Hq, Hkv, D, k, max_len = c0.B, c0.Hq, c0.Hkv, c0.D, c0.top_k, c0.max_seq_len
    gen = torch.Generator(device=dev)
    gen.manual_seed(args.seed + 77)
    q_ring = [torch.randn((B, Hq, D), generator=gen, device=dev).to(torch.bfloat16) for _ in range(R)]
    kn_ring = [torch.randn((B, Hkv, D), generator=gen, device=dev).to(torch.bfloat16) for _ in range(R)]
    vn_ring = [torch.randn((B, Hkv, D), generator=gen, device=dev).to(torch.bfloat16) for _ in range(R)]
    out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    idx_bufs = [torch.empty((B, Hkv, k), dtype=torch.int32, device=dev) for _ in range(L)]
    sc = torch.empty((B, Hkv, (max_len + 63) // 64), dtype=torch.float32, device=dev)
    ws = torch.empty(msa.msa_workspace_size(cfg, msa.MSA_OP_DECODE, B, max_len), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    per = L * R // math.gcd(L, R)
    per = per * max(1, 64 // per)
    n_rep = 10

    def timed(fn, n=per):
        g = timed_graph(fn, n, torch)
        run_graph(g, 2, torch)
        return run_graph(g, n_rep, torch) / (n * n_rep)
    t_step = timed(lambda i: msa.msa_decode_step(cfg, q_ring[i % R], caches[i % L], B, max_len, out,
                                                 k_new=kn_ring[i % R], v_new=vn_ring[i % R], idx_out=idx_bufs[i % L],
                                                 lse_out=lse, workspace=ws))
    t_score = timed(lambda i: msa.msa_score(cfg, q_ring[i % R], caches[i % L], B, max_len, sc))
    # Step 2 alone: one selected list per (cache, query) pair, L * R lists (4 GiB of selected K/V)
    att = []
    for l in range(L):
        for r in range(R):
            idx = torch.empty((B, Hkv, k), dtype=torch.int32, device=dev)
            msa.msa_select(cfg, q_ring[r], caches[l], B, max_len, idx, workspace=ws)
            att.append((caches[l], q_ring[r], idx, cases[l].seq_lens))
    PA = len(att)
    t_att = timed(lambda i: msa.msa_attend(cfg, att[i % PA][1], att[i % PA][0], B, max_len, att[i % PA][2], out,
                                           lse_out=lse, workspace=ws), PA)
    torch.cuda.synchronize()
    kv = float(np.mean([selected_kv_bytes(a[2], a[3]) for a in att]))
    nb_tot = sum((int(n) + 63) // 64 for n in c0.seq_lens)
    score_bytes = nb_tot * Hkv * D * 4 + nb_tot * 4 + nb_tot * Hkv * 4 + B * Hq * D * 2
    step_bytes = score_bytes + kv + 2 * B * Hq * D * 2 + B * Hkv * k * 4
    log("batch-8 x 131072: step %.2f us (%.0f tokens/s, %.0f GB/s of step bytes); score %.2f us (%.0f GB/s); "
        "attend %.2f us (%.0f GB/s of selected KV)" % (t_step * 1e6, B / t_step, step_bytes / t_step / 1e9,
                                                      t_score * 1e6, score_bytes / t_score / 1e9, t_att * 1e6,
                                                      kv / t_att / 1e9))
    del caches, cases, att
    return {"workload": "decode_bf16_b8_128k", "batch": B, "context": int(max_len), "top_k": k,
            "caches_rotated": L, "step_us": t_step * 1e6, "tokens_per_s": B / t_step,
            "step_GBps": step_bytes / t_step / 1e9, "step_hbm_frac": step_bytes / t_step / 1e9 / HBM_PEAK_GBPS,
            "step_bytes": step_bytes, "score_us": t_score * 1e6, "score_GBps": score_bytes / t_score / 1e9,
            "score_bytes_per_launch": score_bytes, "attend_us": t_att * 1e6, "kv_GBps": kv / t_att / 1e9,
            "kv_hbm_frac": kv / t_att / 1e9 / HBM_PEAK_GBPS, "bytes_per_attend": kv}


def bench_large_k(args, torch, np, msa, caches, cases, q_ring, kn_ring, vn_ring, L, R, rot, k=1024):
    """The pages' operating point on the same 1M-token caches: k = 1024 of 16,384 blocks (~6 %),
    256 MiB of selected K/V per step. Whole decode steps, Step 1 (score + top-k) and Step 2."""
    c0 = cases[0]
    B, max_len = c0.B, c0.max_seq_len
    cfg = msa.make_config(c0.Hq, c0.Hkv, k, dtype=c0.dtype, softmax_scale=c0.scale)
    dev = q_ring[0].device
    out = torch.empty((B, c0.Hq, c0.D), dtype=q_ring[0].dtype, device=dev)
    idx_bufs = [torch.empty((B, c0.Hkv, k), dtype=torch.int32, device=dev) for _ in range(L)]
    ws = torch.empty(msa.msa_workspace_size(cfg, msa.MSA_OP_DECODE, B, max_len), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    n_rep = 10
    per_graph = rot * max(1, 32 // rot)   # whole rotations of the caches and queries

    def timed(fn):
        g = timed_graph(fn, per_graph, torch)
        run_graph(g, 2, torch)
        return run_graph(g, n_rep, torch) / (per_graph * n_rep)
    t_step = timed(lambda i: msa.msa_decode_step(cfg, q_ring[i % R], caches[i % L], B, max_len, out,
                                                 k_new=kn_ring[i % R], v_new=vn_ring[i % R],
                                                 idx_out=idx_bufs[i % L], workspace=ws))
    t_sel = timed(lambda i: msa.msa_select(cfg, q_ring[i % R], caches[i % L], B, max_len, idx_bufs[i % L],
                                           workspace=ws))
    t_att = timed(lambda i: msa.msa_attend(cfg, q_ring[i % R], caches[i % L], B, max_len, idx_bufs[i % L], out,
                                           workspace=ws))
    torch.cuda.synchronize()
    elem = 2 if c0.dtype == "bf16" else 4
    kv = float(np.mean([selected_kv_bytes(idx_bufs[l], cases[l].seq_lens, elem=elem) for l in range(L)]))
    log("1M k=%d: step %.1f us (%.0f tokens/s); select %.1f us; attend %.1f us (%.0f GB/s of selected KV)"
        % (k, t_step * 1e6, B / t_step, t_sel * 1e6, t_att * 1e6, kv / t_att / 1e9))
    return {"workload": "decode_bf16_1m_paged", "top_k": k, "step_us": t_step * 1e6, "tokens_per_s": B / t_step,
            "select_us": t_sel * 1e6, "attend_us": t_att * 1e6, "kv_GBps": kv / t_att / 1e9,
            "kv_hbm_frac": kv / t_att / 1e9 / HBM_PEAK_GBPS, "bytes_per_attend": kv,
            "note": "the pages' ~6 % operating point (16,384 blocks, k = 1024); same caches as the headline"}


def bench_forced(args, torch, np, msa, caches, cases, q_ring, kn_ring, vn_ring, L, R, rot, sink=1, local=1):
    """The 1M-token decode with forced blocks on the same rotated caches: the first (sink) and the
    last (local, holding the new token) block of every row are always kept and count toward k.
    Whole decode steps; every list is checked to hold the forced blocks."""
    c0 = cases[0]
    B, max_len = c0.B, c0.max_seq_len
    cfg = msa.make_config(c0.Hq, c0.Hkv, c0.top_k, dtype=c0.dtype, softmax_scale=c0.scale)
    cfg.keep_sink, cfg.keep_local = sink, local
    dev = q_ring[0].device
    out = torch.empty((B, c0.Hq, c0.D), dtype=q_ring[0].dtype, device=dev)
    idx = [torch.empty((B, c0.Hkv, c0.top_k), dtype=torch.int32, device=dev) for _ in range(L)]
    ws = torch.empty(msa.msa_workspace_size(cfg, msa.MSA_OP_DECODE, B, max_len), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    n_rep = 10
    per_graph = rot * max(1, 32 // rot)   # whole rotations of the caches and queries

    def step(i):
        msa.msa_decode_step(cfg, q_ring[i % R], caches[i % L], B, max_len, out, k_new=kn_ring[i % R],
                            v_new=vn_ring[i % R], idx_out=idx[i % L], workspace=ws)
    g = timed_graph(step, per_graph, torch)
    run_graph(g, 2, torch)
    t_step = run_graph(g, n_rep, torch) / (per_graph * n_rep)
    del g
    torch.cuda.synchronize()
    for l in range(L):
        nb = (int(cases[l].seq_lens[0]) + 63) // 64
        rows = idx[l].cpu().numpy().reshape(-1, c0.top_k)
        forced = {j for j in range(nb) if j < sink or j >= nb - local}
        if not all(forced <= set(r.tolist()) for r in rows):
            raise RuntimeError("forced blocks missing from a decode list")
    log("1M forced blocks (sink %d, local %d): step %.1f us (%.0f tokens/s)" % (sink, local, t_step * 1e6, B / t_step))
    return {"workload": "decode_bf16_1m_paged", "keep_sink": sink, "keep_local": local, "step_us": t_step * 1e6,
            "tokens_per_s": B / t_step,
            "note": "the forced-block option on the headline's caches (same k = 64, the forced blocks among them)"}


def bench_bf16_summaries(args, torch, np, msa, caches, cases, q_ring, kn_ring, vn_ring, L, R, rot):
    """The 1M-token decode with a bf16 summary pool (32 MiB instead of 64 MiB read by Step 1) on
    the same rotated K/V caches: whole decode steps and the scoring kernel alone."""
    c0 = cases[0]
    B, max_len = c0.B, c0.max_seq_len
    cfg = msa.make_config(c0.Hq, c0.Hkv, c0.top_k, dtype=c0.dtype, softmax_scale=c0.scale, summary_dtype="bf16")
    dev = q_ring[0].device
    bcaches = []
    for l in range(L):
        S = torch.empty((c0.num_pages, c0.Hkv, c0.D), dtype=torch.bfloat16, device=dev)
        cb = msa.KVCache(caches[l].k_pages, caches[l].v_pages, S, caches[l].block_table, caches[l].seq_lens)
        msa.msa_build_summaries(cfg, cb, B, max_len)
        bcaches.append(cb)
    out = torch.empty((B, c0.Hq, c0.D), dtype=q_ring[0].dtype, device=dev)
    idx = [torch.empty((B, c0.Hkv, c0.top_k), dtype=torch.int32, device=dev) for _ in range(L)]
    mb = (max_len + 63) // 64
    sc = torch.empty((B, c0.Hkv, mb), dtype=torch.float32, device=dev)
    ws = torch.empty(msa.msa_workspace_size(cfg, msa.MSA_OP_DECODE, B, max_len), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    n_rep = 10
    per_graph = rot * max(1, 32 // rot)   # whole rotations of the caches and queries

    def timed(fn):
        g = timed_graph(fn, per_graph, torch)
        run_graph(g, 2, torch)
        return run_graph(g, n_rep, torch) / (per_graph * n_rep)
    t_step = timed(lambda i: msa.msa_decode_step(cfg, q_ring[i % R], bcaches[i % L], B, max_len, out,
                                                 k_new=kn_ring[i % R], v_new=vn_ring[i % R], idx_out=idx[i % L],
                                                 workspace=ws))
    # scoring alone over 2 * SCORE_POOLS bf16 pools (~1 GB), beyond the infinity cache as above
    spools = list(bcaches)
    while len(spools) < 2 * SCORE_POOLS:
        base = bcaches[len(spools) % L]
        spools.append(msa.KVCache(base.k_pages, base.v_pages, base.summaries.clone(), base.block_table,
                                  base.seq_lens))
    P = len(spools)
    g_score = timed_graph(lambda i: msa.msa_score(cfg, q_ring[i % R], spools[i % P], B, max_len, sc), P, torch)
    run_graph(g_score, 2, torch)
    n_score = max(2, args.steps // P)
    t_score = run_graph(g_score, n_score, torch) / (n_score * P)
    del g_score, spools
    torch.cuda.synchronize()
    nb = sum((int(n) + 63) // 64 for n in c0.seq_lens)
    score_bytes = nb * c0.Hkv * c0.D * 2 + nb * 4 + nb * c0.Hkv * 4 + B * c0.Hq * c0.D * 2
    log("1M bf16 summaries: step %.1f us (%.0f tokens/s); score %.2f us (%.0f GB/s)"
        % (t_step * 1e6, B / t_step, t_score * 1e6, score_bytes / t_score / 1e9))
    del bcaches
    return {"workload": "decode_bf16_1m_paged", "summary_dtype": "bf16", "step_us": t_step * 1e6,
            "tokens_per_s": B / t_step, "score_us": t_score * 1e6, "score_bytes_per_launch": score_bytes,
            "score_GBps": score_bytes / t_score / 1e9, "score_hbm_frac": score_bytes / t_score / 1e9 / HBM_PEAK_GBPS,
            "note": "same caches and queries as the headline; summaries rounded to bf16 (a different, coarser "
                    "ranking input, so not the headline number)"}


def bench_mixed(args, torch, np, msa, make_decode_case_torch, workload, dev):
    """Batch-32 decode over log-uniform lengths (4096 .. 1,048,576, about 8M tokens in one
    shuffled page pool, k = min(64, blocks)): whole decode steps, and the scoring and attend
    stages alone. One cache (32 GiB of K/V): far beyond the infinity cache without rotation."""
    kw = workload("decode_bf16_mixed_b32", seed=args.seed)
    c = make_decode_case_torch(device=dev, **kw)
    table = torch.from_numpy(c.block_table).to(dev)
    lens = torch.from_numpy(c.seq_lens).to(dev)
    S = torch.empty((c.num_pages, c.Hkv, c.D), dtype=torch.float32, device=dev)
    cache = msa.KVCache(c.k_pool, c.v_pool, S, table, lens)
    cfg = msa.make_config(c.Hq, c.Hkv, c.top_k, dtype="bf16", softmax_scale=c.scale)
    msa.msa_build_summaries(cfg, cache, c.B, c.max_seq_len)
    B, R = c.B, 8
    gen = torch.Generator(device=dev)
    gen.manual_seed(args.seed + 91)
    q_ring = [torch.randn((B, c.Hq, c.D), generator=gen, device=dev).to(torch.bfloat16) for _ in range(R)]
    kn_ring = [torch.randn((B, c.Hkv, c.D), generator=gen, device=dev).to(torch.bfloat16) for _ in range(R)]
    vn_ring = [torch.randn((B, c.Hkv, c.D), generator=gen, device=dev).to(torch.bfloat16) for _ in range(R)]
    out = torch.empty((B, c.Hq, c.D), dtype=torch.bfloat16, device=dev)
    idx = torch.empty((B, c.Hkv, c.top_k), dtype=torch.int32, device=dev)
    mb = (c.max_seq_len + 63) // 64
    sc = torch.empty((B, c.Hkv, mb), dtype=torch.float32, device=dev)
    ws = torch.empty(msa.msa_workspace_size(cfg, msa.MSA_OP_DECODE, B, c.max_seq_len), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def timed(fn, n=10):
        g = timed_graph(fn, R, torch)
        run_graph(g, 2, torch)
        return run_graph(g, n, torch) / (R * n)
    t_step = timed(lambda i: msa.msa_decode_step(cfg, q_ring[i], cache, B, c.max_seq_len, out, k_new=kn_ring[i],
                                                 v_new=vn_ring[i], idx_out=idx, workspace=ws))
    t_score = timed(lambda i: msa.msa_score(cfg, q_ring[i], cache, B, c.max_seq_len, sc))
    msa.msa_select(cfg, q_ring[0], cache, B, c.max_seq_len, idx, workspace=ws)
    t_att = timed(lambda i: msa.msa_attend(cfg, q_ring[i], cache, B, c.max_seq_len, idx, out, workspace=ws))
    torch.cuda.synchronize()
    kv = float(selected_kv_bytes(idx, c.seq_lens))
    nb_tot = sum((int(n) + 63) // 64 for n in c.seq_lens)
    score_bytes = nb_tot * c.Hkv * c.D * 4 + nb_tot * 4 + nb_tot * c.Hkv * 4 + B * c.Hq * c.D * 2
    log("mixed batch-32 (%d tokens): step %.1f us (%.0f tokens/s); score %.1f us (%.0f GB/s); attend %.1f us "
        "(%.0f GB/s of selected KV)" % (int(np.sum(c.seq_lens)), t_step * 1e6, B / t_step, t_score * 1e6,
                                         score_bytes / t_score / 1e9, t_att * 1e6, kv / t_att / 1e9))
    return {"workload": "decode_bf16_mixed_b32", "batch": B, "total_tokens": int(np.sum(c.seq_lens)),
            "step_us": t_step * 1e6, "tokens_per_s": B / t_step,
            "score_us": t_score * 1e6, "score_GBps": score_bytes / t_score / 1e9,
            "score_hbm_frac": score_bytes / t_score / 1e9 / HBM_PEAK_GBPS,
            "attend_us": t_att * 1e6, "kv_GBps": kv / t_att / 1e9, "kv_hbm_frac": kv / t_att / 1e9 / HBM_PEAK_GBPS,
            "bytes_per_attend": kv, "bytes_per_score": score_bytes}


def bench_index(args, torch, np, msa, dev, L=2, R=8):
    """Step 1 as the diagram's index branch on the 1M-token shape: single-head 128-dim bf16 index
    keys (256 MiB per cache, two caches rotated), one index query per group (8 groups), Block Max
    Pool, top-64. Times msa_select_index (scoring kernel + top-k)."""
    from synth import make_index_case_torch
    items = []
    for layer in range(L):
        c = make_index_case_torch(B=1, Hkv=8, lens=[1 << 20], top_k=64, dtype="bf16", permute=True,
                                  plant=("count", 16), seed=args.seed + 1000 * layer, device=dev)
        items.append((c, torch.from_numpy(c.block_table).to(dev), torch.from_numpy(c.seq_lens).to(dev)))
    c0 = items[0][0]
    cfg = msa.make_config(c0.Hkv, c0.Hkv, c0.top_k, dtype="bf16")
    gen = torch.Generator(device=dev)
    gen.manual_seed(args.seed + 93)
    q_ring = [torch.randn((1, c0.Hkv, c0.Di), generator=gen, device=dev).to(torch.bfloat16) for _ in range(R)]
    idx = [torch.empty((1, c0.Hkv, c0.top_k), dtype=torch.int32, device=dev) for _ in range(L)]
    ws = torch.empty(msa.msa_workspace_size(cfg, msa.MSA_OP_SELECT, 1, c0.max_seq_len), dtype=torch.uint8,
                     device=dev)
    torch.cuda.synchronize()
    per = L * R // math.gcd(L, R)
    g = timed_graph(lambda i: msa.msa_select_index(cfg, q_ring[i % R], items[i % L][0].index_keys, items[i % L][1],
                                                   items[i % L][2], 1, c0.max_seq_len, idx[i % L], workspace=ws),
                    per, torch)
    run_graph(g, 2, torch)
    n = 10
    t = run_graph(g, n, torch) / (per * n)
    nb = (c0.max_seq_len + 63) // 64
    key_bytes = nb * 64 * c0.Di * 2 + nb * 4 + c0.Hkv * c0.Di * 2 + c0.Hkv * nb * 4
    log("index-branch select (1M, 8 groups, k=64): %.1f us, %.0f GB/s of index keys over the whole select"
        % (t * 1e6, key_bytes / t / 1e9))
    return {"workload": "index_bf16_1m_paged", "context": int(c0.max_seq_len), "kv_groups": c0.Hkv,
            "index_dim": c0.Di, "top_k": c0.top_k, "select_us": t * 1e6,
            "score_bytes_per_launch": key_bytes, "GBps_over_select": key_bytes / t / 1e9,
            "note": "single-head index keys paged like K; the top-k time is included in select_us"}


def cpu_baseline(args, case, torch, np):
    """The fp64 oracle (untuned) on a bounded sample of the same decode workload: select from cached
    block summaries + attend. One oracle call threads over the (sequence, KV group) units (8 at
    batch 1); to use every host core of this process, independent steps run concurrently in as many
    instances as the units divide into the cores (ctypes releases the interpreter lock during the
    oracle call). Three runs of about --cpu-seconds / 3 each; the median rate is the value."""
    import threading
    import oracle

    def host_storage(t):
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).cpu().numpy().view(np.uint16)
        return t.cpu().numpy()
    q = host_storage(case.q)
    k = host_storage(case.k_pool)
    v = host_storage(case.v_pool)
    S = oracle.summaries(k_pool=k, block_table=case.block_table, seq_lens=case.seq_lens, Hkv=case.Hkv,
                         D=case.D, P=case.P)
    units = case.B * case.Hkv
    cores = oracle.default_threads()
    per_inst = min(cores, units)
    inst = max(1, cores // per_inst)
    kw = dict(q=q, k_pool=k, v_pool=v, block_table=case.block_table, seq_lens=case.seq_lens, Hq=case.Hq,
              Hkv=case.Hkv, top_k=case.top_k, scale=case.scale, P=case.P, summaries_in=S, nthreads=per_inst)

    def run(n):
        """wall seconds for inst concurrent instances of n oracle steps each"""
        def worker():
            for _ in range(n):
                oracle.decode(**kw)
        ts = [threading.Thread(target=worker) for _ in range(inst)]
        t0 = time.perf_counter()
        for t in ts:
            t.start()
        for t in ts:
            t.join()
        return time.perf_counter() - t0
    one = min(run(1) for _ in range(2))   # calibration on warm calls (the first pays for cold caches)
    n = int(max(2, min(5000, args.cpu_seconds / 3.0 / max(one, 1e-3))))
    rates = sorted(inst * n * case.B / run(n) for _ in range(3))
    log("cpu oracle: %d instances x %d threads, %d steps each per run, rates %s tokens/s"
        % (inst, per_inst, n, ", ".join("%.1f" % r for r in rates)))
    # the same oracle on one thread, over a sample of about a fifth of the time
    kw1 = dict(kw, nthreads=1)
    t0 = time.perf_counter()
    oracle.decode(**kw1)
    one1 = time.perf_counter() - t0
    n1 = int(max(1, min(1000, 0.2 * args.cpu_seconds / max(one1, 1e-3))))
    t0 = time.perf_counter()
    for _ in range(n1):
        oracle.decode(**kw1)
    dt1 = time.perf_counter() - t0
    log("cpu oracle, one thread: %d steps in %.1f s" % (n1, dt1))
    return {"value": rates[1], "unit": "tokens/s", "cores": inst * per_inst, "kind": "oracle",
            "host_cores": cores, "runs": rates, "single_thread_value": n1 * case.B / dt1,
            "sample": "median of 3 runs; each run: %d concurrent instances x %d decode steps (select from cached "
                      "fp64 summaries + attend) of the same 1M-token workload, fp64 C oracle threaded over the %d "
                      "(sequence, KV group) units, %d threads per instance; %d more steps on one thread for "
                      "single_thread_value" % (inst, n, units, per_inst, n1)}


if __name__ == "__main__":
    main()
