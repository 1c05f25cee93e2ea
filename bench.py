"""Benchmark of the sparse-attention decode step on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload headline]

One step = the whole hot path of one decode step over one batch: row store of
the step's new K / V / index rows, e4m3 query store, index scores over every
page, top-k, split attention over the selected pages and the merge
(decode_step of libmxsparse). The K timed steps run on R cache replicas in
turn (step i on replica i % R, as the layers of a decode each have their own
cache) and are captured in one HIP graph of K steps, replayed once. The default workload is
the 256K-context one: B = 4 sequences x q = 8 query rows (1 + 7 drafts), 16
query heads per KV head, head_dim 128, MXFP4 K / V / index caches, top-k 32.

The replicas share one page table and one context-length vector (the layers
of a decode share the sequences' block table); each has its own K / V / index
pools. Inputs are resident in HBM before timing starts, and the GPU has been kept
busy with untimed step replays for --settle-ms of wall time (it lowers its
clocks when idle; each later kernel timing is preceded by its own shorter
settle), then the W warmup steps run. Each timed step runs on the
next of R cache replicas, R at least --replicas (6) and enough that R steps
touch 512 MB, twice the 256 MB Infinity Cache (the 256K workload: 6 x ~88 MB),
so that every workload's scan streams from HBM, as a model's layers would, not
from the MALL; the one-replica (warm) number is reported separately (its index
pages are copied non-temporally too, so it stays close to the streaming one).

Prints one JSON line (rank 0): the metric (query rows/s), the whole step's
algorithmic HBM bytes and GB/s, the roofline of the dominant kernel (the index
scorer: 100 back-to-back launches over rotating replicas captured in one HIP
graph, timed with HIP events on the stream they run on, beside a plain
streaming read of the same pages, its ceiling) and the oracle's throughput on
a bounded sample on the host cores (all of them, and one thread).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
# bytes the R replicas' steps must touch together: twice the 256 MB Infinity Cache
ROTATION_BYTES = 512_000_000
PAGE_MX = 8704
# page bytes and bytes of one stored 128-element row, per cache format
PAGE_BYTES = {"mxfp4": 8704, "fp8": 16896, "nvfp4": 9728}
ROW_BYTES = {"mxfp4": 64 + 4, "fp8": 128 + 4, "nvfp4": 64 + 8 + 4}
CSRC = os.path.join(ROOT, "sparse_attention_decode_mxfp4_amd", "csrc")
# the sources the index scorer kernel is built from; the HBM traffic measured
# with rocprofv3 counters is reported only while they are unchanged
SCORER_SOURCES = ("score.hip", "score.hpp", "common.hpp", "rowstore.hpp", "launch.hpp")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "scorer_traffic_{}.json")      # per workload


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def query_bytes(wl) -> int:
    """Bytes of one attention-query element as the step reads it."""
    return 4 if (wl.kv_format == "mxfp4" and wl.q_dtype == "f32") else 2


def algorithmic_bytes(inp, table: np.ndarray) -> dict:
    """Bytes the step must move at minimum: every index page of every sequence
    once, the distinct K and V pages the sequence's rows selected, the new rows
    (read as fp32, stored in the cache formats), the query, index query,
    weights, page table and the bf16 output with its lse."""
    wl = inp.wl
    idx_pages = int(sum((int(L) + 127) // 128 for L in inp.contexts))
    kv_pages = 0
    for b in range(wl.B):
        kv_pages += len(np.unique(table[b][table[b] >= 0]))
    rows = wl.B * wl.q
    pi, pkv = PAGE_BYTES[wl.idx_format], PAGE_BYTES[wl.kv_format]
    other = (3 * rows * 128 * 4                           # new rows in
             + 2 * rows * ROW_BYTES[wl.kv_format] + rows * ROW_BYTES[wl.idx_format]   # stored rows out
             + rows * wl.H * 128 * query_bytes(wl)        # query
             + rows * wl.H_I * 128 * 2 + rows * wl.H_I * 4  # index query, weights
             + wl.B * inp.max_pages * 4 + wl.B * 4        # page table, contexts
             + rows * wl.H * 128 * 2 + rows * wl.H * 4)   # output bf16, lse
    return {"index_pages": idx_pages * pi, "kv_pages": 2 * kv_pages * pkv, "other": other,
            "total": idx_pages * pi + 2 * kv_pages * pkv + other,
            "n_index_pages": idx_pages, "n_kv_pages": 2 * kv_pages}


def scorer_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in SCORER_SOURCES:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def cache_replicas(step_bytes: int, at_least: int = 6) -> int:
    """Cache replicas the timed steps rotate over: at least `at_least`, and
    enough that their steps touch ROTATION_BYTES together (each replica is
    then out of the caches when its turn comes again)."""
    return max(1, at_least, -(-ROTATION_BYTES // max(1, int(step_bytes))))


def measured_traffic(workload: str):
    """HBM bytes per scorer launch from the committed rocprofv3 counter summary
    (FETCH_SIZE + WRITE_SIZE, each scaled by a plain copy's reading), or None
    when there is none for this workload or the scorer changed since."""
    try:
        with open(TRAFFIC_FILE.format(workload)) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("workload") != workload or t.get("scorer_sources_sha256") != scorer_source_hash():
        return None
    return t["fetch_bytes_per_launch"] + t["write_bytes_per_launch"]


def copy_calibration(n_bytes: int = 256 << 20, reps: int = 20):
    """A plain device copy of known size, for scaling rocprofv3's FETCH_SIZE /
    WRITE_SIZE readings: each launch reads and writes n_bytes."""
    import torch
    src = torch.ones(n_bytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read_per_launch": n_bytes, "bytes_written_per_launch": n_bytes,
                                           "launches": reps}}), flush=True)


def settle(replay, min_ms: float) -> float:
    """Untimed replays of a captured graph (or any enqueueing callable), back to
    back, for at least ``min_ms`` of wall time: the GPU lowers its clocks when
    idle and takes milliseconds to raise them again, so a measurement that
    starts right after host-side setup catches it mid-ramp (the stand-alone
    scorer measured 20-24 us per launch after 1 s idle against 17.8-18.3 us
    once loaded). Returns the wall time spent."""
    import torch
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < min_ms:
        for _ in range(8):                      # keep work queued: no idle gap between replays
            replay()
        torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3


def contiguous_read_ceiling(n_launch: int = 20, settle_ms: float = 30.0) -> dict:
    """The device's sustained streaming-read rate: mxs_read_index_pages over a
    contiguous pool of 16 x 8192 MXFP4 pages (1.14 GB, identity page table),
    far larger than the 256 MB Infinity Cache; launches captured in one HIP
    graph and timed with events on the stream they run on."""
    import torch
    import sparse_attention_decode_mxfp4_amd as mx
    B, stride = 16, 8192
    pool = torch.zeros(B * stride * PAGE_MX, dtype=torch.uint8, device="cuda")
    table = torch.arange(B * stride, dtype=torch.int32, device="cuda").view(B, stride)
    ctx = torch.full((B,), stride * 128, dtype=torch.int32, device="cuda")
    cache = mx.Cache(pool, pool, pool, table, ctx, "mxfp4", "mxfp4")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    mx.read_index_pages(cache, B, sink)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(n_launch):
            mx.read_index_pages(cache, B, sink)
    settle(g.replay, settle_ms)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / n_launch
    nbytes = B * stride * PAGE_MX
    del pool
    return {"what": "mxs_read_index_pages over a contiguous 1.14 GB pool (16 x 8192 pages, identity table)",
            "bytes": nbytes, "avg_launch_us": us, "GBps": nbytes / (us * 1e-6) / 1e9,
            "frac_of_peak": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS}


def cpu_baseline(inp, min_seconds=10.0, max_seconds=30.0) -> dict:
    """The oracle (NumPy, float64) on sequence 0 of the workload: its whole
    decode step (row store of the new rows, scores over every page, top-k,
    attention), repeated until at least ``min_seconds`` of CPU work, then once
    more on one thread."""
    from threadpoolctl import threadpool_info, threadpool_limits
    from oracle import step as OS
    wl = inp.wl
    fmts = {"k": wl.kv_format, "v": wl.kv_format, "idx": wl.idx_format}
    pools = {s: OS.build_cache(inp, s, f, seqs=[0]) for s, f in fmts.items()}
    reps, t0 = 0, time.perf_counter()
    while True:
        OS.decode_step_ref(inp, pools=pools, seqs=[0])
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds or el + el / reps > max_seconds:
            break
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    with threadpool_limits(1):                 # the same step on one thread, once
        t1 = time.perf_counter()
        OS.decode_step_ref(inp, pools=pools, seqs=[0])
        el1 = time.perf_counter() - t1
    return {"value": reps * wl.q / el, "unit": "query rows/s", "cores": int(threads), "kind": "oracle",
            "one_thread_value": wl.q / el1,
            "sample": f"sequence 0 of {wl.B} ({wl.q} query rows, {int(inp.contexts[0])}-token context): the "
                      f"oracle's full step for that sequence, {reps} run(s) in {el:.1f} s (one thread: one run in {el1:.1f} s); "
                      f"host affinity {len(os.sched_getaffinity(0))} cores"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=600)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="headline")
    ap.add_argument("--replicas", type=int, default=6,
                    help="at least this many cache replicas (more if their steps would touch under 512 MB)")
    ap.add_argument("--scorer-launches", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--settle-ms", type=float, default=200.0,
                    help="untimed step replays (wall ms) before the warmup steps, so the GPU runs at its "
                         "loaded clocks; each kernel timing after the step's is preceded by a quarter of it")
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of graph replays")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain copy of known size (for scaling rocprofv3 byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only: the decode step of one rank is a "
                                   "single-GPU kernel chain with no collectives; run with --gpus 1"}))
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration()
        return
    import torch
    import sparse_attention_decode_mxfp4_amd as mx
    import workloads as W
    import workloads.gpu as WG

    torch.cuda.set_device(0)
    mx.lib()
    wl = W.WORKLOADS[args.workload]
    inp = W.make_inputs(wl)
    t_setup = time.perf_counter()
    pools0 = WG.fill_prefix(inp, WG.empty_pools(inp))
    torch.cuda.synchronize()
    log(f"[bench] filled {wl.name} caches in {time.perf_counter() - t_setup:.1f} s")
    t = WG.step_tensors(inp)

    def make_step(c, tb):
        return mx.DecodeStep(c, t["query"], t["q_idx"], t["w"], wl.topk, wl.sm_scale, k_new=t.get("k_new"),
                             v_new=t.get("v_new"), idx_new=t.get("idx_new"), block_table_out=tb)

    # replica 0 first: one step gives the block table, hence the bytes a step
    # touches; then R replicas, at least --replicas and enough that R steps
    # touch ROTATION_BYTES, so that no replica is still in the caches when its
    # turn comes again (a step rewrites the same new rows each time, so the
    # copies of replica 0 hold what their own first step would leave). The
    # replicas share one page table and context-length vector, as the layers of
    # a decode step share the sequences' block table; each has its own pools.
    c0 = WG.make_cache(inp, pools0)
    tables = [torch.empty((wl.B, wl.q, wl.topk), dtype=torch.int32, device="cuda")]
    steps = [make_step(c0, tables[0])]
    steps[0].run()
    torch.cuda.synchronize()
    ab = algorithmic_bytes(inp, tables[0].cpu().numpy())
    R = cache_replicas(ab["total"], args.replicas)
    caches = [c0]
    for _ in range(R - 1):
        pools = {s_: p.clone() for s_, p in pools0.items()}
        caches.append(WG.make_cache(inp, pools, table=c0.page_table, ctx=c0.context_lens))
        tables.append(torch.empty((wl.B, wl.q, wl.topk), dtype=torch.int32, device="cuda"))
        steps.append(make_step(caches[-1], tables[-1]))
    for s in steps:
        s.run()
    torch.cuda.synchronize()

    # ---- the timed region: exactly K steps, rotating replicas (step i runs on
    # replica i % R, like the layers of one decode step, each with its own
    # cache), captured in one HIP graph of K steps and replayed once, so no
    # host launch gap falls between steps; the W warmup steps are a graph of
    # their own.
    def steps_graph(k):
        if k <= 0:
            return None
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(k):
                steps[i % R].run()
        return g

    if args.eager:
        def run_steps(k):
            for i in range(k):
                steps[i % R].run()
        warm_run = lambda: run_steps(args.warmup)
        timed_run = lambda: run_steps(args.steps)
    else:
        g_warm, g_timed = steps_graph(args.warmup), steps_graph(args.steps)
        warm_run = g_warm.replay if g_warm is not None else (lambda: None)
        timed_run = g_timed.replay
    # the same R-step graph used below for the per-replay distribution
    chunk = None if args.eager else steps_graph(R)

    # untimed: bring the GPU to its loaded clocks (steps on the R replicas, as
    # timed), then the W warmup steps
    settle_main = settle(chunk.replay if chunk is not None else (lambda: [s_.run() for s_ in steps]),
                         args.settle_ms)
    settle_each = args.settle_ms / 4
    warm_run()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()                                 # (the GPU is idle: it stamps this at once)
    t0 = time.perf_counter()
    timed_run()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    ev_ms_step = ev0.elapsed_time(ev1) / args.steps

    # per-replay distribution (outside the timed region): each replay of the
    # R-step graph bracketed by its own events; median and spread per step
    rep_us = []
    if chunk is not None:
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(max(100, args.steps // R))]
        for a_, b_ in evs:
            a_.record()
            chunk.replay()
            b_.record()
        torch.cuda.synchronize()
        rep_us = sorted(a_.elapsed_time(b_) * 1e3 / R for a_, b_ in evs)

    # warm (MALL-resident) number: one replica, one graph of R steps on it
    warm = torch.cuda.CUDAGraph()
    with torch.cuda.graph(warm):
        for _ in range(R):
            steps[0].run()
    settle(warm.replay, settle_each)
    ev0.record()
    for _ in range(max(1, args.steps // R)):
        warm.replay()
    ev1.record()
    torch.cuda.synchronize()
    warm_ms = ev0.elapsed_time(ev1) / (max(1, args.steps // R) * R)

    # ---- the dominant kernel: the index scorer, K back-to-back launches (rotating
    # replicas) captured in one HIP graph, timed with HIP events on the stream
    # it runs on; the average includes the short gap between graph nodes
    scores = [torch.empty((wl.B, wl.q, inp.max_pages), dtype=torch.float32, device="cuda") for _ in range(R)]
    for i in range(R):
        mx.index_score(caches[i], t["q_idx"], t["w"], scores[i])
    torch.cuda.synchronize()
    n_launch = args.scorer_launches
    gs = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gs):
        for i in range(n_launch):
            mx.index_score(caches[i % R], t["q_idx"], t["w"], scores[i % R])
    settle(gs.replay, settle_each)
    ev0.record()
    gs.replay()
    ev1.record()
    torch.cuda.synchronize()
    score_us = ev0.elapsed_time(ev1) * 1e3 / n_launch
    score_bytes = ab["index_pages"] + ab["n_index_pages"] * wl.q * 4 + wl.B * wl.q * wl.H_I * (256 + 4)
    score_gbps = score_bytes / (score_us * 1e-6) / 1e9

    # ---- the scan's streaming-read ceiling: the same index pages, read in the
    # same page-table order with plain loads and no arithmetic
    # (mxs_read_index_pages), timed the same way as the scorer
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    for i in range(R):
        mx.read_index_pages(caches[i], wl.B, sink)
    torch.cuda.synchronize()
    gread = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gread):
        for i in range(n_launch):
            mx.read_index_pages(caches[i % R], wl.B, sink)
    settle(gread.replay, settle_each)
    ev0.record()
    gread.replay()
    ev1.record()
    torch.cuda.synchronize()
    read_us = ev0.elapsed_time(ev1) * 1e3 / n_launch
    read_gbps = ab["index_pages"] / (read_us * 1e-6) / 1e9

    # ---- the step of a layer that reuses a block selection (decode_step_reuse
    # over the tables the full steps wrote): its K / V row store and query
    # store, split attention over the selected pages and the merge; R
    # consecutive steps in one graph, as above
    rows = wl.B * wl.q
    reuse = [mx.DecodeStepReuse(c, t["query"], tb, wl.sm_scale, k_new=t.get("k_new"), v_new=t.get("v_new"))
             for c, tb in zip(caches, tables)]
    for s in reuse:
        s.run()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        for s in reuse:
            s.run()
    settle(gr.replay, settle_each)
    n_rep = max(1, args.steps // R)
    ev0.record()
    for _ in range(n_rep):
        gr.replay()
    ev1.record()
    torch.cuda.synchronize()
    reuse_us = ev0.elapsed_time(ev1) * 1e3 / (n_rep * R)
    # the same step as one launch (decode_step_reuse_one_launch), timed the same way
    reuse1 = [mx.DecodeStepReuse(c, t["query"], tb, wl.sm_scale, k_new=t.get("k_new"), v_new=t.get("v_new"),
                                 one_launch=True) for c, tb in zip(caches, tables)]
    for s_ in reuse1:
        s_.run()
    gr1 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr1):
        for s_ in reuse1:
            s_.run()
    settle(gr1.replay, settle_each)
    ev0.record()
    for _ in range(n_rep):
        gr1.replay()
    ev1.record()
    torch.cuda.synchronize()
    reuse1_us = ev0.elapsed_time(ev1) * 1e3 / (n_rep * R)
    reuse_bytes = (ab["kv_pages"] + 2 * rows * 128 * 4 + 2 * rows * ROW_BYTES[wl.kv_format]
                   + rows * wl.H * 128 * query_bytes(wl)
                   + wl.B * inp.max_pages * 4 + wl.B * 4 + rows * wl.topk * 4 + rows * wl.H * 128 * 2 + rows * wl.H * 4)
    reuse_gbps = reuse_bytes / (reuse_us * 1e-6) / 1e9

    # ---- the device's sustained streaming-read rate (contiguous, > 1 GiB)
    sustained = contiguous_read_ceiling(settle_ms=settle_each)
    # ---- the same step as one launch (decode_step_one_launch), when the
    # workload is one it takes: a graph of R consecutive steps, as above
    one_us = None
    if wl.kv_format == "mxfp4" and wl.idx_format == "mxfp4" and wl.q <= 8 and wl.B * inp.max_pages >= 8192:
        one = [mx.DecodeStep(c, t["query"], t["q_idx"], t["w"], wl.topk, wl.sm_scale, k_new=t.get("k_new"),
                             v_new=t.get("v_new"), idx_new=t.get("idx_new"), one_launch=True) for c in caches]
        for s_ in one:
            s_.run()
        g1 = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g1):
            for s_ in one:
                s_.run()
        settle(g1.replay, settle_each)
        ev0.record()
        for _ in range(n_rep):
            g1.replay()
        ev1.record()
        torch.cuda.synchronize()
        one_us = ev0.elapsed_time(ev1) * 1e3 / (n_rep * R)
        log(f"[bench] one-launch step {one_us:.1f} us")

    step_gbps = ab["total"] / (ms_step * 1e-3) / 1e9
    out = {
        "metric": "decode sparse-attn query rows/s + HBM GB/s (% peak), 256K ctx, B=4, q=8",
        "value": rows / (ms_step * 1e-3),
        "unit": "query rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{wl.name}: B={wl.B}, q={wl.q} (1+{wl.q - 1} drafts), {wl.H}:1 GQA, head_dim 128, "
                        f"context {int(inp.contexts.min())}..{int(inp.contexts.max())} tokens, "
                        f"{wl.kv_format} K/V, {wl.idx_format} index, top-k {wl.topk}, {wl.H_I} index heads, "
                        f"full decode_step ({'eager' if args.eager else 'HIP graph replay'})",
            "B": wl.B, "q": wl.q, "H": wl.H, "H_I": wl.H_I, "topk": wl.topk,
            "context": int(inp.contexts.max()), "cache_replicas": R,
            "arithmetic": ("f16 MFMA for index scores and QK (NVFP4 codes times their e4m3 block scale, widened "
                           "exactly to f16; the bf16 query scaled per row into f16), bf16 MFMA for PV, f32 accumulate"
                           if wl.kv_format == "nvfp4" else
                           "bf16 MFMA for index scores, QK and PV (e2m1 codes times their block scale, e4m3 codes: "
                           "widened exactly to bf16), f32 accumulate"),
        },
        "hbm": {"algorithmic_bytes_per_step": ab["total"], "GBps": step_gbps, "peak_GBps": HBM_PEAK_GBPS,
                "frac": step_gbps / HBM_PEAK_GBPS, "index_bytes": ab["index_pages"],
                "kv_bytes": ab["kv_pages"], "other_bytes": ab["other"]},
        "event_ms_per_step": ev_ms_step,
        "replays": ({"n": len(rep_us), "steps_per_replay": R, "median_us_per_step": rep_us[len(rep_us) // 2],
                     "p10_us_per_step": rep_us[len(rep_us) // 10], "p90_us_per_step": rep_us[(9 * len(rep_us)) // 10]}
                    if rep_us else None),
        "warm_mall_ms_per_step": warm_ms,
        "settle": {"what": "untimed replays, back to back, so that timing starts at the GPU's loaded clocks "
                           "(it lowers them when idle): steps before the warmup steps, the kernel's own graph "
                           "before each kernel timing", "ms_before_warmup": settle_main,
                   "ms_before_each_kernel_timing": settle_each},
        "roofline": {"bound": "hbm", "kernel": "index scorer (k_index_score)", "achieved": score_gbps,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": score_gbps / HBM_PEAK_GBPS,
                     "traffic": measured_traffic(wl.name), "avg_launch_us": score_us,
                     "algorithmic_bytes_per_launch": score_bytes,
                     "read_ceiling": {"what": "plain streaming read of the same index pages in page-table order "
                                              "(mxs_read_index_pages), timed like the scorer",
                                      "avg_launch_us": read_us, "GBps": read_gbps,
                                      "frac_of_peak": read_gbps / HBM_PEAK_GBPS,
                                      "scorer_frac_of_ceiling": score_gbps / read_gbps},
                     "sustained_read": dict(sustained, scorer_frac=score_gbps / sustained["GBps"])},
    }
    out["hbm"]["frac_of_sustained_read"] = step_gbps / sustained["GBps"]
    out["attention_only_step"] = {
        "what": "decode_step_reuse: the step of a layer reusing a block selection (K/V row store, q store, "
                "split attention over the selected pages, merge), graph of R steps",
        "us_per_step": reuse_us, "query_rows_per_s": rows / (reuse_us * 1e-6),
        "roofline": {"bound": "hbm", "achieved": reuse_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": reuse_gbps / HBM_PEAK_GBPS, "algorithmic_bytes_per_step": reuse_bytes},
        "one_launch": {"what": "decode_step_reuse_one_launch: the same step as one launch (store workgroups, "
                               "then attention workgroups that wait for their sequence's stores)",
                       "us_per_step": reuse1_us, "query_rows_per_s": rows / (reuse1_us * 1e-6),
                       "GBps": reuse_bytes / (reuse1_us * 1e-6) / 1e9},
    }
    if one_us is not None:
        out["one_launch_step"] = {"what": "decode_step_one_launch: the same step as one launch (scoring and attention "
                                          "workgroups in one grid), graph of R steps",
                                  "us_per_step": one_us, "query_rows_per_s": rows / (one_us * 1e-6),
                                  "GBps": ab["total"] / (one_us * 1e-6) / 1e9}
    log(f"[bench] attention-only step {reuse_us:.1f} us = {reuse_gbps:.0f} GB/s; as one launch {reuse1_us:.1f} us")
    if rep_us:
        log(f"[bench] per replay of {R} steps: median {rep_us[len(rep_us) // 2]:.1f} us per step "
            f"(p10 {rep_us[len(rep_us) // 10]:.1f}, p90 {rep_us[(9 * len(rep_us)) // 10]:.1f}; {len(rep_us)} replays)")
    log(f"[bench] step {ms_step * 1e3:.1f} us (events {ev_ms_step * 1e3:.1f} us, warm {warm_ms * 1e3:.1f} us), "
        f"{step_gbps:.0f} GB/s; scorer {score_us:.1f} us = {score_gbps:.0f} GB/s; "
        f"read ceiling {read_us:.1f} us = {read_gbps:.0f} GB/s; sustained contiguous read "
        f"{sustained['GBps']:.0f} GB/s ({sustained['frac_of_peak']:.3f} of peak)")
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
