#!/usr/bin/env python3
"""Benchmark of one decode step of the paged KV cache on one MI355X.

A step is the whole hot path over one batch, as one library call
(pkv_decode_step): the slot-mapping scatter of each row's new token K/V into
the pool, then the paged decode read of every row (GQA heads, split-context
partitions + merge); the stream read appends the tokens itself.  The workload is a
Llama-3-8B-shaped attention layer: 64 rows, 32 query heads, 8 kv heads,
head_dim 128, bf16 pool of 16-position blocks, context lengths uniform in
[512, 4096], block tables drawn from a 1.5x pool.  Every input is synthetic
and seeded; inputs are resident in HBM before timing starts.

Prints one JSON line: whole-step HBM throughput (algorithmic bytes / step
time, wall clock over the timed steps), the read's µs per call and its
fraction of MI355X's 8 TB/s (the read alone, called as many times again,
each call bracketed by HIP events on the stream it runs on), and the CPU
oracle timed on this host as a reported baseline.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged decode read µs/call + achieved HBM GB/s (% peak), 8B-shaped layer"
HBM_PEAK_GBS = 8000.0

# HBM bytes per one-call decode step and per plain read, measured with
# rocprofv3 FETCH_SIZE + WRITE_SIZE and scaled by a plain copy of known size
# (profiles/decode_stream_<workload>_hbm_counters.md), valid only for the
# kernel sources they were taken on.
PROFILED_TRAFFIC = {
    "llama3_8b_layer": {"src": "397b8efc058c85e1", "step_bytes": 577262720, "read_bytes": 576641116},
}
KERNEL_SOURCES = ("decode.hip", "pkv_internal.h", "abi.hip")


def kernel_source_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "paged_kv_cache_13_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def profiled_traffic(workload):
    rec = PROFILED_TRAFFIC.get(workload)
    if rec is None or rec["src"] != kernel_source_hash():
        return None
    return rec["step_bytes"]


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama3_8b_layer")
    ap.add_argument("--partition", type=int, default=0, help="partition_tokens (0 = library default)")
    ap.add_argument("--flushed", type=int, default=30,
                    help="extra reads timed with the 256 MB Infinity Cache flushed before each")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target CPU time of the oracle baseline (0 disables it)")
    ap.add_argument("--headline-only", action="store_true",
                    help="skip the other workloads (small fp32 reads, skewed batch, decode runs)")
    ap.add_argument("--prompt-scatter-only", action="store_true",
                    help="time only the 65536-token prompt scatter (for profiling)")
    ap.add_argument("--prompt-block-size", type=int, default=16,
                    help="pool block size of the --prompt-scatter-only workload (8, 16 or 32)")
    ap.add_argument("--prefill-chunk-only", action="store_true",
                    help="only time the multi-query read of a 64-query chunk over 16 rows of the 8B "
                         "layer (the prefill_chunk entry of other_workloads) and print it")
    ap.add_argument("--graph-step-only", action="store_true",
                    help="only time the 8B layer's one-call decode step eager and replayed from a "
                         "captured HIP graph (the decode_step_graph entry of other_workloads) and print it")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device-to-device copy 5 times (a kernel of "
                         "known traffic, to scale HBM counters by) and exit")
    return ap.parse_args()


def cpu_threads():
    """Host threads for the parallel oracle leg: the cores this process may
    run on, at most 16 (one GPU's share of its host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baseline(batch, new_k, new_v, slots_h, budget_s):
    """The CPU oracle (plain C, fp64) on the same inputs, copied to host
    memory outside the timing: scatter of the step's new tokens, then the read
    of every row.  Two legs: one thread, repeated until about `budget_s` / 2
    seconds of CPU work; then every host core this process may use, each
    thread calling the unchanged oracle on its share of the rows (rows
    i, i + T, ...; ctypes releases the GIL during the call), for about as
    long.  The parallel leg is the reported value."""
    import concurrent.futures

    import numpy as np
    import torch

    import oracle
    from paged_kv_cache_13_amd import harness

    oracle.build()
    oracle._load()
    q = batch.q.cpu()
    kp = batch.k_pool.cpu()
    vp = batch.v_pool.cpu()
    kn, vn = new_k.cpu(), new_v.cpu()
    cfg = batch.cfg
    nbytes = harness.read_bytes(batch.ctx_host, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim,
                                cfg.block_size, 2, 2)
    nbytes += harness.scatter_bytes(cfg.rows, cfg.n_kv_heads, cfg.head_dim, 2)

    def repeat(step, budget):
        reps, spent = 0, 0.0
        while spent < budget and (reps == 0 or spent / reps * (reps + 1) <= 2 * budget):
            t0 = time.perf_counter()
            step()
            spent += time.perf_counter() - t0
            reps += 1
        return spent / reps, reps

    def serial_step():
        oracle.reshape_and_cache(kn, vn, slots_h, kp, vp)
        oracle.paged_attention(q, kp, vp, batch.table_host, batch.ctx_host, batch.scale)

    threads = cpu_threads()
    shares = [np.arange(i, cfg.rows, threads) for i in range(threads)]
    shares = [(q[torch.from_numpy(ix)], batch.table_host[ix], batch.ctx_host[ix]) for ix in shares if ix.size]
    pool = concurrent.futures.ThreadPoolExecutor(len(shares))

    def parallel_step():
        oracle.reshape_and_cache(kn, vn, slots_h, kp, vp)
        list(pool.map(lambda s: oracle.paged_attention(s[0], kp, vp, s[1], s[2], batch.scale), shares))

    one_s, one_reps = repeat(serial_step, budget_s / 2)
    par_s, par_reps = repeat(parallel_step, budget_s / 2)
    pool.shutdown()
    return {"value": round(nbytes / par_s / 1e9, 4), "unit": "GB/s", "cores": len(shares), "kind": "oracle",
            "ms_per_step": round(par_s * 1e3, 2),
            "sample": "the full workload (%d rows, sum ctx %d): scatter + read per step, plain C in fp64; "
                      "%d step(s) on %d threads (rows split round-robin), %d step(s) on one thread"
                      % (cfg.rows, int(batch.ctx_host.sum()), par_reps, len(shares), one_reps),
            "single_thread": {"value": round(nbytes / one_s / 1e9, 4), "unit": "GB/s", "cores": 1,
                              "ms_per_step": round(one_s * 1e3, 2)},
            "nproc": os.cpu_count(), "cpu": cpu_model()}


def _timed(fn, stream, calls, lead_cycles=200000):
    """Mean and median µs of `calls` calls of fn, each bracketed by HIP events.
    A short spin kernel runs before each call so that the host has enqueued
    the events and the call before the GPU reaches them: the events then
    measure GPU time only, not Python launch overhead."""
    import numpy as np
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]
    for a, b in ev:
        torch.cuda._sleep(lead_cycles)
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    us = np.array([a.elapsed_time(b) for a, b in ev]) * 1e3
    return float(us.mean()), float(np.median(us))


def other_workloads(dev, stream):
    """The remaining synthetic workloads: each read's µs and HBM rate, and the
    decode-run sweep's per-step scatter / paged read / gathered-rectangle read."""
    import numpy as np
    import torch

    import paged_kv_cache_13_amd as pkv
    from paged_kv_cache_13_amd import harness, synth

    res = {}
    for name, calls in (("tiny_f32", 100), ("gqa_f32", 100), ("skewed_long", 20)):
        cfg = synth.CONFIGS[name]
        b = synth.make_batch(cfg, device=dev)
        out = torch.empty_like(b.q)
        ws = torch.zeros(max(pkv.workspace_size(b.q, b.k_pool, b.block_table), 1), dtype=torch.uint8, device=dev)

        def read():
            pkv.paged_attention_into(b.q, b.k_pool, b.v_pool, b.block_table, b.context_lens, b.scale, out, ws)

        for _ in range(5):
            read()
        mean, med = _timed(read, stream, calls)
        e = 2 if cfg.dtype == "bf16" else 4
        nb = harness.read_bytes(b.ctx_host, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.block_size, e, e)
        res[name] = {"read_us": round(mean, 2), "read_us_median": round(med, 2), "read_bytes": nb,
                     "GB/s": round(nb / (mean * 1e-6) / 1e9, 1),
                     "pct_peak": round(100 * nb / (mean * 1e-6) / 1e9 / HBM_PEAK_GBS, 2),
                     "sum_ctx": int(b.ctx_host.sum())}
        del b, out, ws
    runs = {}
    for rows in (32, 128):
        for bs in (8, 16, 32):
            run = synth.DecodeRun(rows=rows, block_size=bs, prompt=512, steps=256, device=dev,
                                  seed=5000 + rows + bs)
            k, v, slots = run.prefill()
            pre_us, _ = _timed(lambda: pkv.reshape_and_cache(k, v, slots, run.k_pool, run.v_pool), stream, 1,
                               lead_cycles=2000000)
            # every step's inputs are drawn first (host-side block allocation),
            # so that the timed loop only enqueues GPU work
            steps = []
            for _ in range(run.steps):
                q, kn, vn, sl = run.step()
                bt, cl = run.block_table(), run.context_lens()
                ws = torch.zeros(max(pkv.workspace_size(q, run.k_pool, bt), 1), dtype=torch.uint8, device=dev)
                steps.append((q, kn, vn, sl, bt, cl, ws, run.ctx_host.copy()))
            out = torch.empty(rows, run.n_heads, run.head_dim, dtype=torch.bfloat16, device=dev)
            stats = pkv.ReadCounters("streamed", block=pkv.read_tile(out, run.k_pool, steps[0][4]))
            t_sc, t_rd, t_step, t_rect, rbytes = [], [], [], [], 0
            for q, kn, vn, sl, bt, cl, ws, ctx in steps:
                # the step as one call first, then again as a scatter and a read
                # (writing the same token to the same slot again): the later
                # calls find more of the step's data in the Infinity Cache
                t_step.append(_timed(lambda: pkv.decode_step(q, kn, vn, sl, run.k_pool, run.v_pool, bt, cl,
                                                             run.scale, out=out, workspace=ws), stream, 1)[0])
                t_sc.append(_timed(lambda: pkv.reshape_and_cache(kn, vn, sl, run.k_pool, run.v_pool), stream, 1)[0])
                t_rd.append(_timed(lambda: pkv.paged_attention_into(q, run.k_pool, run.v_pool, bt, cl, run.scale,
                                                                     out, ws), stream, 1)[0])
                t_rect.append(_timed(lambda: harness.gathered_rect_read(q, run.k_pool, run.v_pool, bt, cl,
                                                                        run.scale), stream, 1,
                                     lead_cycles=1000000)[0])
                stats.record(rows, run.n_heads, 1, int(ctx.max()))
                rbytes += harness.read_bytes(ctx, run.n_heads, run.n_kv_heads, run.head_dim, bs, 2, 2)
            rd = float(np.mean(t_rd))
            runs["rows%d_bs%d" % (rows, bs)] = {
                "prefill_scatter_us": round(pre_us, 1),
                "prefill_scatter_GB/s": round(harness.scatter_bytes(rows * run.prompt, run.n_kv_heads,
                                                                    run.head_dim, 2) / (pre_us * 1e-6) / 1e9, 1),
                "step_scatter_us": round(float(np.mean(t_sc)), 2), "step_read_us": round(rd, 2),
                "step_one_call_us": round(float(np.mean(t_step)), 2),
                "step_read_GB/s": round(rbytes / run.steps / (rd * 1e-6) / 1e9, 1),
                "step_rect_us": round(float(np.mean(t_rect)), 2),
                "rect_over_paged": round(float(np.mean(t_rect)) / rd, 2),
                "readstats": {"calls": stats.calls, "rows": stats.rows, "score_cells": stats.score_cells,
                              "held_cells": stats.held_cells, "saving": round(stats.saving, 2)}}
            del run, out, steps
    res["decode_run"] = runs
    res["decode_step_graph"] = graph_step(dev, stream)
    res["prompt_scatter"] = prompt_scatter(dev, stream)
    res["prefill_chunk"] = prefill_chunk(dev, stream)
    return res


def prompt_scatter(dev, stream, rows=128, prompt=512, calls=20, block_size=16):
    """The slot-mapping scatter of a whole prompt batch (rows x prompt tokens,
    each row's prompt in consecutive slots of its blocks, 8 kv heads, head_dim
    128, bf16, blocks of 16): µs per call and the HBM rate of the bytes it
    must move (K and V read once and written once, plus the slots)."""
    import torch

    import paged_kv_cache_13_amd as pkv
    from paged_kv_cache_13_amd import harness, synth

    run = synth.DecodeRun(rows=rows, block_size=block_size, prompt=prompt, steps=0, device=dev, seed=11)
    k, v, slots = run.prefill()

    def call():
        pkv.reshape_and_cache(k, v, slots, run.k_pool, run.v_pool)

    for _ in range(3):
        call()
    mean, med = _timed(call, stream, calls, lead_cycles=1000000)
    nb = harness.scatter_bytes(k.shape[0], k.shape[1], k.shape[2], 2)
    return {"tokens": int(k.shape[0]), "block_size": block_size, "bytes": nb, "us": round(mean, 2),
            "us_median": round(med, 2),
            "GB/s": round(nb / (mean * 1e-6) / 1e9, 1)}


def prefill_chunk(dev, stream, rows=16, qlen=64):
    """Multi-query read of a 64-query chunk at the end of every row of an
    8B-shaped layer (lengths uniform in [512, 4096]): µs per call, K/V bytes
    read once (HBM floor) and the causal FLOPs."""
    import numpy as np
    import torch

    import paged_kv_cache_13_amd as pkv
    from paged_kv_cache_13_amd import harness, synth

    cfg = synth.CONFIGS["llama3_8b_layer"].replace(rows=rows, seed=7)
    b = synth.make_batch(cfg, device=dev)
    g = torch.Generator(device=dev).manual_seed(8)
    q = torch.randn(rows, qlen, cfg.n_heads, cfg.head_dim, generator=g, device=dev).to(torch.bfloat16)
    out = torch.empty_like(q)
    ws = torch.zeros(max(pkv.workspace_size_multi(q, b.k_pool, b.block_table), 1), dtype=torch.uint8, device=dev)

    def call():
        pkv.paged_attention_multi(q, b.k_pool, b.v_pool, b.block_table, b.context_lens, b.scale, out=out,
                                  workspace=ws)

    for _ in range(10):  # the first calls on fresh pools run 5-12 % slow
        call()
    mean, med = _timed(call, stream, 20)
    kv = harness.read_bytes(b.ctx_host, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.block_size, 2, 2)
    kv += (qlen - 1) * rows * cfg.n_heads * cfg.head_dim * 4  # the other queries' q and out
    vis = sum(int(n) - qlen + i + 1 for n in b.ctx_host for i in range(qlen))
    flops = 4 * cfg.n_heads * cfg.head_dim * vis
    return {"rows": rows, "query_len": qlen, "sum_ctx": int(b.ctx_host.sum()), "us": round(mean, 2),
            "us_median": round(med, 2), "GB/s_kv_once": round(kv / (mean * 1e-6) / 1e9, 1),
            "TFLOP/s": round(flops / (mean * 1e-6) / 1e12, 2)}


def graph_step(dev, stream, reps=100, per_graph=8):
    """The 8B-shaped layer's whole decode step (scatter + read) as one library
    call, eager and replayed from captured HIP graphs: GPU µs per step (events,
    host ahead) and wall-clock µs per step for back-to-back steps.  Each graph
    launch costs a fixed gap before its first kernel (about 8 us in a kernel
    trace on this runtime), so a graph of one step pays it every step; a graph
    of `per_graph` steps (as a serving loop would capture many layers) pays it
    once for all of them."""
    import torch

    import paged_kv_cache_13_amd as pkv
    from paged_kv_cache_13_amd import synth

    cfg = synth.CONFIGS["llama3_8b_layer"]
    b = synth.make_batch(cfg, device=dev)
    bs = cfg.block_size
    last = b.ctx_host - 1
    slots = torch.from_numpy((b.table_host[range(cfg.rows), last // bs].astype("int64") * bs + last % bs)).to(dev)
    g = torch.Generator(device=dev).manual_seed(cfg.seed + 200)
    kn = torch.randn(cfg.rows, cfg.n_kv_heads, cfg.head_dim, generator=g, device=dev).to(b.q.dtype)
    vn = torch.randn(cfg.rows, cfg.n_kv_heads, cfg.head_dim, generator=g, device=dev).to(b.q.dtype)
    out = torch.empty_like(b.q)
    ws = torch.zeros(max(pkv.workspace_size(b.q, b.k_pool, b.block_table), 1), dtype=torch.uint8, device=dev)

    def step():
        pkv.decode_step(b.q, kn, vn, slots, b.k_pool, b.v_pool, b.block_table, b.context_lens, b.scale,
                        out=out, workspace=ws)

    for _ in range(10):
        step()
    eager_us, _ = _timed(step, stream, 50)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    graph_n = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph_n):
        for _ in range(per_graph):
            step()
    for _ in range(10):
        graph.replay()
        graph_n.replay()
    graph_us, _ = _timed(graph.replay, stream, 50)
    graph_n_us, _ = _timed(graph_n.replay, stream, 20)
    walls = {}
    for name, fn, n in (("eager", step, 1), ("graph", graph.replay, 1), ("graph_n", graph_n.replay, per_graph)):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps // n):
            fn()
        torch.cuda.synchronize()
        walls[name] = (time.perf_counter() - t0) / (reps // n * n) * 1e6
    return {"workload": cfg.name, "eager_step_us": round(eager_us, 2), "graph_step_us": round(graph_us, 2),
            "graph_%d_steps_us_per_step" % per_graph: round(graph_n_us / per_graph, 2),
            "eager_wall_us_per_step": round(walls["eager"], 2), "graph_wall_us_per_step": round(walls["graph"], 2),
            "graph_%d_steps_wall_us_per_step" % per_graph: round(walls["graph_n"], 2)}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import paged_kv_cache_13_amd as pkv
    from paged_kv_cache_13_amd import harness, synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": src.numel() * 4,
                          "copy_calibration_bytes_written": dst.numel() * 4, "calls": 5}))
        return
    pkv.load_library()
    if args.prompt_scatter_only:
        stream = torch.cuda.current_stream()
        print(json.dumps({"prompt_scatter": prompt_scatter(dev, stream, block_size=args.prompt_block_size)}),
              flush=True)
        return
    if args.prefill_chunk_only:
        stream = torch.cuda.current_stream()
        print(json.dumps({"prefill_chunk": prefill_chunk(dev, stream)}), flush=True)
        return
    if args.graph_step_only:
        stream = torch.cuda.current_stream()
        print(json.dumps({"decode_step_graph": graph_step(dev, stream)}), flush=True)
        return
    cfg = synth.CONFIGS[args.workload]
    batch = synth.make_batch(cfg, device=dev)
    bs = cfg.block_size
    elem = 2 if cfg.dtype == "bf16" else 4

    # The step's new token of each row is its last position (already counted in
    # context_lens): its slot is overwritten every step, so every step reads the
    # same lengths.
    last = batch.ctx_host - 1
    slots_h = (batch.table_host[np.arange(cfg.rows), last // bs].astype(np.int64) * bs + last % bs)
    slots = torch.from_numpy(slots_h).to(dev)
    g = torch.Generator(device=dev).manual_seed(cfg.seed + 100)
    new_k = torch.randn(cfg.rows, cfg.n_kv_heads, cfg.head_dim, generator=g, device=dev).to(batch.q.dtype)
    new_v = torch.randn(cfg.rows, cfg.n_kv_heads, cfg.head_dim, generator=g, device=dev).to(batch.q.dtype)
    out = torch.empty_like(batch.q)
    wsz = pkv.workspace_size(batch.q, batch.k_pool, batch.block_table, partition_tokens=args.partition)
    ws = torch.empty(max(wsz, 1), dtype=torch.uint8, device=dev)

    def step():  # one call: append every row's new token, then read
        pkv.decode_step(batch.q, new_k, new_v, slots, batch.k_pool, batch.v_pool, batch.block_table,
                        batch.context_lens, batch.scale, out=out, workspace=ws,
                        partition_tokens=args.partition)

    def read():
        pkv.paged_attention_into(batch.q, batch.k_pool, batch.v_pool, batch.block_table,
                                 batch.context_lens, batch.scale, out, ws,
                                 partition_tokens=args.partition)

    stream = torch.cuda.current_stream(dev)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # the timed steps: wall clock over K back-to-back steps
    K = args.steps
    mk_events = lambda: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                         for _ in range(K)]
    region = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    region[0].record(stream)
    for i in range(K):  # the timed steps, back to back
        step()
    region[1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    region_ms = region[0].elapsed_time(region[1])

    def per_call(fn):  # K more calls, each bracketed by HIP events on its stream
        ev = mk_events()
        for i in range(K):
            ev[i][0].record(stream)
            fn()
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        return np.array([a.elapsed_time(b) for a, b in ev])

    step_ms = per_call(step)  # the step's kernels, launch by launch
    for _ in range(args.warmup):
        read()
    read_ms = per_call(read)  # the read alone

    # reads with the Infinity Cache flushed (a 512 MiB write) before each
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    fl_ms = []
    for _ in range(args.flushed):
        flush.fill_(1)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        read()
        b.record(stream)
        torch.cuda.synchronize()
        fl_ms.append(a.elapsed_time(b))
    del flush

    rb = harness.read_bytes(batch.ctx_host, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, bs, elem, elem)
    sb = harness.scatter_bytes(cfg.rows, cfg.n_kv_heads, cfg.head_dim, elem)
    ms_step = wall * 1e3 / K
    read_us = float(read_ms.mean() * 1e3)
    step_us = float(step_ms.mean() * 1e3)
    region_us = region_ms * 1e3 / K  # one event pair around the K timed steps, per step
    achieved = (rb + sb) / (region_us * 1e-6) / 1e9
    stats = pkv.ReadCounters("streamed", block=pkv.read_tile(batch.q, batch.k_pool, batch.block_table))
    stats.record(cfg.rows, cfg.n_heads, 1, int(batch.ctx_host.max()))
    print("readstats: mode=%s block=%d calls=%d rows=%d score_cells=%d held_cells=%d saving=%.1fx"
          % (stats.mode, stats.block, stats.calls, stats.rows, stats.score_cells, stats.held_cells,
             stats.saving), file=sys.stderr)

    res = {
        "metric": METRIC,
        "value": round((rb + sb) / (ms_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name, "rows": cfg.rows, "n_heads": cfg.n_heads,
                   "n_kv_heads": cfg.n_kv_heads, "head_dim": cfg.head_dim, "block_size": bs,
                   "context_lens": "uniform[512,4096]" if cfg.name == "llama3_8b_layer" else str(cfg.ctx),
                   "sum_ctx": int(batch.ctx_host.sum()), "num_blocks": batch.num_blocks,
                   "partition_tokens": args.partition or "library default"},
        "read_us": round(read_us, 2),
        "read_us_median": round(float(np.median(read_ms)) * 1e3, 2),
        "read_us_p10": round(float(np.percentile(read_ms, 10)) * 1e3, 2),
        "read_us_p90": round(float(np.percentile(read_ms, 90)) * 1e3, 2),
        "read_us_flushed": round(float(np.median(fl_ms)) * 1e3, 2) if fl_ms else None,
        "read_pct_peak": round(100 * rb / (read_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 2),
        "read_bytes": rb,
        "scatter_bytes": sb,
        "step_us": round(step_us, 2),
        "step_us_median": round(float(np.median(step_ms)) * 1e3, 2),
        "step_us_timed_region": round(region_us, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": profiled_traffic(cfg.name),
                     "kernel": "one-call decode step: decode_stream (appending the step's tokens) + "
                               "decode_stream_merge",
                     "bytes_per_launch": rb + sb, "us_per_launch": round(region_us, 2)},
    }
    if args.cpu_seconds > 0:
        res["cpu_baseline"] = cpu_baseline(batch, new_k, new_v, slots_h, args.cpu_seconds)
    if not args.headline_only:
        del batch, out, ws, new_k, new_v
        torch.cuda.empty_cache()
        res["other_workloads"] = other_workloads(dev, stream)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
