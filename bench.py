#!/usr/bin/env python3
"""Throughput of the fused layerwise QK-Norm forward on one MI355X.

One step = one fused forward (statistic, slice combine, scaling, store) over
the query rows and key rows of one batch of T tokens, inputs resident in HBM.
The default workload is the large-prefill configuration (T = 16384, query and
key rows of 4096 bf16, Laplace(0, 1) values, 8 column slices, in-place
output), the one measured against the HBM roofline. Buffer sets are rotated
so that no launch finds its data in the 256 MB Infinity Cache.

Prints one JSON line. The timed region is K launches back to back on the
stream the kernel runs on (torch's current stream), bracketed by HIP events;
a spin kernel queued ahead of it keeps the host's launch rate out of the
measurement. The per-launch average of that region is the kernel time used
for the roofline.

Beside the headline the line carries, each timed the same way:
  - the other workloads (2048-token grouped-query prefill, 256- and
    64-token decode batches) with their own rotated buffers;
  - the ceiling: hand-written streaming copy, read-only and write-only
    kernels (libqkceil) over the same bytes, and an empty launch;
  - the headwise form, the split path (whole computation, and one rank's
    share on contiguous shards), FP8 rows of the same shape;
  - the fp64 CPU oracle on the host's cores (median of 5 runs);
  - the shader clock the back-to-back launches met (a one-wavefront probe
    between every 10 launches of a separate pass): long runs of the most
    arithmetic-heavy launches lower it.
"""
import argparse
import ctypes
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "QK-Norm tokens/sec and achieved HBM GB/s (% of peak) at 1 MI355X"
HBM_PEAK_GBS = 8000.0  # MI355X published HBM3E bandwidth
CPU_SHARE = 16         # host cores per GPU on the measurement boxes
KERNEL_SOURCES = ("attention_qk_norm_amd/csrc/qknorm_kernels.h",
                  "attention_qk_norm_amd/csrc/qknorm_kernels_f32.hip",
                  "attention_qk_norm_amd/csrc/qknorm_kernels_bf16.hip",
                  "attention_qk_norm_amd/csrc/qknorm_kernels_fp8.hip",
                  "attention_qk_norm_amd/csrc/qknorm_launch.cpp",
                  "attention_qk_norm_amd/csrc/qknorm_api.cpp",
                  "attention_qk_norm_amd/csrc/qknorm_launch.h")
TRAFFIC_FILE = "profiles/qknorm_fwd_{workload}_traffic.json"
ELEM_BYTES = {"f32": 4, "bf16": 2, "fp8": 1}
ROTATE_MIB = 2048      # total size of the rotated buffer sets of each figure


def kernel_source_sha():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=400)
    p.add_argument("--warmup", type=int, default=40)
    p.add_argument("--workload", default="c5", choices=["c2", "c3", "c4", "c5", "c4f8", "c5f8"])
    p.add_argument("--num-slices", type=int, default=None,
                   help="slices of the row statistic (default: the workload's primary count)")
    p.add_argument("--rotate-mib", type=int, default=ROTATE_MIB,
                   help="total size of the rotated buffer sets")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="approximate CPU time spent timing the oracle (5 runs on all threads, "
                        "plus a fifth of it on one thread)")
    p.add_argument("--waves-per-row", type=int, default=0)
    p.add_argument("--max-workgroups", type=int, default=0)
    p.add_argument("--cached-rows", type=int, default=0)
    p.add_argument("--calibrate-copy", action="store_true",
                   help="also launch a plain elementwise copy of known size (counter calibration)")
    p.add_argument("--main-only", action="store_true",
                   help="time only the main forward (the profiler runs use this)")
    p.add_argument("--ceiling-only", action="store_true",
                   help="time only the ceiling kernels over the workload's bytes (the profiler runs use this)")
    p.add_argument("--quiet", action="store_true")
    return p.parse_args()


def log(args, *a):
    if not args.quiet:
        print("[bench]", *a, file=sys.stderr, flush=True)


class Clock:
    """Gated back-to-back timing on one stream: a spin kernel long enough for
    the host to enqueue every timed launch goes first, so the region between
    the two events measures the GPU, not Python's launch rate."""

    def __init__(self, torch, stream):
        self.torch = torch
        self.stream = stream
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(1000)
        e0.record(stream)
        torch.cuda._sleep(2_000_000)
        e1.record(stream)
        torch.cuda.synchronize()
        self.cyc_per_us = 2_000_000 / max(e0.elapsed_time(e1) * 1e3, 1.0)

    def region(self, n, fn, launches=1):
        """Milliseconds per step of n steps of fn(i), and the host's enqueue
        time in microseconds."""
        torch = self.torch
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        torch.cuda._sleep(int(self.cyc_per_us * (200.0 + 40.0 * n * launches)))
        e0.record(self.stream)
        h0 = time.perf_counter()
        for i in range(n):
            fn(i)
        host_us = (time.perf_counter() - h0) * 1e6
        e1.record(self.stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n, host_us

    def shader_clock(self, n, fn, every=10):
        """The shader clock met by n back-to-back steps of fn(i) (gated like
        region()): a one-wavefront probe (libqkceil) samples it before every
        `every` steps and after the last; MHz as min / median / max."""
        from attention_qk_norm_amd import ceiling
        torch = self.torch
        m = n // every + 2
        buf = torch.zeros(2 * m, dtype=torch.int64, device=torch.device("cuda", torch.cuda.current_device()))
        sp = ctypes.c_void_p(self.stream.cuda_stream)
        torch.cuda.synchronize()
        torch.cuda._sleep(int(self.cyc_per_us * (200.0 + 40.0 * n)))
        k = 0
        for i in range(n):
            if i % every == 0:
                ceiling.clock(buf.data_ptr() + 16 * k, sp)
                k += 1
            fn(i)
        ceiling.clock(buf.data_ptr() + 16 * k, sp)
        k += 1
        torch.cuda.synchronize()
        mhz = [100.0 * c / r for c, r in buf.cpu().view(-1, 2)[:k].tolist() if r > 0]  # 100 MHz real-time clock
        return {"min": min(mhz), "median": statistics.median(mhz), "max": max(mhz), "samples": len(mhz)}

    def steady(self, n, warmup, fn, launches=1):
        for i in range(warmup):
            fn(i)
        return self.region(n, fn, launches)[0]

    def call_to_done(self, n, fn):
        """Host view of single calls: enqueue, then wait for completion (the
        latency a decode step sees). p10/p50/p90 in microseconds."""
        lat = []
        for i in range(n):
            t0 = time.perf_counter()
            fn(i)
            self.torch.cuda.synchronize()
            lat.append((time.perf_counter() - t0) * 1e6)
        lat.sort()
        return [lat[len(lat) // 10], lat[len(lat) // 2], lat[(9 * len(lat)) // 10]]


def buffer_sets(torch, d, dev, rotate_mib):
    """Rotated copies of a workload's rows: (q, k, y_q, y_k) per set."""
    w = d["w"]
    set_bytes = w.T * (w.hq + w.hk) * w.elem_bytes * (1 if w.in_place else 2)
    nsets = max(2, math.ceil(rotate_mib * 2**20 / set_bytes))
    q0, k0 = d["q"].to(dev), d["k"].to(dev)
    sets = []
    for _ in range(nsets):
        q, k = q0.clone(), k0.clone()
        sets.append((q, k, q, k) if w.in_place else (q, k, torch.empty_like(q), torch.empty_like(k)))
    return sets


def cpu_baseline(d, num_slices, seconds):
    """The fp64 oracle, as it is, on a bounded sample of the workload's rows:
    5 runs on all the host's threads (up to 16), together about 80% of
    `seconds`, and 5 on one thread in the rest; the medians are reported,
    with every run's value and the spread."""
    import oracle
    cores = min(CPU_SHARE, os.cpu_count() or 1)
    w = d["w"]
    qs, ks = oracle.as_f32(d["q"]), oracle.as_f32(d["k"])
    gq, gk = oracle.as_f32(d["gamma_q"]), oracle.as_f32(d["gamma_k"])

    def runs(threads, run_seconds):
        oracle.set_threads(threads)
        rows = min(w.T, 64)
        while True:  # a sample of whole rows that takes at least a quarter of a run
            t0 = time.perf_counter()
            oracle.qk_forward(qs[:rows], ks[:rows], gq, gk, w.eps, num_slices)
            dt = time.perf_counter() - t0
            if dt >= run_seconds / 4 or rows >= w.T:
                break
            rows = min(w.T, rows * 2)
        reps = max(1, int(run_seconds / max(dt, 1e-6)))
        vals = []
        for _ in range(5):
            t0 = time.perf_counter()
            for _ in range(reps):
                oracle.qk_forward(qs[:rows], ks[:rows], gq, gk, w.eps, num_slices)
            vals.append(rows * reps / (time.perf_counter() - t0))
        return rows, reps, vals

    rows, reps, vals = runs(cores, seconds / 5 * 0.8)
    rows1, reps1, vals1 = runs(1, seconds / 5 * 0.2)
    oracle.set_threads(1)
    return {"value": statistics.median(vals), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": "%d of %d tokens (q %d + k %d columns, %s), K=%d, %d passes per run, median of 5 runs" % (
                rows, w.T, w.hq, w.hk, w.dtype, num_slices, reps),
            "runs": [round(v, 1) for v in vals], "min": min(vals), "max": max(vals),
            "one_thread": {"value": statistics.median(vals1), "unit": "tokens/s", "min": min(vals1),
                           "max": max(vals1),
                           "sample": "%d tokens, %d passes per run, median of 5 runs" % (rows1, reps1)},
            "host_cpus": os.cpu_count()}


def ceiling_figures(torch, clock, dev, nbytes, steps, warmup, rotate_mib, vpls=None):
    """The streaming kernels of libqkceil over `nbytes` per direction
    (rotated): the best copy over the per-lane vector counts, the read-only
    and write-only streams at the same count, and an empty launch."""
    from attention_qk_norm_amd import ceiling
    sp = ctypes.c_void_p(clock.stream.cuda_stream)
    stride = (nbytes + (2 << 20) - 1) // (2 << 20) * (2 << 20)
    nsets = max(2, math.ceil(rotate_mib * 2**20 / (2 * stride)))
    src = torch.empty(nsets * stride, dtype=torch.uint8, device=dev)
    dst = torch.empty(nsets * stride, dtype=torch.uint8, device=dev)
    sink = torch.empty(1024, dtype=torch.uint8, device=dev)
    src.random_()
    s0, d0 = src.data_ptr(), dst.data_ptr()
    copy_us = {}
    for vpl in (vpls or ceiling.VECTORS_PER_LANE):
        copy_us[vpl] = clock.steady(steps, warmup, lambda i, v=vpl: ceiling.copy(
            s0 + (i % nsets) * stride, d0 + (i % nsets) * stride, nbytes, v, sp)) * 1e3
    best = min(copy_us, key=copy_us.get)
    read_us = clock.steady(steps, warmup, lambda i: ceiling.read(
        s0 + (i % nsets) * stride, nbytes, best, sink.data_ptr(), sp)) * 1e3
    write_us = clock.steady(steps, warmup, lambda i: ceiling.write(
        d0 + (i % nsets) * stride, nbytes, best, sp)) * 1e3
    empty_us = clock.steady(steps, warmup, lambda i: ceiling.empty(1024, sp)) * 1e3
    del src, dst
    return {"bytes_each_way": nbytes, "copy_us": copy_us[best], "copy_vectors_per_lane": best,
            "copy_gbs": 2 * nbytes / (copy_us[best] * 1e-6) / 1e9,
            "copy_us_by_vectors_per_lane": {str(k): v for k, v in copy_us.items()},
            "read_us": read_us, "write_us": write_us, "empty_launch_us": empty_us}


def forward_step(qk, sets, gq, gk, eps, K, ctx, stream):
    def step(i):
        q, k, yq, yk = sets[i % len(sets)]
        qk.forward(q, k, gq, gk, eps=eps, num_slices=K, out_q=yq, out_k=yk, ctx=ctx, stream=stream)
    return step


def workload_figures(torch, qk, workloads, name, args, ctx, clock, dev, latency=False, ceiling=True):
    """One workload's fused forward (each of its slice counts) over its own
    rotated buffers, with the same-bytes copy ceiling and, for decode
    shapes, the host's call-to-completion latency."""
    d = workloads.generate(name)
    w = d["w"]
    sets = buffer_sets(torch, d, dev, args.rotate_mib)
    gq, gk = d["gamma_q"].to(dev), d["gamma_k"].to(dev)
    ab = w.algorithmic_bytes()
    out = {"workload": "%s %s: T=%d, q rows %d, k rows %d, %s%s" % (
        name, w.name, w.T, w.hq, w.hk, w.dtype, ", in place" if w.in_place else ""),
        "tokens": w.T, "algorithmic_bytes": ab}
    for K in w.slices:
        step = forward_step(qk, sets, gq, gk, w.eps, K, ctx, clock.stream)
        ms = clock.steady(args.steps, args.warmup, step)
        gbs = ab / (ms * 1e-3) / 1e9
        fig = {"kernel_us": ms * 1e3, "tokens_per_s": w.T / (ms * 1e-3), "gbs": gbs, "frac": gbs / HBM_PEAK_GBS,
               "shader_clock_mhz_back_to_back": clock.shader_clock(args.steps, step)}
        if latency:
            fig["call_to_done_us_p10_p50_p90"] = clock.call_to_done(min(args.steps, 200), step)
        out["K%d" % K] = fig
    del sets
    if ceiling:
        c = ceiling_figures(torch, clock, dev, w.T * (w.hq + w.hk) * w.elem_bytes, args.steps, args.warmup,
                            args.rotate_mib)
        c["kernel_over_copy"] = out["K%d" % w.slices[0]]["kernel_us"] / c["copy_us"]
        out["ceiling"] = c
    torch.cuda.empty_cache()
    return out


def split_figures(torch, qk, w, d, sets, gq, gk, ctx, clock, args):
    """The split entry points over the workload's rows (x read by both steps,
    y written once, gamma once, the partials written and read):
      whole: every slice's partial sums, then every slice's normalisation,
             both tensors per launch, on column views of the full rows (2K
             launches, the single-GPU emulation of K ranks);
      rank_share: one tensor-parallel rank's work on its own contiguous
             [T, H/K] shards of q and k (2 launches), and the same on column
             views (what a rank would not hold);
      partial_stats: the rank's statistics launch alone, a read-only pass,
             against the read-only ceiling over the same bytes."""
    dev = gq.device
    stream = clock.stream
    K = max(w.slices)
    eb = w.elem_bytes
    gb = ELEM_BYTES[w.gamma_dtype]
    T = w.T
    wq, wk = w.hq // K, w.hk // K
    sq = torch.zeros((K, T), dtype=torch.float32, device=dev)
    sk = torch.zeros((K, T), dtype=torch.float32, device=dev)

    def views(q, k, y_q, y_k, r):
        return (q[:, r * wq:(r + 1) * wq], k[:, r * wk:(r + 1) * wk], y_q[:, r * wq:(r + 1) * wq],
                y_k[:, r * wk:(r + 1) * wk])

    def whole(i):
        q, k, yq, yk = sets[i % len(sets)]
        for r in range(K):
            xq, xk, _, _ = views(q, k, yq, yk, r)
            qk.partial_stats_qk(xq, xk, r, K, sq, sk, ctx=ctx, stream=stream)
        for r in range(K):
            xq, xk, oq, ok = views(q, k, yq, yk, r)
            qk.apply_stats_qk(xq, xk, gq[r * wq:(r + 1) * wq], gk[r * wk:(r + 1) * wk], sq, sk, w.hq, w.hk,
                              eps=w.eps, out_q=oq, out_k=ok, ctx=ctx, stream=stream)

    # contiguous shards: each rotated set holds slice 0's columns of q and k, as rank 0 would
    shard_bytes = T * (wq + wk) * eb * (1 if w.in_place else 2)
    nsh = max(2, math.ceil(args.rotate_mib * 2**20 / shard_bytes))
    xq0 = d["q"][:, :wq].contiguous().to(dev)
    xk0 = d["k"][:, :wk].contiguous().to(dev)
    shards = []
    for _ in range(nsh):
        a, b = xq0.clone(), xk0.clone()
        shards.append((a, b, a, b) if w.in_place else (a, b, torch.empty_like(a), torch.empty_like(b)))
    gq0, gk0 = gq[:wq], gk[:wk]

    def rank_stats(i):
        a, b, _, _ = shards[i % nsh]
        qk.partial_stats_qk(a, b, 0, K, sq, sk, ctx=ctx, stream=stream)

    def rank(i):
        a, b, oa, ob = shards[i % nsh]
        qk.partial_stats_qk(a, b, 0, K, sq, sk, ctx=ctx, stream=stream)
        qk.apply_stats_qk(a, b, gq0, gk0, sq, sk, w.hq, w.hk, eps=w.eps, out_q=oa, out_k=ob, ctx=ctx,
                          stream=stream)

    def rank_views(i):
        q, k, yq, yk = sets[i % len(sets)]
        xq, xk, oq, ok = views(q, k, yq, yk, 0)
        qk.partial_stats_qk(xq, xk, 0, K, sq, sk, ctx=ctx, stream=stream)
        qk.apply_stats_qk(xq, xk, gq0, gk0, sq, sk, w.hq, w.hk, eps=w.eps, out_q=oq, out_k=ok, ctx=ctx,
                          stream=stream)

    n = max(10, min(args.steps, 100))
    whole_ms = clock.steady(n, 5, whole, launches=2 * K)
    rank_ms = clock.steady(n, 5, rank, launches=2)
    rank_views_ms = clock.steady(n, 5, rank_views, launches=2)
    stats_ms = clock.steady(n, 5, rank_stats)
    H2 = w.hq + w.hk
    stat_bytes = 2 * K * T * 4
    whole_bytes = 3 * T * H2 * eb + H2 * gb + 2 * (K * T * 4) + K * stat_bytes
    shard_x = T * (wq + wk) * eb
    rank_bytes = 3 * shard_x + (wq + wk) * gb + 2 * T * 4 + stat_bytes
    stats_bytes = shard_x + 2 * T * 4
    read_ceiling = ceiling_figures(clock.torch, clock, dev, shard_x, n, 5, args.rotate_mib, vpls=(1, 2, 4, 8))
    del shards

    def fig(ms, nbytes, launches):
        gbs = nbytes / (ms * 1e-3) / 1e9
        return {"us": ms * 1e3, "launches": launches, "bytes": nbytes, "gbs": gbs, "frac": gbs / HBM_PEAK_GBS}

    return {"split_path": {
        "num_slices": K,
        "whole": fig(whole_ms, whole_bytes, 2 * K),
        "rank_share_contiguous": fig(rank_ms, rank_bytes, 2),
        "rank_share_column_views": fig(rank_views_ms, rank_bytes, 2),
        "partial_stats_contiguous": dict(fig(stats_ms, stats_bytes, 1),
                                         read_only_ceiling_us=read_ceiling["read_us"],
                                         empty_launch_us=read_ceiling["empty_launch_us"])}}


def fp8_figures(torch, qk, workloads, name, args, ctx, clock, dev):
    """The fused forward on the FP8 version of the workload, rotated over
    buffer sets like the main figure, for each of its slice counts."""
    d = workloads.generate(name)
    w = d["w"]
    sets = buffer_sets(torch, d, dev, args.rotate_mib)
    gq, gk = d["gamma_q"].to(dev), d["gamma_k"].to(dev)
    out = {"workload": "%s: T=%d, q rows %d, k rows %d, e4m3 in/out, bf16 weights%s" % (
        name, w.T, w.hq, w.hk, ", in place" if w.in_place else ""),
        "algorithmic_bytes": w.algorithmic_bytes()}
    for K in w.slices:
        step = forward_step(qk, sets, gq, gk, w.eps, K, ctx, clock.stream)
        ms = clock.steady(args.steps, args.warmup, step)
        gbs = w.algorithmic_bytes() / (ms * 1e-3) / 1e9
        out["K%d" % K] = {"kernel_us": ms * 1e3, "tokens_per_s": w.T / (ms * 1e-3), "gbs": gbs,
                          "frac": gbs / HBM_PEAK_GBS,
                          "shader_clock_mhz_back_to_back": clock.shader_clock(args.steps, step)}
    del sets
    torch.cuda.empty_cache()
    return out


def secondary(torch, qk, workloads, w, d, args, K, sets, gq, gk, ctx, clock, dev, step):
    """Figures next to the main one."""
    eb = w.elem_bytes
    extra = {}
    for k_alt in w.slices:
        if k_alt != K:
            extra["kernel_us_K%d" % k_alt] = clock.steady(args.steps, args.warmup,
                                                          lambda i: step(i, k_alt)) * 1e3

    # host cost of one C call (validation, planning, launch) with the
    # arguments marshalled once, as a C caller would pass them
    q, k, yq, yk = sets[0]
    L = qk.lib()
    rq = qk.Rows(q.data_ptr(), yq.data_ptr(), w.hq, w.hq, w.hq)
    rk = qk.Rows(k.data_ptr(), yk.data_ptr(), w.hk, w.hk, w.hk)
    dt = qk._dtype_code(q)
    sp = ctypes.c_void_p(clock.stream.cuda_stream)
    n_host = min(args.steps, 200)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(n_host):
        L.qknorm_forward(ctx.handle, dt, w.T, ctypes.byref(rq), ctypes.byref(rk), gq.data_ptr(), gk.data_ptr(),
                         ctypes.c_float(w.eps), K, sp)
    extra["host_c_call_us"] = (time.perf_counter() - t0) * 1e6 / n_host
    torch.cuda.synchronize()
    extra["host_call_to_done_us_p10_p50_p90"] = clock.call_to_done(min(args.steps, 200), step)

    # the same-bytes ceiling
    c = ceiling_figures(torch, clock, dev, w.T * (w.hq + w.hk) * eb, args.steps, args.warmup, args.rotate_mib)
    extra["ceiling"] = c

    # headwise QK-Norm over the same rows (heads of the model's width)
    D = workloads.HEAD_DIM[args.workload]
    hgq = workloads.head_weights(w, "q", D).to(dev)
    hgk = workloads.head_weights(w, "k", D).to(dev)

    def head_step(i):
        q, k, yq, yk = sets[i % len(sets)]
        qk.forward_headwise(q, k, hgq, hgk, D, eps=w.eps, out_q=yq, out_k=yk, ctx=ctx, stream=clock.stream)

    head_ms = clock.steady(args.steps, args.warmup, head_step)
    head_bytes = 2 * w.T * (w.hq + w.hk) * eb + 2 * D * eb
    extra["headwise"] = {"head_dim": D, "kernel_us": head_ms * 1e3, "algorithmic_bytes": head_bytes,
                         "gbs": head_bytes / (head_ms * 1e-3) / 1e9,
                         "frac": head_bytes / (head_ms * 1e-3) / 1e9 / HBM_PEAK_GBS}

    if max(w.slices) > 1:
        extra.update(split_figures(torch, qk, w, d, sets, gq, gk, ctx, clock, args))
    return extra


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(requested --gpus %d, WORLD_SIZE %d)" % (args.gpus, world), file=sys.stderr)
        sys.exit(2)

    import torch
    import attention_qk_norm_amd as qk
    from attention_qk_norm_amd import ceiling as qkceil
    from attention_qk_norm_amd import workloads

    if not os.path.exists(qk.LIB_PATH) or not os.path.exists(qkceil.LIB_PATH):
        from attention_qk_norm_amd import build as qbuild
        qbuild.build()
        qbuild.build_ceiling()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    clock = Clock(torch, stream)

    d = workloads.generate(args.workload)
    w = d["w"]
    K = args.num_slices or w.slices[0]
    algo_bytes = w.algorithmic_bytes()
    log(args, "workload %s (%s): T=%d Hq=%d Hk=%d %s K=%d in_place=%s, %.1f MB per call" % (
        args.workload, w.name, w.T, w.hq, w.hk, w.dtype, K, w.in_place, algo_bytes / 1e6))

    if args.ceiling_only:
        c = ceiling_figures(torch, clock, dev, w.T * (w.hq + w.hk) * w.elem_bytes, args.steps, args.warmup,
                            args.rotate_mib)
        print(json.dumps({"ceiling_only": args.workload, "ceiling": c}), flush=True)
        return

    sets = buffer_sets(torch, d, dev, args.rotate_mib)
    log(args, "%d buffer sets" % len(sets))
    gq, gk = d["gamma_q"].to(dev), d["gamma_k"].to(dev)
    ctx = qk.Context(0, waves_per_row=args.waves_per_row, max_workgroups=args.max_workgroups,
                     cached_rows=args.cached_rows)

    def step(i, num_slices=K):
        q, k, yq, yk = sets[i % len(sets)]
        qk.forward(q, k, gq, gk, eps=w.eps, num_slices=num_slices, out_q=yq, out_k=yk, ctx=ctx, stream=stream)

    calib = None
    if args.calibrate_copy:
        n = 64 * 2**20  # elements of fp32: 256 MiB read + 256 MiB written
        src = torch.randn(n, device=dev)
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        calib = {"kernel": "torch.neg fp32", "read_bytes": 4 * n, "write_bytes": 4 * n}
        del src, dst

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # timed region: K launches back to back, bracketed by events
    ms_per_step, host_us = clock.region(args.steps, step)

    # per-launch event pairs (they add a little time of their own): spread only
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        starts[i].record(stream)
        step(i)
        ends[i].record(stream)
    torch.cuda.synchronize()
    per = sorted(s_.elapsed_time(e_) for s_, e_ in zip(starts, ends))
    ev = [per[len(per) // 10] * 1e3, per[len(per) // 2] * 1e3, per[(9 * len(per)) // 10] * 1e3]

    extra = {}
    if not args.main_only:
        extra["shader_clock_mhz_back_to_back"] = clock.shader_clock(args.steps, step)
        extra.update(secondary(torch, qk, workloads, w, d, args, K, sets, gq, gk, ctx, clock, dev, step))
        del sets
        torch.cuda.empty_cache()
        if args.workload == "c5":
            log(args, "other workloads")
            extra["workloads"] = {
                "c4": workload_figures(torch, qk, workloads, "c4", args, ctx, clock, dev),
                "c3": workload_figures(torch, qk, workloads, "c3", args, ctx, clock, dev, latency=True),
                "c2": workload_figures(torch, qk, workloads, "c2", args, ctx, clock, dev, latency=True),
            }
        f8 = args.workload + "f8"
        if f8 in workloads.WORKLOADS:
            extra["fp8"] = fp8_figures(torch, qk, workloads, f8, args, ctx, clock, dev)
    achieved_gbs = algo_bytes / (ms_per_step * 1e-3) / 1e9
    traffic = None
    tf = os.path.join(ROOT, TRAFFIC_FILE.format(workload=args.workload))
    if os.path.exists(tf):
        with open(tf) as f:
            t = json.load(f)
        if t.get("kernel_source_sha") == kernel_source_sha() and t.get("num_slices") == K:
            traffic = t.get("bytes_per_launch")

    result = {
        "metric": METRIC,
        "value": w.T / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "accumulate": "f32",
        "data": "synthetic",
        "config": {"workload": "%s %s: T=%d, q rows %d, k rows %d, %s in/out, %s values, K=%d slices%s" % (
            args.workload, w.name, w.T, w.hq, w.hk, w.dtype, w.dist, K, ", in place" if w.in_place else ""),
            "tokens": w.T, "q_width": w.hq, "k_width": w.hk, "io_dtype": w.dtype, "num_slices": K,
            "in_place": w.in_place, "buffer_sets": math.ceil(args.rotate_mib * 2**20 / (
                w.T * (w.hq + w.hk) * w.elem_bytes * (1 if w.in_place else 2))), "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": achieved_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved_gbs / HBM_PEAK_GBS, "traffic": traffic},
        "hbm_gbs": achieved_gbs,
        "algorithmic_bytes_per_launch": algo_bytes,
        "kernel_us": ms_per_step * 1e3,
        "host_enqueue_us_per_launch": host_us / args.steps,
        "event_pair_us_p10_p50_p90": ev,
        "kernel_source_sha": kernel_source_sha(),
    }
    result.update(extra)
    if "ceiling" in result:
        result["ceiling"]["kernel_over_copy"] = result["kernel_us"] / result["ceiling"]["copy_us"]
    if calib:
        result["calibration_copy"] = calib
    if not args.no_cpu_baseline:
        log(args, "timing the CPU oracle (~%.0f s)" % args.cpu_seconds)
        result["cpu_baseline"] = cpu_baseline(d, K, args.cpu_seconds)
    print(json.dumps(result), flush=True)
    try:
        import psutil
        kids = psutil.Process().children(recursive=True)
        if kids:
            log(args, "child processes at exit: %s" % [(p.pid, p.name()) for p in kids])
    except Exception:
        pass


if __name__ == "__main__":
    main()
