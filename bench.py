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
"""
import argparse
import hashlib
import json
import math
import os
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


def kernel_source_sha():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def calibrate_sleep(torch, stream):
    """Spin-kernel cycles per microsecond on this device."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(1000)
    e0.record(stream)
    torch.cuda._sleep(2_000_000)
    e1.record(stream)
    torch.cuda.synchronize()
    return 2_000_000 / max(e0.elapsed_time(e1) * 1e3, 1.0)


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=400)
    p.add_argument("--warmup", type=int, default=40)
    p.add_argument("--workload", default="c5", choices=["c2", "c3", "c4", "c5", "c4f8", "c5f8"])
    p.add_argument("--num-slices", type=int, default=None,
                   help="slices of the row statistic (default: the workload's primary count)")
    p.add_argument("--rotate-mib", type=int, default=2048,
                   help="total size of the rotated buffer sets")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=16.0,
                   help="approximate CPU time spent timing the oracle")
    p.add_argument("--waves-per-row", type=int, default=0)
    p.add_argument("--max-workgroups", type=int, default=0)
    p.add_argument("--cached-rows", type=int, default=0)
    p.add_argument("--calibrate-copy", action="store_true",
                   help="also launch a plain elementwise copy of known size (counter calibration)")
    p.add_argument("--main-only", action="store_true",
                   help="time only the main forward (no other slicing, copy, latency, headwise or "
                        "split-path figures): the profiler runs use this")
    p.add_argument("--quiet", action="store_true")
    return p.parse_args()


def log(args, *a):
    if not args.quiet:
        print("[bench]", *a, file=sys.stderr, flush=True)


def cpu_baseline(d, num_slices, seconds):
    """The fp64 oracle, as it is, on a bounded sample of the workload's rows."""
    import numpy as np
    import oracle
    cores = min(CPU_SHARE, os.cpu_count() or 1)
    oracle.set_threads(cores)
    w = d["w"]
    # sample: the first `rows` tokens of q and k; grow until one pass is >= 0.5 s
    rows = min(w.T, 256)
    qs = oracle.as_f32(d["q"])
    ks = oracle.as_f32(d["k"])
    gq, gk = oracle.as_f32(d["gamma_q"]), oracle.as_f32(d["gamma_k"])
    while True:
        t0 = time.perf_counter()
        oracle.qk_forward(qs[:rows], ks[:rows], gq, gk, w.eps, num_slices)
        dt = time.perf_counter() - t0
        if dt >= 0.5 or rows >= w.T:
            break
        rows = min(w.T, rows * 2)
    reps = max(1, int(seconds / max(dt, 1e-6)))
    t0 = time.perf_counter()
    for _ in range(reps):
        oracle.qk_forward(qs[:rows], ks[:rows], gq, gk, w.eps, num_slices)
    total = time.perf_counter() - t0
    # the same oracle on one thread, for about a fifth of the time
    oracle.set_threads(1)
    t0 = time.perf_counter()
    oracle.qk_forward(qs[:rows], ks[:rows], gq, gk, w.eps, num_slices)
    one = time.perf_counter() - t0
    reps1 = max(1, int(seconds / 5.0 / max(one, 1e-6)))
    t0 = time.perf_counter()
    for _ in range(reps1):
        oracle.qk_forward(qs[:rows], ks[:rows], gq, gk, w.eps, num_slices)
    one = time.perf_counter() - t0
    return {"value": rows * reps / total, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": "%d of %d tokens (q %d + k %d columns, %s), K=%d, %d passes in %.1f s" % (
                rows, w.T, w.hq, w.hk, w.dtype, num_slices, reps, total),
            "one_thread": {"value": rows * reps1 / one, "unit": "tokens/s",
                           "sample": "%d tokens, %d passes in %.1f s" % (rows, reps1, one)},
            "host_cpus": os.cpu_count()}


def split_path(torch, qk, w, sets, gq, gk, ctx, stream, timed, K, args):
    """The split entry points over the workload's rows. Two readings:
    the whole computation on this GPU (every slice's partial_stats, then every
    slice's apply_stats, for q and k), and one tensor-parallel rank's share
    (slice 0 of q and of k: its partial sums, then its normalisation with all
    K partials). Bytes count what each call must move: x read by both calls,
    y written once, gamma once, and the partial sums written and read."""
    dev = gq.device
    eb = w.elem_bytes
    stats = (torch.zeros((K, w.T), dtype=torch.float32, device=dev),
             torch.zeros((K, w.T), dtype=torch.float32, device=dev))
    views = []
    for q, k, yq, yk in sets:
        per = []
        for x, y, g, st, H in ((q, yq, gq, stats[0], w.hq), (k, yk, gk, stats[1], w.hk)):
            ws = H // K
            per.append([(x[:, s * ws:(s + 1) * ws], y[:, s * ws:(s + 1) * ws], g[s * ws:(s + 1) * ws], st, H, s)
                        for s in range(K)])
        views.append(per)

    def stats_of(sl):
        for xs, _, _, st, _, s in sl:
            qk.partial_stats(xs, s, K, stats=st, ctx=ctx, stream=stream)

    def apply_of(sl):
        for xs, ys, gs, st, H, _ in sl:
            qk.apply_stats(xs, gs, st, H, eps=w.eps, out=ys, ctx=ctx, stream=stream)

    def whole(i):
        for sl in views[i % len(views)]:
            stats_of(sl)
        for sl in views[i % len(views)]:
            apply_of(sl)

    def rank(i):
        per = views[i % len(views)]
        for sl in per:
            stats_of(sl[:1])
        for sl in per:
            apply_of(sl[:1])

    n = max(10, min(args.steps, 50))
    for i in range(5):
        whole(i)
    whole_ms = timed(n, whole, launches=4 * K)[0]
    rank_ms = timed(n, rank, launches=4)[0]
    H2 = w.hq + w.hk
    whole_bytes = 3 * w.T * H2 * eb + H2 * eb + 2 * (K * w.T * 4 + K * K * w.T * 4)
    rank_bytes = 3 * w.T * H2 // K * eb + H2 // K * eb + 2 * (w.T * 4 + K * w.T * 4)
    return {"split_path": {
        "num_slices": K,
        "whole_us": whole_ms * 1e3, "whole_launches": 4 * K, "whole_bytes": whole_bytes,
        "whole_gbs": whole_bytes / (whole_ms * 1e-3) / 1e9,
        "rank_share_us": rank_ms * 1e3, "rank_share_launches": 4, "rank_share_bytes": rank_bytes,
        "rank_share_gbs": rank_bytes / (rank_ms * 1e-3) / 1e9}}


def secondary(torch, qk, workloads, w, args, K, sets, gq, gk, ctx, stream, dev, timed, step):
    """Figures next to the main one: the workload's other slice count, a
    same-bytes device copy (the achievable-bandwidth ceiling), the host's
    call-to-completion latency, the headwise form over the same rows, and the
    split path."""
    eb = w.elem_bytes
    extra = {}
    for k_alt in w.slices:
        if k_alt == K:
            continue
        for i in range(args.warmup):
            step(i, k_alt)
        extra["kernel_us_K%d" % k_alt] = timed(args.steps, lambda i: step(i, k_alt))[0] * 1e3
    nb = w.T * (w.hq + w.hk) * eb
    csets = max(2, math.ceil(args.rotate_mib * 2**20 / (2 * nb)))
    cbufs = [(torch.empty(nb, dtype=torch.uint8, device=dev), torch.empty(nb, dtype=torch.uint8, device=dev))
             for _ in range(csets)]
    for s_, t_ in cbufs:
        t_.copy_(s_)
    copy_ms = timed(args.steps, lambda i: cbufs[i % csets][1].copy_(cbufs[i % csets][0]))[0]
    del cbufs
    extra["copy_same_bytes_us"] = copy_ms * 1e3
    extra["copy_same_bytes_gbs"] = 2 * nb / (copy_ms * 1e-3) / 1e9

    # host cost of one C call (validation, planning, launch) with the
    # arguments marshalled once, as a C caller would pass them
    import ctypes
    q, k, yq, yk = sets[0]
    L = qk.lib()
    rq = qk.Rows(q.data_ptr(), yq.data_ptr(), w.hq, w.hq, w.hq)
    rk = qk.Rows(k.data_ptr(), yk.data_ptr(), w.hk, w.hk, w.hk)
    dt = qk._dtype_code(q)
    sp = ctypes.c_void_p(stream.cuda_stream)
    n_host = min(args.steps, 200)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(n_host):
        L.qknorm_forward(ctx.handle, dt, w.T, ctypes.byref(rq), ctypes.byref(rk), gq.data_ptr(), gk.data_ptr(),
                         ctypes.c_float(w.eps), K, sp)
    extra["host_c_call_us"] = (time.perf_counter() - t0) * 1e6 / n_host
    torch.cuda.synchronize()

    # host view of one call: enqueue, then wait for completion (decode latency)
    lat = []
    for i in range(min(args.steps, 200)):
        t0 = time.perf_counter()
        step(i)
        torch.cuda.synchronize()
        lat.append((time.perf_counter() - t0) * 1e6)
    lat.sort()
    extra["host_call_to_done_us_p10_p50_p90"] = [lat[len(lat) // 10], lat[len(lat) // 2],
                                                  lat[(9 * len(lat)) // 10]]

    # headwise QK-Norm over the same rows (heads of the model's width)
    D = workloads.HEAD_DIM[args.workload]
    hgq = workloads.head_weights(w, "q", D).to(dev)
    hgk = workloads.head_weights(w, "k", D).to(dev)

    def head_step(i):
        q, k, yq, yk = sets[i % len(sets)]
        qk.forward_headwise(q, k, hgq, hgk, D, eps=w.eps, out_q=yq, out_k=yk, ctx=ctx, stream=stream)

    for i in range(args.warmup):
        head_step(i)
    head_ms = timed(args.steps, head_step)[0]
    head_bytes = 2 * w.T * (w.hq + w.hk) * eb + 2 * D * eb
    extra["headwise"] = {"head_dim": D, "kernel_us": head_ms * 1e3, "algorithmic_bytes": head_bytes,
                         "gbs": head_bytes / (head_ms * 1e-3) / 1e9,
                         "frac": head_bytes / (head_ms * 1e-3) / 1e9 / HBM_PEAK_GBS}

    # the split path (partial statistics, then apply) over the same rows
    if max(w.slices) > 1:
        extra.update(split_path(torch, qk, w, sets, gq, gk, ctx, stream, timed, max(w.slices), args))

    # the same shape with FP8-E4M3 rows (bf16 weights), when one exists
    f8 = args.workload + "f8"
    if f8 in workloads.WORKLOADS:
        extra["fp8"] = fp8_figures(torch, qk, workloads, f8, args, ctx, stream, dev, timed)
    return extra


def fp8_figures(torch, qk, workloads, name, args, ctx, stream, dev, timed):
    """The fused forward on the FP8 version of the workload, rotated over
    buffer sets like the main figure, for each of its slice counts."""
    d = workloads.generate(name)
    w = d["w"]
    nb = w.T * (w.hq + w.hk) * w.elem_bytes * (1 if w.in_place else 2)
    nsets = max(2, math.ceil(args.rotate_mib * 2**20 / nb))
    q0, k0 = d["q"].to(dev), d["k"].to(dev)
    gq, gk = d["gamma_q"].to(dev), d["gamma_k"].to(dev)
    sets = []
    for _ in range(nsets):
        q, k = q0.clone(), k0.clone()
        sets.append((q, k, q, k) if w.in_place else (q, k, torch.empty_like(q), torch.empty_like(k)))
    del q0, k0
    out = {"workload": "%s: T=%d, q rows %d, k rows %d, e4m3 in/out, bf16 weights%s" % (
        name, w.T, w.hq, w.hk, ", in place" if w.in_place else ""),
        "algorithmic_bytes": w.algorithmic_bytes()}
    for K in w.slices:
        def step(i, K=K):
            q, k, yq, yk = sets[i % nsets]
            qk.forward(q, k, gq, gk, eps=w.eps, num_slices=K, out_q=yq, out_k=yk, ctx=ctx, stream=stream)
        for i in range(args.warmup):
            step(i)
        ms = timed(args.steps, step)[0]
        gbs = w.algorithmic_bytes() / (ms * 1e-3) / 1e9
        out["K%d" % K] = {"kernel_us": ms * 1e3, "tokens_per_s": w.T / (ms * 1e-3), "gbs": gbs,
                          "frac": gbs / HBM_PEAK_GBS}
    del sets
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(requested --gpus %d, WORLD_SIZE %d)" % (args.gpus, world), file=sys.stderr)
        sys.exit(2)

    import torch
    import attention_qk_norm_amd as qk
    from attention_qk_norm_amd import workloads

    if not os.path.exists(qk.LIB_PATH):
        from attention_qk_norm_amd import build as qbuild
        qbuild.build()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    d = workloads.generate(args.workload)
    w = d["w"]
    K = args.num_slices or w.slices[0]
    eb = w.elem_bytes
    algo_bytes = w.algorithmic_bytes()
    log(args, "workload %s (%s): T=%d Hq=%d Hk=%d %s K=%d in_place=%s, %.1f MB per call" % (
        args.workload, w.name, w.T, w.hq, w.hk, w.dtype, K, w.in_place, algo_bytes / 1e6))

    # buffer sets, rotated so consecutive launches touch different memory
    set_bytes = w.T * (w.hq + w.hk) * eb * (1 if w.in_place else 2)
    nsets = max(2, math.ceil(args.rotate_mib * 2**20 / set_bytes))
    q0, k0 = d["q"].to(dev), d["k"].to(dev)
    gq, gk = d["gamma_q"].to(dev), d["gamma_k"].to(dev)
    sets = []
    for _ in range(nsets):
        q, k = q0.clone(), k0.clone()
        if w.in_place:
            sets.append((q, k, q, k))
        else:
            sets.append((q, k, torch.empty_like(q), torch.empty_like(k)))
    del q0, k0
    log(args, "%d buffer sets, %.0f MiB" % (nsets, nsets * set_bytes / 2**20))

    ctx = qk.Context(0, waves_per_row=args.waves_per_row, max_workgroups=args.max_workgroups,
                     cached_rows=args.cached_rows)
    stream = torch.cuda.current_stream(dev)

    def step(i, num_slices=K):
        q, k, yq, yk = sets[i % nsets]
        qk.forward(q, k, gq, gk, eps=w.eps, num_slices=num_slices, out_q=yq, out_k=yk, ctx=ctx,
                   stream=stream)

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

    # The GPU first runs a spin kernel long enough for the host to enqueue all
    # timed launches behind it, so the timed region measures back-to-back
    # kernels, not the host's launch rate.
    cyc_per_us = calibrate_sleep(torch, stream)

    def timed(n, fn, launches=1):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        torch.cuda._sleep(int(cyc_per_us * (200.0 + 40.0 * n * launches)))
        e0.record(stream)
        h0 = time.perf_counter()
        for i in range(n):
            fn(i)
        host_us = (time.perf_counter() - h0) * 1e6
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n, host_us

    # timed region: K launches back to back, bracketed by events
    ms_per_step, host_us = timed(args.steps, step)
    kern_ms = ms_per_step

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
    ev_p10, ev_p50, ev_p90 = per[len(per) // 10], per[len(per) // 2], per[(9 * len(per)) // 10]

    extra = {}
    if not args.main_only:
        extra.update(secondary(torch, qk, workloads, w, args, K, sets, gq, gk, ctx, stream, dev, timed, step))
    achieved_gbs = algo_bytes / (kern_ms * 1e-3) / 1e9
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
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "%s %s: T=%d, q rows %d, k rows %d, %s in/out, %s values, K=%d slices%s" % (
            args.workload, w.name, w.T, w.hq, w.hk, w.dtype, w.dist, K, ", in place" if w.in_place else ""),
            "tokens": w.T, "q_width": w.hq, "k_width": w.hk, "io_dtype": w.dtype, "num_slices": K,
            "in_place": w.in_place, "buffer_sets": nsets, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": achieved_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved_gbs / HBM_PEAK_GBS, "traffic": traffic},
        "hbm_gbs": achieved_gbs,
        "algorithmic_bytes_per_launch": algo_bytes,
        "kernel_us": kern_ms * 1e3,
        "host_enqueue_us_per_launch": host_us / args.steps,
        "event_pair_us_p10_p50_p90": [ev_p10 * 1e3, ev_p50 * 1e3, ev_p90 * 1e3],
        "kernel_source_sha": kernel_source_sha(),
    }
    result.update({k2: v for k2, v in extra.items()})
    if calib:
        result["calibration_copy"] = calib
    if not args.no_cpu_baseline:
        log(args, "timing the CPU oracle (~%.0f s)" % args.cpu_seconds)
        result["cpu_baseline"] = cpu_baseline(d, K, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
