"""Parity of the HIP path (through the C ABI) with the fp64 oracle, on the GPU.

Every case prints what it runs before the GPU call so a failing run names it.
"""
import os

import numpy as np
import pytest
import torch

import attention_qk_norm_amd as qk
import oracle
from attention_qk_norm_amd import workloads
from conftest import read_golden
from gpu_checks import assert_near_each_other, assert_parity, host64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(*a):
    print("[case]", *a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _oracle_threads():
    oracle.set_threads(min(16, os.cpu_count() or 1))
    yield
    oracle.set_threads(1)


def gpu(t):
    return t.to(DEV).contiguous()


def run_forward(q, k, gq, gk, eps, K, in_place=False, ctx=None):
    qd, kd = gpu(q), (gpu(k) if k is not None else None)
    out_q = qd if in_place else None
    out_k = kd if (in_place and kd is not None) else None
    yq, yk = qk.forward(qd, kd, gpu(gq), gpu(gk) if gk is not None else None, eps=eps, num_slices=K,
                        out_q=out_q, out_k=out_k, ctx=ctx)
    torch.cuda.synchronize()
    return yq, yk


# ---- the five workloads at full size ------------------------------------------

@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5"])
def test_workload_parity(name):
    d = workloads.generate(name)
    w = d["w"]
    refs = {}
    outs = {}
    for K in w.slices:
        say(name, w.name, "T=%d Hq=%d Hk=%d %s K=%d in_place=%s" % (w.T, w.hq, w.hk, w.dtype, K, w.in_place))
        yq, yk = run_forward(d["q"], d["k"], d["gamma_q"], d["gamma_k"], w.eps, K, in_place=w.in_place)
        if not refs:
            refs["q"], _ = oracle.forward(d["q"], d["gamma_q"], w.eps, K)
            refs["k"], _ = oracle.forward(d["k"], d["gamma_k"], w.eps, K)
        eq = assert_parity(yq, refs["q"], w.torch_dtype, "%s q K=%d" % (name, K))
        ek = assert_parity(yk, refs["k"], w.torch_dtype, "%s k K=%d" % (name, K))
        print("  q errors", eq, "\n  k errors", ek, flush=True)
        outs[K] = (yq.cpu(), yk.cpu())
        del yq, yk
    # the K-slice statistic reaches the same outputs as one slice up to rounding
    if len(outs) > 1:
        (a_q, a_k), (b_q, b_k) = list(outs.values())[:2]
        for a, b in ((a_q, b_q), (a_k, b_k)):
            same = assert_near_each_other(a, b, w.torch_dtype, name + " K vs 1")
            print("  K=%d vs K=%d: %.4f of elements bitwise equal" % (w.slices[0], w.slices[1], same),
                  flush=True)


# ---- pins that hold on the GPU too ------------------------------------------------

def test_worked_example_on_gpu():
    """SwiftQK review section 4b, Eqs. (2)-(8), in fp32: fused with K = 2 and
    K = 1, and the per-shard split path."""
    g = read_golden("swiftqk_worked_example.txt")
    x = torch.tensor([g["x"]], dtype=torch.float32)
    gam = torch.tensor(g["gamma"], dtype=torch.float32)
    eps = g["eps"][0]
    ref, _ = oracle.forward(x, gam, eps, 2)
    for K in (2, 1):
        say("worked example fp32 K=%d" % K)
        yq, _ = run_forward(x, None, gam, None, eps, K)
        assert_parity(yq, ref, torch.float32, "worked example K=%d" % K)
        y = host64(yq)[0]
        for j in range(8):
            assert abs(y[j] - g["y"][j]) <= 0.5e-3 + abs(g["x"][j]) * 0.5e-4, (j, y[j])
    say("worked example split path")
    xd = gpu(x)
    stats = torch.zeros((2, 1), dtype=torch.float32, device=DEV)
    for r in range(2):
        qk.partial_stats(xd[:, 4 * r:4 * r + 4], r, 2, stats)
    torch.cuda.synchronize()
    assert stats.cpu().flatten().tolist() == g["S_local"]  # Eqs. 3-4, exact
    for r in range(2):
        yr = qk.apply_stats(xd[:, 4 * r:4 * r + 4], gpu(gam[4 * r:4 * r + 4]), stats, 8, eps)
        torch.cuda.synchronize()
        assert_parity(yr, ref[:, 4 * r:4 * r + 4], torch.float32, "Eq. %d" % (7 + r))


def test_four_element_closed_form_on_gpu():
    x = torch.tensor([[1.0, 2.0, -1.0, 0.5]])
    say("four-element closed form")
    y, _ = run_forward(x, None, torch.ones(4), None, 0.0, 1)
    assert_parity(y, np.array([[0.8, 1.6, -0.8, 0.4]]), torch.float32, "eps=0")
    y, _ = run_forward(x, None, torch.tensor([1.0, 0.5, 2.0, 4.0]), None, 0.0, 1)
    assert_parity(y, np.array([[0.8, 0.8, -1.6, 1.6]]), torch.float32, "gamma")


def bits(t):
    return t.cpu().contiguous().view(torch.uint8)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "fp8"])
def test_exact_sums_bitwise_across_slicings(dtype):
    """On n/16 inputs (exact in fp32, bf16 and e4m3) every partial is exact in
    fp32, so the statistic is the same whatever the slicing: K-slice outputs
    are bitwise those of K = 1, and the split path's partials equal the exact
    integer sums (which also pins each type's decoding of the squares)."""
    T, H = 37, 4096
    x = workloads.exact_sum_rows(T, H, dtype, 71)
    k = workloads.exact_sum_rows(T, 1024, dtype, 72)
    gdt = "bf16" if dtype == "fp8" else dtype
    gq = workloads.random_weights(H, gdt, 73)
    gk = workloads.random_weights(1024, gdt, 74)
    n = np.rint(host64(x) * 16).astype(np.int64)
    base = None
    for K in (1, 2, 4, 8, 16, 32, 64):
        say("exact sums", dtype, "K=%d" % K)
        yq, yk = run_forward(x, k, gq, gk, 1e-6, K)
        if base is None:
            base = (bits(yq), bits(yk))
            ref, _ = oracle.forward(x, gq, 1e-6, 1)
            assert_parity(yq, ref, workloads.DTYPES[dtype], "exact-sum forward")
        else:
            assert torch.equal(bits(yq), base[0]), K
            assert torch.equal(bits(yk), base[1]), K
        w = H // K
        xd = gpu(x)
        stats = torch.zeros((K, T), dtype=torch.float32, device=DEV)
        for s in range(K):
            qk.partial_stats(xd[:, s * w:(s + 1) * w], s, K, stats)
        torch.cuda.synchronize()
        ns = n.reshape(T, K, w)
        want = (ns * ns).sum(axis=2).T / 256.0
        assert np.array_equal(stats.cpu().numpy().astype(np.float64), want), K


# ---- split path -------------------------------------------------------------------

@pytest.mark.parametrize("name", ["c3", "c5"])
def test_split_path_matches_oracle(name):
    """partial_stats for every slice, then apply_stats per slice (the
    single-GPU analogue of scalar aggregation across tensor-parallel ranks)."""
    d = workloads.generate(name)
    w = d["w"]
    K = w.slices[0]
    T = min(w.T, 2048)
    for which in ("q", "k"):
        x, g = d[which][:T], d["gamma_" + which]
        H = x.shape[1]
        wd = H // K
        say("split path", name, which, "T=%d H=%d K=%d" % (T, H, K))
        ref, Pref = oracle.forward(x, g, w.eps, K)
        xd, gd = gpu(x), gpu(g)
        stats = torch.zeros((K, T), dtype=torch.float32, device=DEV)
        for s in range(K):
            qk.partial_stats(xd[:, s * wd:(s + 1) * wd], s, K, stats)
        torch.cuda.synchronize()
        np.testing.assert_allclose(stats.cpu().numpy(), Pref, rtol=1e-5)
        y = torch.empty_like(xd)
        for s in range(K):
            qk.apply_stats(xd[:, s * wd:(s + 1) * wd], gd[s * wd:(s + 1) * wd], stats, H, w.eps,
                           out=y[:, s * wd:(s + 1) * wd])
        torch.cuda.synchronize()
        assert_parity(y, ref, w.torch_dtype, "split %s %s" % (name, which))
        # in place, slice by slice
        for s in range(K):
            v = xd[:, s * wd:(s + 1) * wd]
            qk.apply_stats(v, gd[s * wd:(s + 1) * wd], stats, H, w.eps, out=v)
        torch.cuda.synchronize()
        assert torch.equal(xd.cpu(), y.cpu())


# ---- ragged shapes, strides, schedules ---------------------------------------------

RAGGED = [
    # (dtype, T, Hq, Hk, K)
    ("bf16", 1, 8, 8, 1),
    ("bf16", 3, 24, 16, 1),
    ("bf16", 5, 1000, 200, 5),       # slices of 25 / 5 vectors: 32- and 8-lane sub-teams over 4 wavefronts
    ("bf16", 63, 1032, 520, 1),
    ("bf16", 65, 5120, 1024, 4),     # C3/C4 widths, odd T
    ("bf16", 7, 4096, 4096, 64),     # 64 slices of 8 vectors: 4-lane sub-teams, LDS combine
    ("bf16", 7, 1536, 1536, 64),     # slices of 3 vectors: ragged 4-lane sub-teams
    ("bf16", 11, 2048, 512, 32),     # 8- and 2-lane sub-teams
    ("bf16", 5000, 1024, 1024, 8),   # 8-lane sub-teams, one wavefront per row
    ("bf16", 2048, 3072, 3072, 48),  # 4-lane sub-teams taking 3 slices each in turn
    ("f32", 9, 4096, 256, 64),       # 4-lane and 1-lane sub-teams
    ("bf16", 9, 12288, 1536, 3),
    ("bf16", 4, 16384, 16384, 8),    # wider than one wavefront's 16 slots
    ("bf16", 3, 65536, 8, 1),        # widest accepted row, with a tiny key row
    ("bf16", 2, 32768, 32768, 16),
    ("bf16", 3000, 16384, 2048, 8),  # 2-wavefront query teams in a narrow-slice launch with 8-lane key sub-teams
    ("bf16", 3700, 16384, 2048, 8),  # the same pair past 2^23 vectors: one launch per tensor
    ("f32", 3000, 4096, 1024, 8),    # 16-slot query rows beside 8-lane key sub-teams
    ("f32", 1, 4, 4, 1),
    ("f32", 6, 260, 12, 1),
    ("f32", 33, 256, 256, 4),
    ("f32", 17, 4096, 1024, 2),
    ("f32", 3, 8192, 8192, 8),
    ("f32", 2, 32768, 4, 1),         # widest fp32 row
    ("f32", 5, 1536, 1536, 48),      # 48 slices of 8 vectors: 4-lane sub-teams
    ("f32", 5, 1920, 1920, 40),      # slices of 12 vectors: ragged 4-lane sub-teams
    ("f32", 2048, 200, 200, 5),      # slices of 10 vectors: masked layout, one wavefront per row
    ("f32", 3, 200, 40, 10),         # masked layout over 4 wavefronts (LDS combine)
    # bodies of odd slot counts: 3 slots in teams of 4 wavefronts; 3 slots
    # over several rounds; 5 slots with a 1-slot key segment; 7 and 3 slots
    ("bf16", 128, 5120, 5120, 4),
    ("bf16", 4096, 1536, 1536, 1),
    ("bf16", 2048, 2560, 512, 1),
    ("f32", 1500, 1792, 768, 1),
    # many narrow slices over several rounds of wavefronts: 8-lane sub-teams
    # taking 4 (64 slices) or 2 (16 slices) slices in turn
    ("bf16", 5000, 4096, 4096, 64),
    ("bf16", 2048, 5120, 1024, 16),
    # query rows in teams of 4 wavefronts make several rounds of wavefronts,
    # so the 8-slot key rows take two wavefronts each
    ("bf16", 2048, 32768, 4096, 1),
    # several rounds: 8-slot query rows beside 2-slot key rows keep one
    # wavefront per row
    ("bf16", 5000, 4096, 1024, 1),
    # 16-wavefront workgroups: 65536-column query rows, and 8192-column key
    # rows widened to teams of 16 wavefronts (one slot each); fp32 likewise
    ("bf16", 600, 65536, 8192, 1),
    ("f32", 1200, 32768, 4096, 2),
]


@pytest.mark.parametrize("dtype,T,Hq,Hk,K", RAGGED)
def test_ragged_shapes(dtype, T, Hq, Hk, K):
    q = workloads.random_rows(T, Hq, dtype, [T, Hq, 1], dist="laplace")
    k = workloads.random_rows(T, Hk, dtype, [T, Hk, 2], scale=3.0)
    gq = workloads.random_weights(Hq, dtype, [Hq, 3])
    gk = workloads.random_weights(Hk, dtype, [Hk, 4])
    say("ragged", dtype, T, Hq, Hk, K)
    yq, yk = run_forward(q, k, gq, gk, 1e-6, K)
    rq, _ = oracle.forward(q, gq, 1e-6, K)
    rk, _ = oracle.forward(k, gk, 1e-6, K)
    assert_parity(yq, rq, workloads.DTYPES[dtype], "q")
    assert_parity(yk, rk, workloads.DTYPES[dtype], "k")


@pytest.mark.parametrize("opts", [dict(waves_per_row=1), dict(waves_per_row=2), dict(waves_per_row=4),
                                  dict(waves_per_row=8), dict(waves_per_row=16),
                                  dict(max_workgroups=7), dict(max_workgroups=300, waves_per_row=2),
                                  dict(max_workgroups=1), dict(max_workgroups=33, cached_rows=1),
                                  dict(max_workgroups=5, waves_per_row=4),
                                  dict(max_workgroups=3, waves_per_row=16),
                                  dict(cached_rows=1)],
                         ids=lambda o: ",".join("%s=%s" % kv for kv in o.items()))
def test_schedules_agree(opts):
    """Every schedule (team size, persistent grid, streaming stores) computes
    the same rows."""
    ctx = qk.Context(0, **opts)
    for dtype, T, Hq, Hk, K in (("bf16", 131, 5120, 1024, 4), ("f32", 45, 2048, 512, 2),
                                ("bf16", 70, 4096, 4096, 64), ("bf16", 19, 1000, 8, 1)):
        q = workloads.random_rows(T, Hq, dtype, [7, T])
        k = workloads.random_rows(T, Hk, dtype, [8, T])
        gq = workloads.random_weights(Hq, dtype, 9)
        gk = workloads.random_weights(Hk, dtype, 10)
        say("schedule", opts, dtype, T, Hq, Hk, K)
        try:
            yq, yk = run_forward(q, k, gq, gk, 1e-6, K, ctx=ctx)
        except qk.QKNormError as e:
            # a pinned team too small for the row is refused on the host
            assert e.status == qk.ERR_SHAPE and "waves_per_row" in opts
            continue
        rq, _ = oracle.forward(q, gq, 1e-6, K)
        rk, _ = oracle.forward(k, gk, 1e-6, K)
        assert_parity(yq, rq, workloads.DTYPES[dtype], "q")
        assert_parity(yk, rk, workloads.DTYPES[dtype], "k")


def test_strided_views_and_packed_qkv_in_place():
    """q and k as column blocks of one packed [T, Hq + Hk + Hv] buffer,
    normalised in place; the value columns and everything outside the views
    must come back untouched."""
    T, Hq, Hk, Hv = 77, 2048, 512, 512
    H = Hq + Hk + Hv
    qkv = workloads.random_rows(T, H, "bf16", 81)
    gq = workloads.random_weights(Hq, "bf16", 82)
    gk = workloads.random_weights(Hk, "bf16", 83)
    rq, _ = oracle.forward(qkv[:, :Hq], gq, 1e-6, 1)
    rk, _ = oracle.forward(qkv[:, Hq:Hq + Hk], gk, 1e-6, 1)
    dev = gpu(qkv)
    q, k = dev[:, :Hq], dev[:, Hq:Hq + Hk]
    say("packed qkv in place")
    qk.forward(q, k, gpu(gq), gpu(gk), eps=1e-6, out_q=q, out_k=k)
    torch.cuda.synchronize()
    out = dev.cpu()
    assert_parity(out[:, :Hq], rq, torch.bfloat16, "q")
    assert_parity(out[:, Hq:Hq + Hk], rk, torch.bfloat16, "k")
    assert torch.equal(out[:, Hq + Hk:], qkv[:, Hq + Hk:])
    # out-of-place into strided output views: bytes between rows stay as they were
    src = gpu(workloads.random_rows(T, Hq, "bf16", 84))
    canvas = torch.full((T, Hq + 64), 7.0, dtype=torch.bfloat16, device=DEV)
    say("strided output view")
    qk.forward(src, None, gpu(gq), None, out_q=canvas[:, 32:32 + Hq])
    torch.cuda.synchronize()
    c = canvas.cpu()
    ref, _ = oracle.forward(src.cpu(), gq, 1e-6, 1)
    assert_parity(c[:, 32:32 + Hq], ref, torch.bfloat16, "strided out")
    assert (c[:, :32] == 7.0).all() and (c[:, 32 + Hq:] == 7.0).all()


def test_special_rows():
    """Zero rows give zeros; eps = 0 is allowed; a constant row gives
    a / sqrt(a^2 + eps) * gamma; results are bit-reproducible."""
    T, H = 8, 1024
    x = workloads.random_rows(T, H, "f32", 91)
    x[0] = 0.0
    x[1] = 0.375
    g = workloads.random_weights(H, "f32", 92)
    for eps in (1e-6, 0.0):
        say("special rows eps=%g" % eps)
        xx = x.clone()
        if eps == 0.0:
            xx[0] = 1.0  # keep 0/0 out of it
        y1, _ = run_forward(xx, None, g, None, eps, 1)
        y2, _ = run_forward(xx, None, g, None, eps, 1)
        assert torch.equal(y1, y2)
        ref, _ = oracle.forward(xx, g, eps, 1)
        assert_parity(y1, ref, torch.float32, "eps=%g" % eps)
        if eps > 0:
            assert (y1[0] == 0).all()


@pytest.mark.parametrize("dtype", ["f32", "bf16", "fp8"])
def test_zero_rows_with_zero_eps(dtype):
    """With eps = 0 a zero row's statistic stays zero and Eq. 1 divides 0 by
    0: the oracle's fp64 arithmetic gives NaN for every element of that row
    (and +inf for its inverse RMS), and so does the GPU, fused, headwise and
    split; the other rows are normalised as usual."""
    T, H, D, zero = 6, 1024, 128, 2
    tdt = workloads.DTYPES[dtype]
    x = workloads.random_rows(T, H, dtype, 95).float()
    x[zero] = 0.0
    x = x.to(tdt)
    g = workloads.random_weights(H, "bf16" if dtype == "fp8" else dtype, 96)
    live = [t for t in range(T) if t != zero]

    def check(y, ref, what):
        yh = host64(y)
        assert np.isnan(ref[zero]).all() and np.isfinite(ref[live]).all(), what
        assert np.isnan(yh[zero]).all(), (what, yh[zero][:4])
        assert_parity(y.float()[live], ref[live], tdt, what)  # float: exact for every output type

    for K in (1, 4):
        say("zero row, eps=0", dtype, "K=%d" % K)
        y, _ = run_forward(x, None, g, None, 0.0, K)
        check(y, oracle.forward(x, g, 0.0, K)[0], "forward K=%d" % K)
        r, _ = qk.inv_rms(gpu(x), None, eps=0.0, num_slices=K)
        torch.cuda.synchronize()
        rr = oracle.inv_rms(x, 0.0, K)
        assert np.isposinf(rr[zero]) and torch.isposinf(r[zero]).item()
        assert_parity(r[live], rr[live], torch.float32, "inv_rms K=%d" % K)
        # split path: every slice's partials, then every slice scaled
        stats = torch.zeros((K, T), dtype=torch.float32, device=DEV)
        w = H // K
        xs = gpu(x)
        for s in range(K):
            qk.partial_stats(xs[:, s * w:(s + 1) * w], s, K, stats=stats)
        ys = torch.empty_like(xs)
        gd = gpu(g)
        for s in range(K):
            qk.apply_stats(xs[:, s * w:(s + 1) * w], gd[s * w:(s + 1) * w], stats, H, eps=0.0,
                           out=ys[:, s * w:(s + 1) * w])
        torch.cuda.synchronize()
        check(ys, oracle.forward(x, g, 0.0, K)[0], "split K=%d" % K)
    say("zero row, eps=0, headwise", dtype)
    gh = workloads.random_weights(D, "bf16" if dtype == "fp8" else dtype, 97)
    yh, _ = run_headwise(x, None, gh, None, D, 0.0)
    check(yh, oracle.qk_headwise(x, x, gh, gh, D, 0.0)[0], "headwise")


def test_empty_and_single_tensor():
    z = torch.empty((0, 4096), dtype=torch.bfloat16, device=DEV)
    g = torch.ones(4096, dtype=torch.bfloat16, device=DEV)
    say("T=0")
    yq, yk = qk.forward(z, z, g, g)
    torch.cuda.synchronize()
    assert yq.shape == (0, 4096)


# ---- headwise QK-Norm (one statistic per head) ---------------------------------

def run_headwise(q, k, gq, gk, D, eps, in_place=False, ctx=None):
    qd, kd = gpu(q), (gpu(k) if k is not None else None)
    out_q = qd if in_place else None
    out_k = kd if (in_place and kd is not None) else None
    yq, yk = qk.forward_headwise(qd, kd, gpu(gq), gpu(gk) if gk is not None else None, D, eps=eps,
                                 out_q=out_q, out_k=out_k, ctx=ctx)
    torch.cuda.synchronize()
    return yq, yk


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5"])
def test_headwise_workload_parity(name):
    """The five workloads' rows cut into their models' heads, each head
    normalised on its own (review, "Layerwise vs. headwise QK-Norm")."""
    d = workloads.generate(name)
    w = d["w"]
    D = workloads.HEAD_DIM[name]
    gq, gk = workloads.head_weights(w, "q", D), workloads.head_weights(w, "k", D)
    say("headwise", name, "T=%d Hq=%d Hk=%d %s head_dim=%d in_place=%s" % (w.T, w.hq, w.hk, w.dtype, D,
                                                                           w.in_place))
    yq, yk = run_headwise(d["q"], d["k"], gq, gk, D, w.eps, in_place=w.in_place)
    rq, rk = oracle.qk_headwise(d["q"], d["k"], gq, gk, D, w.eps)
    print("  q errors", assert_parity(yq, rq, w.torch_dtype, name + " headwise q"), flush=True)
    print("  k errors", assert_parity(yk, rk, w.torch_dtype, name + " headwise k"), flush=True)


HEAD_CASES = [
    # dtype, T, Hq, Hk, head_dim: every head width from one vector to 64,
    # ragged slots, teams of several wavefronts, rows past the grid
    ("bf16", 37, 2048, 512, 8),
    ("bf16", 37, 2048, 512, 16),
    ("bf16", 37, 2048, 512, 32),
    ("bf16", 37, 2048, 512, 64),
    ("bf16", 37, 5120, 1024, 128),
    ("bf16", 5, 5120, 1536, 256),
    ("bf16", 9, 8192, 512, 512),
    ("bf16", 3, 65536, 512, 512),     # widest bf16 row: 16-wavefront teams
    ("bf16", 2000, 1024, 128, 128),   # many rows per SIMD
    ("f32", 21, 1024, 256, 4),
    ("f32", 21, 1024, 256, 32),
    ("f32", 21, 3072, 256, 64),
    ("f32", 11, 4096, 512, 128),
    ("f32", 11, 4096, 1280, 256),
    ("f32", 1, 256, 256, 256),        # one head: the layerwise norm
]


@pytest.mark.parametrize("dtype,T,Hq,Hk,D", HEAD_CASES)
def test_headwise_shapes(dtype, T, Hq, Hk, D):
    q = workloads.random_rows(T, Hq, dtype, [T, Hq, D, 1], dist="laplace")
    k = workloads.random_rows(T, Hk, dtype, [T, Hk, D, 2], scale=3.0)
    # give the heads very different scales, so a statistic taken over the
    # wrong columns shows
    q = (q.float() * torch.linspace(0.01, 10.0, Hq // D).repeat_interleave(D)).to(q.dtype)
    gq = workloads.random_weights(D, dtype, [D, 3])
    gk = workloads.random_weights(D, dtype, [D, 4])
    say("headwise", dtype, T, Hq, Hk, D)
    yq, yk = run_headwise(q, k, gq, gk, D, 1e-6)
    rq, rk = oracle.qk_headwise(q, k, gq, gk, D, 1e-6)
    assert_parity(yq, rq, workloads.DTYPES[dtype], "q")
    assert_parity(yk, rk, workloads.DTYPES[dtype], "k")


def test_headwise_closed_form_on_gpu():
    """The worked example's row in two heads of 4: with eps = 0 the first
    head's RMS is exactly 1.25, the second head's sqrt(3.875)."""
    x = torch.tensor([[1.0, 2.0, -1.0, 0.5, 3.0, -2.0, 1.5, 0.5]])
    r1 = 1.0 / np.sqrt(3.875)
    say("headwise closed form")
    y, _ = run_headwise(x, None, torch.ones(4), None, 4, 0.0)
    ref = np.array([[0.8, 1.6, -0.8, 0.4, 3.0 * r1, -2.0 * r1, 1.5 * r1, 0.5 * r1]])
    assert_parity(y, ref, torch.float32, "heads of 4")
    y, _ = run_headwise(x, None, torch.tensor([1.0, 0.5, 2.0, 4.0]), None, 4, 0.0)
    ref = np.array([[0.8, 0.8, -1.6, 1.6, 3.0 * r1, -1.0 * r1, 3.0 * r1, 2.0 * r1]])
    assert_parity(y, ref, torch.float32, "shared weights")


@pytest.mark.parametrize("opts", [dict(waves_per_row=1), dict(waves_per_row=2), dict(waves_per_row=4),
                                  dict(waves_per_row=16), dict(max_workgroups=7),
                                  dict(max_workgroups=2, waves_per_row=4)],
                         ids=lambda o: ",".join("%s=%s" % kv for kv in o.items()))
def test_headwise_schedules_agree(opts):
    ctx = qk.Context(0, **opts)
    for dtype, T, Hq, Hk, D in (("bf16", 131, 5120, 1024, 128), ("f32", 45, 2048, 512, 64),
                                ("bf16", 19, 1024, 64, 64)):
        q = workloads.random_rows(T, Hq, dtype, [17, T])
        k = workloads.random_rows(T, Hk, dtype, [18, T])
        gq = workloads.random_weights(D, dtype, 19)
        gk = workloads.random_weights(D, dtype, 20)
        say("headwise schedule", opts, dtype, T, Hq, Hk, D)
        try:
            yq, yk = run_headwise(q, k, gq, gk, D, 1e-6, ctx=ctx)
        except qk.QKNormError as e:
            assert e.status == qk.ERR_SHAPE and "waves_per_row" in opts
            continue
        rq, rk = oracle.qk_headwise(q, k, gq, gk, D, 1e-6)
        assert_parity(yq, rq, workloads.DTYPES[dtype], "q")
        assert_parity(yk, rk, workloads.DTYPES[dtype], "k")


def test_headwise_packed_qkv_in_place():
    """Headwise norm of the query and key columns of a packed QKV buffer, in
    place; the value columns stay untouched."""
    T, Hq, Hk, Hv, D = 33, 2048, 256, 256, 128
    H = Hq + Hk + Hv
    qkv = workloads.random_rows(T, H, "bf16", 85)
    gq = workloads.random_weights(D, "bf16", 86)
    gk = workloads.random_weights(D, "bf16", 87)
    rq, rk = oracle.qk_headwise(qkv[:, :Hq], qkv[:, Hq:Hq + Hk], gq, gk, D, 1e-6)
    dev = gpu(qkv)
    q, k = dev[:, :Hq], dev[:, Hq:Hq + Hk]
    say("headwise packed qkv in place")
    qk.forward_headwise(q, k, gpu(gq), gpu(gk), D, eps=1e-6, out_q=q, out_k=k)
    torch.cuda.synchronize()
    out = dev.cpu()
    assert_parity(out[:, :Hq], rq, torch.bfloat16, "q")
    assert_parity(out[:, Hq:Hq + Hk], rk, torch.bfloat16, "k")
    assert torch.equal(out[:, Hq + Hk:], qkv[:, Hq + Hk:])


def test_headwise_zero_heads_and_reproducibility():
    """A head of zeros gives zeros (eps > 0) while its neighbours are
    normalised normally; repeated calls are bitwise identical."""
    T, H, D = 6, 1024, 128
    x = workloads.random_rows(T, H, "bf16", 88)
    x[:, 2 * D:3 * D] = 0.0
    g = workloads.random_weights(D, "bf16", 89)
    say("headwise zero head")
    y1, _ = run_headwise(x, None, g, None, D, 1e-6)
    y2, _ = run_headwise(x, None, g, None, D, 1e-6)
    assert torch.equal(y1, y2)
    assert (y1[:, 2 * D:3 * D] == 0).all()
    ref, _ = oracle.qk_headwise(x, x, g, g, D, 1e-6)
    assert_parity(y1, ref, torch.bfloat16, "zero head")


# ---- the per-token inverse RMS alone ------------------------------------------------

def forward_from_rinv(x, r, g, dtype):
    """(x * gamma) * r in fp32, rounded once to the output type: the fused
    forward's arithmetic, given its factor r (for bf16 rows x * gamma is
    exact in fp32)."""
    y = (x.float() * g.float()) * r.cpu()[:, None]
    return y.to(dtype)


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5"])
def test_inv_rms_workloads(name):
    """r_t against the oracle's Eq. 6 at fp32 tolerance, and bit for bit the
    factor the fused forward applies (same K)."""
    d = workloads.generate(name)
    w = d["w"]
    q, k = gpu(d["q"]), gpu(d["k"])
    for K in w.slices:
        say("inv_rms", name, "K=%d" % K)
        rq, rk = qk.inv_rms(q, k, eps=w.eps, num_slices=K)
        yq, yk = qk.forward(q, k, gpu(d["gamma_q"]), gpu(d["gamma_k"]), eps=w.eps, num_slices=K)
        torch.cuda.synchronize()
        for r, x, g, y, which in ((rq, d["q"], d["gamma_q"], yq, "q"), (rk, d["k"], d["gamma_k"], yk, "k")):
            ref = oracle.inv_rms(x, w.eps, K)
            assert_parity(r, ref, torch.float32, "%s rinv %s K=%d" % (name, which, K))
            assert torch.equal(y.cpu(), forward_from_rinv(x, r, g, w.torch_dtype)), (name, which, K)
        del yq, yk


@pytest.mark.parametrize("dtype,T,Hq,Hk,K", [("bf16", 70, 4096, 4096, 64), ("bf16", 5, 1536, 1536, 48),
                                            ("f32", 33, 1000, 8, 1), ("bf16", 3, 65536, 1024, 16),
                                            ("f32", 9, 32768, 4, 1), ("bf16", 3000, 512, 128, 2)])
def test_inv_rms_shapes(dtype, T, Hq, Hk, K):
    """Narrow slices (masked layout), the widest rows, many rows per SIMD."""
    q = workloads.random_rows(T, Hq, dtype, [T, Hq, 11], dist="laplace")
    k = workloads.random_rows(T, Hk, dtype, [T, Hk, 12], scale=0.01)
    say("inv_rms", dtype, T, Hq, Hk, K)
    rq, rk = qk.inv_rms(gpu(q), gpu(k), eps=1e-6, num_slices=K)
    torch.cuda.synchronize()
    assert_parity(rq, oracle.inv_rms(q, 1e-6, K), torch.float32, "q")
    assert_parity(rk, oracle.inv_rms(k, 1e-6, K), torch.float32, "k")


def test_inv_rms_worked_example_and_strided_rows():
    """Eq. 6 of the worked example (printed 0.6065), and rows read through a
    strided view of a packed buffer with outputs placed by the caller."""
    g = read_golden("swiftqk_worked_example.txt")
    x = torch.tensor([g["x"]], dtype=torch.float32)
    for K in (2, 1):
        say("inv_rms worked example K=%d" % K)
        r, _ = qk.inv_rms(gpu(x), eps=g["eps"][0], num_slices=K)
        torch.cuda.synchronize()
        assert abs(float(r[0]) - g["rms_inv"][0]) <= 0.5e-4
        assert_parity(r, oracle.inv_rms(x, g["eps"][0], K), torch.float32, "Eq. 6")
    T, Hq, Hk = 40, 2048, 512
    qkv = gpu(workloads.random_rows(T, Hq + 2 * Hk, "bf16", 95))
    out = torch.full((3, T), -1.0, device=DEV)
    say("inv_rms strided")
    qk.inv_rms(qkv[:, :Hq], qkv[:, Hq:Hq + Hk], out_q=out[0], out_k=out[2])
    torch.cuda.synchronize()
    host = qkv.cpu()
    assert_parity(out[0], oracle.inv_rms(host[:, :Hq], 1e-6, 1), torch.float32, "q")
    assert_parity(out[2], oracle.inv_rms(host[:, Hq:Hq + Hk], 1e-6, 1), torch.float32, "k")
    assert (out[1] == -1.0).all()


# ---- several narrow rows per wavefront -----------------------------------------

ROWS_PER_WAVE = [
    # dtype, T, Hq, Hk, K: rows of 1 or 2 slots and 16 or more rows per SIMD,
    # so each wavefront takes 4 or 2 rows; T not a multiple of the rows per
    # workgroup
    ("bf16", 9001, 1024, 512, 1),
    ("bf16", 9001, 1024, 512, 2),
    ("f32", 20001, 256, None, 1),
    ("f32", 17003, 512, 128, 4),
    ("fp8", 17000, 1024, 2048, 1),
    # rows of 1 slot: forward and apply launches take 4 rows per wavefront too
    ("bf16", 9001, 512, 512, 1),
    ("bf16", 12000, 512, None, 1),
    ("fp8", 17000, 1024, 1024, 1),
]


@pytest.mark.parametrize("dtype,T,Hq,Hk,K", ROWS_PER_WAVE)
def test_rows_per_wavefront(dtype, T, Hq, Hk, K):
    """Parity of every launch that gives a wavefront several rows, and bit
    equality with the same launches pinned to one row per wavefront (a
    forced team of one wavefront turns the rule off): a row's arithmetic
    does not depend on how many rows its wavefront holds."""
    gdt = "bf16" if dtype == "fp8" else dtype
    q = workloads.random_rows(T, Hq, dtype, [T, Hq, 5], dist="laplace")
    k = workloads.random_rows(T, Hk, dtype, [T, Hk, 6]) if Hk else None
    gq = workloads.random_weights(Hq, gdt, [Hq, 7])
    gk = workloads.random_weights(Hk, gdt, [Hk, 8]) if Hk else None
    say("rows per wavefront", dtype, T, Hq, Hk, K)
    yq, yk = run_forward(q, k, gq, gk, 1e-6, K)
    refq, Pq = oracle.forward(q, gq, 1e-6, K)
    assert_parity(yq, refq, workloads.DTYPES[dtype], "q")
    if Hk:
        refk, Pk = oracle.forward(k, gk, 1e-6, K)
        assert_parity(yk, refk, workloads.DTYPES[dtype], "k")
    rq, _ = qk.inv_rms(gpu(q), eps=1e-6, num_slices=K)
    torch.cuda.synchronize()
    assert_parity(rq, oracle.inv_rms(q, 1e-6, K), torch.float32, "rinv")
    one = qk.Context(0, waves_per_row=1)
    yq1, yk1 = run_forward(q, k, gq, gk, 1e-6, K, ctx=one)
    rq1, _ = qk.inv_rms(gpu(q), eps=1e-6, num_slices=K, ctx=one)
    torch.cuda.synchronize()
    assert torch.equal(yq, yq1) and torch.equal(rq, rq1)
    if Hk:
        assert torch.equal(yk, yk1)
    # the split path's apply step over whole rows, given the oracle's partials
    sq = torch.from_numpy(Pq.astype(np.float32)).to(DEV)
    sk = torch.from_numpy(Pk.astype(np.float32)).to(DEV) if Hk else None
    kd, gkd = (gpu(k), gpu(gk)) if Hk else (None, None)
    aq, ak = qk.apply_stats_qk(gpu(q), kd, gpu(gq), gkd, sq, sk, Hq, Hk or 0, eps=1e-6)
    aq1, ak1 = qk.apply_stats_qk(gpu(q), kd, gpu(gq), gkd, sq, sk, Hq, Hk or 0, eps=1e-6, ctx=one)
    torch.cuda.synchronize()
    assert_parity(aq, refq, workloads.DTYPES[dtype], "apply q")
    assert torch.equal(aq, aq1)
    if Hk:
        assert_parity(ak, refk, workloads.DTYPES[dtype], "apply k")
        assert torch.equal(ak, ak1)


PAIRED = [
    # dtype, T, Hq, Hk, layout: forward launches whose rows of both tensors
    # are one slice in one wavefront, with 1.75 to 4 paired wavefronts per
    # SIMD, so each wavefront takes one token's query row and key row
    ("bf16", 2048, 5120, 1024, "plain"),    # C4's shape
    ("bf16", 1795, 4096, 1024, "plain"),    # T not a multiple of the 4 rows of a workgroup
    ("bf16", 3001, 1024, 4096, "plain"),    # key rows wider: the segments swap
    ("bf16", 4096, 4608, 512, "plain"),     # 9-slot rows on the 10-slot body
    ("bf16", 2500, 1000, 200, "plain"),     # ragged last slots
    ("bf16", 2048, 3072, 1024, "in_place"),
    ("bf16", 2048, 2048, 512, "packed"),    # column blocks of one [T, Hq + Hk + Hv] buffer, in place
    ("f32", 2048, 2048, 512, "plain"),
    ("f32", 4000, 1000, 1000, "in_place"),
]


@pytest.mark.parametrize("dtype,T,Hq,Hk,layout", PAIRED)
def test_paired_rows(dtype, T, Hq, Hk, layout):
    """Parity of paired launches, and bit equality with the same launch
    unpaired (a forced team of one wavefront turns pairing off and keeps the
    rows' layouts): a row's arithmetic does not depend on which row shares
    its wavefront."""
    q = workloads.random_rows(T, Hq, dtype, [T, Hq, 11], dist="laplace")
    k = workloads.random_rows(T, Hk, dtype, [T, Hk, 12])
    gq = workloads.random_weights(Hq, dtype, [Hq, 13])
    gk = workloads.random_weights(Hk, dtype, [Hk, 14])
    say("paired rows", dtype, T, Hq, Hk, layout)
    refq, _ = oracle.forward(q, gq, 1e-6, 1)
    refk, _ = oracle.forward(k, gk, 1e-6, 1)
    outs = []
    for ctx in (None, qk.Context(0, waves_per_row=1)):
        if layout == "packed":
            hv = 256
            buf = torch.zeros((T, Hq + Hk + hv), dtype=q.dtype)
            buf[:, :Hq] = q
            buf[:, Hq:Hq + Hk] = k
            buf[:, Hq + Hk:] = 7.0
            bd = gpu(buf)
            qv, kv = bd[:, :Hq], bd[:, Hq:Hq + Hk]
            qk.forward(qv, kv, gpu(gq), gpu(gk), eps=1e-6, out_q=qv, out_k=kv, ctx=ctx)
            torch.cuda.synchronize()
            assert torch.equal(bd[:, Hq + Hk:].cpu(), buf[:, Hq + Hk:])  # the value columns are untouched
            yq, yk = qv, kv
        else:
            yq, yk = run_forward(q, k, gq, gk, 1e-6, 1, in_place=layout == "in_place", ctx=ctx)
        outs.append((yq, yk))
    (yq, yk), (yq1, yk1) = outs
    assert_parity(yq, refq, workloads.DTYPES[dtype], "q")
    assert_parity(yk, refk, workloads.DTYPES[dtype], "k")
    assert torch.equal(yq, yq1) and torch.equal(yk, yk1)


def test_split_path_on_a_rank_slice():
    """One rank's share of C5 under 8-way column slicing: slices of 512
    columns of 4096-wide rows, 16384 tokens (each wavefront takes 4 rows)."""
    T, H, K = 16384, 4096, 8
    w = H // K
    x = workloads.random_rows(T, H, "bf16", 97, dist="laplace")
    g = workloads.random_weights(H, "bf16", 98)
    ref, _ = oracle.forward(x, g, 1e-6, K)
    P = oracle.slice_sumsq(x, K)
    xd, gd = gpu(x), gpu(g)
    stats = torch.zeros((K, T), dtype=torch.float32, device=DEV)
    say("rank slice partial stats")
    for s in range(K):
        qk.partial_stats(xd[:, s * w:(s + 1) * w], s, K, stats)
    torch.cuda.synchronize()
    np.testing.assert_allclose(stats.cpu().double().numpy(), P, rtol=2e-6)
    for s in (0, 5, 7):
        say("rank slice apply", s)
        ys = qk.apply_stats(xd[:, s * w:(s + 1) * w], gd[s * w:(s + 1) * w], stats, H, eps=1e-6)
        torch.cuda.synchronize()
        assert_parity(ys, ref[:, s * w:(s + 1) * w], torch.bfloat16, "slice %d" % s)


@pytest.mark.parametrize("name", ["c3", "c5"])
def test_split_path_qk_on_rank_shards(name):
    """The two-tensor split calls on what a tensor-parallel rank holds: its
    own contiguous [T, H/K] shards of q and of k (Algorithm 1's X_local).
    Each rank publishes both tensors' partials in one launch, then
    normalises both shards in one launch with all K partials; the result is
    the oracle's, and bit for bit what the single-tensor calls give on
    strided column views of the full rows."""
    d = workloads.generate(name)
    w = d["w"]
    K = w.slices[0]
    T = min(w.T, 4096)
    q, k = d["q"][:T], d["k"][:T]
    refq, Pq = oracle.forward(q, d["gamma_q"], w.eps, K)
    refk, Pk = oracle.forward(k, d["gamma_k"], w.eps, K)
    wq, wk = w.hq // K, w.hk // K
    shards = [(gpu(q[:, r * wq:(r + 1) * wq]), gpu(k[:, r * wk:(r + 1) * wk])) for r in range(K)]
    gq, gk = gpu(d["gamma_q"]), gpu(d["gamma_k"])
    sq = torch.zeros((K, T), dtype=torch.float32, device=DEV)
    sk = torch.zeros((K, T), dtype=torch.float32, device=DEV)
    say("split qk partials", name, "T=%d K=%d shards %d/%d" % (T, K, wq, wk))
    for r, (xq, xk) in enumerate(shards):
        qk.partial_stats_qk(xq, xk, r, K, sq, sk)
    torch.cuda.synchronize()
    np.testing.assert_allclose(sq.cpu().numpy(), Pq, rtol=1e-5)
    np.testing.assert_allclose(sk.cpu().numpy(), Pk, rtol=1e-5)
    say("split qk apply", name)
    outs = []
    for r, (xq, xk) in enumerate(shards):
        yq, yk = qk.apply_stats_qk(xq, xk, gq[r * wq:(r + 1) * wq], gk[r * wk:(r + 1) * wk], sq, sk,
                                   w.hq, w.hk, eps=w.eps)
        outs.append((yq, yk))
    torch.cuda.synchronize()
    assert_parity(torch.cat([o[0] for o in outs], 1), refq, w.torch_dtype, "split qk q")
    assert_parity(torch.cat([o[1] for o in outs], 1), refk, w.torch_dtype, "split qk k")
    # the single-tensor calls on strided views of the full rows give the same bits
    say("split qk vs single-tensor calls on views", name)
    qd, kd = gpu(q), gpu(k)
    st1 = torch.zeros((K, T), dtype=torch.float32, device=DEV)
    for r in range(K):
        qk.partial_stats(qd[:, r * wq:(r + 1) * wq], r, K, st1)
    y1 = qk.apply_stats(qd[:, wq:2 * wq], gq[wq:2 * wq], st1, w.hq, eps=w.eps)
    torch.cuda.synchronize()
    assert torch.equal(st1, sq)
    assert torch.equal(y1, outs[1][0])
    # in place on the shards, query slice alone (k_slice None)
    xq = shards[0][0]
    qk.apply_stats_qk(xq, None, gq[:wq], None, sq, None, w.hq, 0, eps=w.eps, out_q=xq)
    torch.cuda.synchronize()
    assert torch.equal(xq, outs[0][0])


def test_denormal_squares_of_bf16_rows():
    """bf16 rows whose squares are denormal fp32 values: entries m * 2^-70
    with |m| <= 3 (exact in bf16), squares m^2 * 2^-140 (exact fp32
    denormals), row sums below 2^-126, and means (a multiple of 2^-149 for
    these widths) that are exact fp32 denormals too. The bf16 squares go
    through the bf16 dot-product instruction; a flush of denormal products
    or sums would leave S = 0 and, with eps = 0, infinite outputs, where the
    fp64 oracle is finite (review "Prerequisites", Eq. 1). Checked with
    eps = 0 and a denormal eps = 2^-130, for the fused forward (1 and 4
    slices), the split path, the inverse RMS and the headwise form."""
    T, H, D = 40, 512, 128
    rng = np.random.default_rng(101)
    m = rng.integers(-3, 4, size=(T, H)).astype(np.float32)
    m[:, 0] = 3.0  # no row is all zero
    x = torch.from_numpy(m * np.float32(2.0 ** -70)).to(torch.bfloat16)
    assert torch.equal(x.float(), torch.from_numpy(m * np.float32(2.0 ** -70)))
    g = workloads.random_weights(H, "bf16", 102)
    xd, gd = gpu(x), gpu(g)
    for eps in (0.0, 2.0 ** -130):
        for K in (1, 4):
            say("denormal squares bf16 forward eps=%g K=%d" % (eps, K))
            y, _ = qk.forward(xd, None, gd, None, eps=eps, num_slices=K)
            torch.cuda.synchronize()
            ref, P = oracle.forward(x, g, eps, K)
            assert (P.sum(axis=0) < 2.0 ** -126).all(), "the case must reach denormal sums"
            assert_parity(y, ref, torch.bfloat16, "denormal squares forward K=%d eps=%g" % (K, eps))
        say("denormal squares bf16 split eps=%g" % eps)
        K, wd = 4, H // 4
        st = torch.zeros((K, T), dtype=torch.float32, device=DEV)
        for s_ in range(K):
            qk.partial_stats(xd[:, s_ * wd:(s_ + 1) * wd], s_, K, st)
        ys = torch.empty_like(xd)
        for s_ in range(K):
            qk.apply_stats(xd[:, s_ * wd:(s_ + 1) * wd], gd[s_ * wd:(s_ + 1) * wd], st, H, eps,
                           out=ys[:, s_ * wd:(s_ + 1) * wd])
        torch.cuda.synchronize()
        ref, P = oracle.forward(x, g, eps, K)
        np.testing.assert_allclose(st.cpu().double().numpy(), P, rtol=1e-6)
        assert_parity(ys, ref, torch.bfloat16, "denormal squares split eps=%g" % eps)
        say("denormal squares bf16 inverse RMS and headwise eps=%g" % eps)
        r, _ = qk.inv_rms(xd, eps=eps, num_slices=4)
        yh, _ = qk.forward_headwise(xd, None, gd[:D], None, D, eps=eps)
        torch.cuda.synchronize()
        assert_parity(r, oracle.inv_rms(x, eps, 4), torch.float32, "denormal squares rinv eps=%g" % eps)
        assert_parity(yh, oracle.headwise(x, g[:D], D, eps), torch.bfloat16, "denormal squares headwise")


def test_denormal_statistics():
    """Rows whose mean of squares is a denormal fp32 value: three entries of
    +-2^-60 in 256 columns (squares 2^-120, normal and exact) and eps = 2^-130,
    so mean + eps = 13 * 2^-130 exactly. The inverse RMS must still be the
    finite one (the hardware reciprocal square root alone would give
    infinity), for the statistic alone, the layerwise and the headwise form
    (whose empty heads have mean + eps = 2^-130)."""
    T, H, D = 6, 256, 64
    rng = np.random.default_rng(99)
    x = np.zeros((T, H), np.float32)
    for t in range(T):
        cols = rng.choice(H, 3, replace=False)
        x[t, cols] = np.float32(2.0 ** -60) * rng.choice([-1.0, 1.0], 3).astype(np.float32)
    x = torch.from_numpy(x)
    eps = 2.0 ** -130
    g = workloads.random_weights(H, "f32", 100)
    xd = gpu(x)
    say("denormal statistics")
    r, _ = qk.inv_rms(xd, eps=eps)
    y, _ = qk.forward(xd, None, gpu(g), None, eps=eps)
    yh, _ = qk.forward_headwise(xd, None, gpu(g[:D]), None, D, eps=eps)
    torch.cuda.synchronize()
    ref = oracle.inv_rms(x, eps, 1)
    assert (1.0 / (ref * ref) < 2.0 ** -126).all(), "the case must reach denormal means"
    assert_parity(r, ref, torch.float32, "rinv")
    assert_parity(y, oracle.forward(x, g, eps, 1)[0], torch.float32, "forward")
    assert_parity(yh, oracle.headwise(x, g[:D], D, eps), torch.float32, "headwise")


@pytest.mark.parametrize("opts", [dict(max_workgroups=3), dict(max_workgroups=1, waves_per_row=2),
                                  dict(max_workgroups=5, waves_per_row=16)],
                         ids=lambda o: ",".join("%s=%s" % kv for kv in o.items()))
def test_capped_grids_statistics_and_split_path(opts):
    """Grids capped below the row count: the statistic-only, partial-sum and
    apply launches loop over their rows (grid stride) and reproduce, bit for
    bit, the same layout's results on a full grid (a different team size
    would add the squares in another order); both match the oracle."""
    ctx = qk.Context(0, **opts)
    full = qk.Context(0, waves_per_row=opts.get("waves_per_row", 0))
    T, Hq, Hk, K = 300, 4096, 1024, 4
    q = workloads.random_rows(T, Hq, "bf16", [61, T], dist="laplace")
    k = workloads.random_rows(T, Hk, "bf16", [62, T])
    qd, kd = gpu(q), gpu(k)
    say("capped inv_rms", opts)
    a_q, a_k = qk.inv_rms(qd, kd, eps=1e-6, num_slices=K, ctx=full)
    b_q, b_k = qk.inv_rms(qd, kd, eps=1e-6, num_slices=K, ctx=ctx)
    torch.cuda.synchronize()
    assert torch.equal(a_q, b_q) and torch.equal(a_k, b_k)
    for r, x, which in ((b_q, q, "q"), (b_k, k, "k")):
        assert_parity(r, oracle.inv_rms(x, 1e-6, K), torch.float32, "capped rinv " + which)
    w = Hq // K
    P = oracle.slice_sumsq(q, K)
    stats = {}
    for name, c in (("default", full), ("capped", ctx)):
        st = torch.zeros((K, T), dtype=torch.float32, device=DEV)
        say("capped partial_stats", name, opts)
        for s in range(K):
            qk.partial_stats(qd[:, s * w:(s + 1) * w], s, K, st, ctx=c)
        torch.cuda.synchronize()
        stats[name] = st
    assert torch.equal(stats["default"], stats["capped"])
    np.testing.assert_allclose(stats["capped"].cpu().double().numpy(), P, rtol=2e-6)
    g = gpu(workloads.random_weights(Hq, "bf16", 63))
    for s in (0, K - 1):
        say("capped apply_stats", s, opts)
        ya = qk.apply_stats(qd[:, s * w:(s + 1) * w], g[s * w:(s + 1) * w], stats["default"], Hq, eps=1e-6,
                            ctx=full)
        yb = qk.apply_stats(qd[:, s * w:(s + 1) * w], g[s * w:(s + 1) * w], stats["default"], Hq, eps=1e-6,
                            ctx=ctx)
        torch.cuda.synchronize()
        assert torch.equal(ya.view(torch.int16), yb.view(torch.int16))


def test_rows_beyond_the_grid_limit():
    """More workgroups than one launch holds (2^32 - 1 work-items along x):
    2^28 + 4096 one-vector bf16 rows (4.3 GB). The statistic-only launch (16
    rows per workgroup) and the in-place forward (4) cover the rows past the
    first grid with their grid-stride loops; sampled rows (the first, random
    ones, and the last, which only the loop reaches) match the oracle."""
    T, H = (1 << 28) + 4096, 8
    say("rows beyond the grid limit: T=%d, width %d" % (T, H))
    x = workloads.device_rows(T, H, "bf16", 71, DEV)
    g = gpu(workloads.random_weights(H, "bf16", 72))
    r, _ = qk.inv_rms(x, None, eps=1e-6)
    rng = np.random.default_rng(73)
    idx = torch.from_numpy(np.concatenate([np.arange(1000), rng.integers(0, T, 2000),
                                           np.arange(T - 5000, T)])).to(DEV)
    xs = x.index_select(0, idx).cpu()
    rs = r.index_select(0, idx).cpu()
    say("rows beyond the grid limit: forward in place")
    qk.forward(x, None, g, None, eps=1e-6, out_q=x)
    torch.cuda.synchronize()
    ys = x.index_select(0, idx).cpu()
    del x, r
    assert_parity(rs, oracle.inv_rms(xs, 1e-6, 1), torch.float32, "rinv")
    assert_parity(ys, oracle.forward(xs, g.cpu(), 1e-6, 1)[0], torch.bfloat16, "y")
