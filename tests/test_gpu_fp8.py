"""FP8 E4M3 rows on the GPU against the fp64 oracle (through the C ABI).

The rows are OCP e4m3 (torch.float8_e4m3fn) in and out, the weights bf16;
squares accumulate in fp32 (SwiftQK review section 5 and Fig. 2(b)'s FP8
runs). The bar: within one e4m3 ulp of the fp64 result saturated at +-448,
and exactly +-448 past the rounding boundary. Every case prints what it runs
before the GPU call.
"""
import os

import numpy as np
import pytest
import torch

import attention_qk_norm_amd as qk
import oracle
from attention_qk_norm_amd import workloads
from gpu_checks import assert_near_each_other, assert_parity

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
FP8 = torch.float8_e4m3fn


def say(*a):
    print("[case]", *a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _oracle_threads():
    oracle.set_threads(min(16, os.cpu_count() or 1))
    yield
    oracle.set_threads(1)


def gpu(t):
    return t.to(DEV).contiguous()


def rows(T, H, seed, dist="normal", scale=1.0):
    return workloads.random_rows(T, H, "fp8", seed, dist=dist, scale=scale)


def weights(H, seed, lo=0.5, hi=1.5):
    return workloads.random_weights(H, "bf16", seed, lo, hi)


@pytest.mark.parametrize("name", ["c4f8", "c5f8"])
def test_fp8_workloads(name):
    d = workloads.generate(name)
    w = d["w"]
    outs = {}
    for K in w.slices:
        say(name, "T=%d Hq=%d Hk=%d fp8 K=%d in_place=%s" % (w.T, w.hq, w.hk, K, w.in_place))
        q, k = gpu(d["q"]), gpu(d["k"])
        yq, yk = qk.forward(q, k, gpu(d["gamma_q"]), gpu(d["gamma_k"]), eps=w.eps, num_slices=K,
                            out_q=q if w.in_place else None, out_k=k if w.in_place else None)
        torch.cuda.synchronize()
        rq, _ = oracle.forward(d["q"], d["gamma_q"], w.eps, K)
        rk, _ = oracle.forward(d["k"], d["gamma_k"], w.eps, K)
        print("  q errors", assert_parity(yq, rq, FP8, "%s q K=%d" % (name, K)), flush=True)
        print("  k errors", assert_parity(yk, rk, FP8, "%s k K=%d" % (name, K)), flush=True)
        outs[K] = (yq.cpu(), yk.cpu())
        del q, k, yq, yk
    if len(outs) > 1:
        (a_q, a_k), (b_q, b_k) = list(outs.values())[:2]
        for a, b in ((a_q, b_q), (a_k, b_k)):
            assert_near_each_other(a, b, FP8, name + " K vs 1")


SHAPES = [
    # T, Hq, Hk, K: one-vector rows, ragged slots, slices, narrow slices in
    # the masked layout, the widest rows
    (5, 16, 16, 1),
    (33, 1024, 128, 1),
    (70, 4096, 1024, 8),
    (17, 5120, 1024, 4),
    (3, 4096, 4096, 64),       # slices of 64: 4 vectors each
    (9, 3072, 1536, 48),       # slices of 64 and 32 elements: masked layout
    (2, 65536, 16, 1),         # widest fp8 row
    (3000, 512, 128, 2),       # many rows per SIMD
    (2001, 5120, 1024, 1),     # one round of wavefronts, 2 rows each; ragged T
    # FP8 bodies of odd slot counts: 3 slots (2 rows per wavefront); 7 slots
    # with a 2-slot key segment (its 3-slot body keeps one slot empty); 5 and
    # 3 slots over several rounds, sliced; 7 slots over several rounds; 7
    # slots with widened teams
    (1500, 3072, 1024, 1),
    (1100, 7168, 2048, 1),
    (9000, 5120, 3072, 8),
    (12000, 7168, 1024, 1),
    (40, 7168, 7168, 7),
    # narrow slices in a single round of one-wavefront rows: 8-lane sub-teams
    # (C4's widths, K = 8); 4- and 1-lane sub-teams; 1-lane sub-teams, 64
    # slices
    (2048, 5120, 1024, 8),
    (2001, 3072, 1536, 48),
    (2047, 4096, 4096, 64),
    (5000, 4096, 4096, 64),    # several rounds, 4-lane sub-teams taking 4 slices in turn
    # grouped-query rows: 2-wavefront query teams sharing a narrow-slice launch
    # with 8-lane key sub-teams, over several rounds; 16-wavefront query teams
    # beside 2-wavefront key teams
    (3000, 16384, 2048, 8),
    (7300, 16384, 2048, 8),    # past 2^23 vectors: one launch per tensor
    (600, 65536, 8192, 1),
]


@pytest.mark.parametrize("T,Hq,Hk,K", SHAPES)
def test_fp8_shapes(T, Hq, Hk, K):
    q = rows(T, Hq, [T, Hq, 1], dist="laplace")
    k = rows(T, Hk, [T, Hk, 2], scale=3.0)
    gq, gk = weights(Hq, [Hq, 3]), weights(Hk, [Hk, 4])
    say("fp8", T, Hq, Hk, K)
    yq, yk = qk.forward(gpu(q), gpu(k), gpu(gq), gpu(gk), eps=1e-6, num_slices=K)
    torch.cuda.synchronize()
    assert_parity(yq, oracle.forward(q, gq, 1e-6, K)[0], FP8, "q")
    assert_parity(yk, oracle.forward(k, gk, 1e-6, K)[0], FP8, "k")


def test_fp8_saturation_and_nan():
    """Large weights push |y| past 448: those outputs are exactly +-448, not
    NaN; a row holding a NaN comes out NaN; a zero row comes out zero."""
    T, H = 6, 4096
    x = rows(T, H, 5, dist="laplace").float()
    # one dominant element makes |x r| approach sqrt(H) = 64 there
    x[0, 7] = 400.0
    x[3, 2000] = -448.0
    x[1] = 0.0
    x[2, 100] = float("nan")
    x = x.to(FP8)
    g = weights(H, 6, 12.0, 16.0)
    say("fp8 saturation")
    y, _ = qk.forward(gpu(x), None, gpu(g), None, eps=1e-6)
    torch.cuda.synchronize()
    yh = y.cpu().float()
    assert torch.isnan(yh[2]).all()
    assert (yh[1] == 0).all()
    keep = [0, 3, 4, 5]
    ref, _ = oracle.forward(x[keep], g, 1e-6, 1)
    assert (np.abs(ref) >= 464).sum() > 0, "the case must reach saturation"
    assert_parity(y[keep], ref, FP8, "saturating rows")


def test_fp8_split_path():
    T, H, K = 100, 5120, 4
    x = rows(T, H, 7)
    g = weights(H, 8)
    ref, _ = oracle.forward(x, g, 1e-6, K)
    xd = gpu(x)
    w = H // K
    stats = torch.zeros((K, T), dtype=torch.float32, device=DEV)
    say("fp8 split path")
    for s in range(K):
        qk.partial_stats(xd[:, s * w:(s + 1) * w], s, K, stats)
    torch.cuda.synchronize()
    P = oracle.slice_sumsq(x, K)
    np.testing.assert_allclose(stats.cpu().double().numpy(), P, rtol=2e-6)
    gd = gpu(g)
    for s in range(K):
        ys = qk.apply_stats(xd[:, s * w:(s + 1) * w], gd[s * w:(s + 1) * w], stats, H, eps=1e-6)
        torch.cuda.synchronize()
        assert_parity(ys, ref[:, s * w:(s + 1) * w], FP8, "slice %d" % s)


@pytest.mark.parametrize("T,Hq,Hk,D", [(37, 4096, 1024, 128), (9, 2048, 512, 16), (5, 8192, 2048, 1024),
                                      (3000, 1024, 256, 64)])
def test_fp8_headwise(T, Hq, Hk, D):
    q = rows(T, Hq, [T, D, 9], dist="laplace")
    q = (q.float() * torch.linspace(0.05, 8.0, Hq // D).repeat_interleave(D)).to(FP8)
    k = rows(T, Hk, [T, D, 10])
    gq, gk = weights(D, [D, 11]), weights(D, [D, 12])
    say("fp8 headwise", T, Hq, Hk, D)
    yq, yk = qk.forward_headwise(gpu(q), gpu(k), gpu(gq), gpu(gk), D, eps=1e-6)
    torch.cuda.synchronize()
    rq, rk = oracle.qk_headwise(q, k, gq, gk, D, 1e-6)
    assert_parity(yq, rq, FP8, "q")
    assert_parity(yk, rk, FP8, "k")


def test_fp8_inv_rms_is_the_forward_factor():
    T, Hq, Hk, K = 300, 4096, 1024, 8
    q, k = rows(T, Hq, 13, dist="laplace"), rows(T, Hk, 14)
    gq, gk = weights(Hq, 15), weights(Hk, 16)
    say("fp8 inv_rms")
    rq, rk = qk.inv_rms(gpu(q), gpu(k), eps=1e-6, num_slices=K)
    yq, yk = qk.forward(gpu(q), gpu(k), gpu(gq), gpu(gk), eps=1e-6, num_slices=K)
    torch.cuda.synchronize()
    for r, x, g, y in ((rq, q, gq, yq), (rk, k, gk, yk)):
        assert_parity(r, oracle.inv_rms(x, 1e-6, K), torch.float32, "rinv")
        # FP8 rows scale as (x gamma) r: x gamma is exact in fp32, so one rounding
        want = ((x.float() * g.float()) * r.cpu()[:, None]).clamp(-448.0, 448.0).to(FP8)
        assert torch.equal(y.cpu().view(torch.uint8), want.view(torch.uint8))


@pytest.mark.parametrize("opts", [dict(waves_per_row=1), dict(waves_per_row=4), dict(waves_per_row=16),
                                  dict(max_workgroups=7), dict(max_workgroups=3, waves_per_row=2),
                                  dict(cached_rows=1)],
                         ids=lambda o: ",".join("%s=%s" % kv for kv in o.items()))
def test_fp8_schedules(opts):
    ctx = qk.Context(0, **opts)
    T, Hq, Hk, K = 131, 5120, 1024, 4
    q, k = rows(T, Hq, [21, T]), rows(T, Hk, [22, T])
    gq, gk = weights(Hq, 23), weights(Hk, 24)
    say("fp8 schedule", opts)
    try:
        yq, yk = qk.forward(gpu(q), gpu(k), gpu(gq), gpu(gk), eps=1e-6, num_slices=K, ctx=ctx)
    except qk.QKNormError as e:
        assert e.status == qk.ERR_SHAPE and "waves_per_row" in opts
        return
    torch.cuda.synchronize()
    assert_parity(yq, oracle.forward(q, gq, 1e-6, K)[0], FP8, "q")
    assert_parity(yk, oracle.forward(k, gk, 1e-6, K)[0], FP8, "k")


@pytest.mark.parametrize("in_place", [False, True], ids=["out", "in_place"])
@pytest.mark.parametrize("K", [1, 4])
@pytest.mark.parametrize("opts", [dict(), dict(max_workgroups=5), dict(waves_per_row=2)],
                         ids=lambda o: ",".join("%s=%s" % kv for kv in o.items()) or "auto")
def test_fp8_dense_saturation(in_place, K, opts):
    """Weights of +-(200..600) saturate a large share of every row, in many
    lanes and every slot at once: each such vector is encoded a second time
    with the clamp from the input, which in place must still be unwritten.
    T = 300 rows of q and k is one round of wavefronts (two rows each, with
    the automatic schedule); a NaN row stays NaN, a zero row zero."""
    ctx = qk.Context(0, **opts)
    T, Hq, Hk = 300, 5120, 1024
    q = rows(T, Hq, [51, K], dist="laplace").float()
    k = rows(T, Hk, [52, K]).float()
    q[5, 333] = float("nan")
    q[6] = 0.0
    k[7, 1000] = float("nan")
    q, k = q.to(FP8), k.to(FP8)
    gq, gk = weights(Hq, 53, 200.0, 600.0).float(), weights(Hk, 54, 200.0, 600.0).float()
    gq[::3] = -gq[::3]
    gk[1::2] = -gk[1::2]
    gq, gk = gq.to(torch.bfloat16), gk.to(torch.bfloat16)
    keep_q = [t for t in range(T) if t != 5]
    keep_k = [t for t in range(T) if t != 7]
    rq, _ = oracle.forward(q[keep_q], gq, 1e-6, K)
    rk, _ = oracle.forward(k[keep_k], gk, 1e-6, K)
    assert (np.abs(rq) >= 464).mean() > 0.05 and (np.abs(rk) >= 464).mean() > 0.05
    dq, dk = gpu(q), gpu(k)
    say("fp8 dense saturation", opts, "K=%d" % K, "in_place" if in_place else "out of place")
    yq, yk = qk.forward(dq, dk, gpu(gq), gpu(gk), eps=1e-6, num_slices=K, ctx=ctx,
                        out_q=dq if in_place else None, out_k=dk if in_place else None)
    torch.cuda.synchronize()
    hq, hk = yq.cpu().float(), yk.cpu().float()
    assert torch.isnan(hq[5]).all() and torch.isnan(hk[7]).all()
    assert (hq[6] == 0).all()
    assert_parity(yq[keep_q], rq, FP8, "q")
    assert_parity(yk[keep_k], rk, FP8, "k")


@pytest.mark.parametrize("T,Hq,Hk,case", [
    (2048, 5120, 1024, "plain"),        # C4-fp8's shape
    (3001, 1024, 4096, "in_place"),     # key rows wider (the segments swap), T not a multiple of 4
    (2048, 4096, 4096, "plain"),
    (2560, 5120, 1024, "saturating"),   # weights of +-(200..600), a NaN and a zero row, in place
    (2048, 5120, 1024, "saturating"),   # the same with the products formed before the statistic
    (2048, 6144, 6144, "plain"),        # 6 + 6 slots: the widest pair with early products
    (2048, 7168, 7168, "plain"),        # 7 + 7 slots: scaled after the statistic
])
def test_fp8_paired_rows(T, Hq, Hk, case):
    """FP8 forward launches of 2 to 4 paired wavefronts per SIMD (each
    wavefront takes one token's query and key row; at 2 per SIMD the kernel
    forms the products x gamma before the statistic): parity, and bit
    equality with the same launch unpaired (a forced team of one wavefront),
    also when rows saturate and are encoded again with the clamp."""
    q = rows(T, Hq, [61, T], dist="laplace")
    k = rows(T, Hk, [62, T])
    gq, gk = weights(Hq, 63), weights(Hk, 64)
    keep = list(range(T))
    if case == "saturating":
        q, k = q.float(), k.float()
        q[5, 333] = float("nan")
        q[6] = 0.0
        q, k = q.to(FP8), k.to(FP8)
        gq, gk = weights(Hq, 65, 200.0, 600.0).float(), weights(Hk, 66, 200.0, 600.0).float()
        gq[::3] = -gq[::3]
        gq, gk = gq.to(torch.bfloat16), gk.to(torch.bfloat16)
        keep = [t for t in range(T) if t != 5]
    rq, _ = oracle.forward(q[keep], gq, 1e-6, 1)
    rk, _ = oracle.forward(k, gk, 1e-6, 1)
    if case == "saturating":
        assert (np.abs(rq) >= 464).mean() > 0.05 and (np.abs(rk) >= 464).mean() > 0.05
    say("fp8 paired rows", T, Hq, Hk, case)
    outs = []
    for ctx in (None, qk.Context(0, waves_per_row=1)):
        dq, dk = gpu(q), gpu(k)
        in_place = case != "plain"
        yq, yk = qk.forward(dq, dk, gpu(gq), gpu(gk), eps=1e-6, ctx=ctx,
                            out_q=dq if in_place else None, out_k=dk if in_place else None)
        torch.cuda.synchronize()
        outs.append((yq.view(torch.uint8).cpu(), yk.view(torch.uint8).cpu(), yq, yk))
    (bq, bk, yq, yk), (bq1, bk1, _, _) = outs
    assert torch.equal(bq, bq1) and torch.equal(bk, bk1)
    if case == "saturating":
        hq = yq.cpu().float()
        assert torch.isnan(hq[5]).all() and (hq[6] == 0).all()
    assert_parity(yq[keep], rq, FP8, "q")
    assert_parity(yk, rk, FP8, "k")


def test_fp8_packed_qkv_in_place():
    T, Hq, Hk, Hv = 45, 2048, 512, 512
    H = Hq + Hk + Hv
    qkv = rows(T, H, 31)
    gq, gk = weights(Hq, 32), weights(Hk, 33)
    rq, _ = oracle.forward(qkv[:, :Hq], gq, 1e-6, 1)
    rk, _ = oracle.forward(qkv[:, Hq:Hq + Hk], gk, 1e-6, 1)
    dev = gpu(qkv)
    q, k = dev[:, :Hq], dev[:, Hq:Hq + Hk]
    say("fp8 packed qkv in place")
    qk.forward(q, k, gpu(gq), gpu(gk), eps=1e-6, out_q=q, out_k=k)
    torch.cuda.synchronize()
    out = dev.cpu()
    assert_parity(out[:, :Hq], rq, FP8, "q")
    assert_parity(out[:, Hq:Hq + Hk], rk, FP8, "k")
    assert torch.equal(out[:, Hq + Hk:].view(torch.uint8), qkv[:, Hq + Hk:].view(torch.uint8))


def test_fp8_saturation_headwise_and_split():
    """The headwise form (bound sqrt(head_dim) * max|gamma|) and the split
    path's apply step (partials from the caller: always clamped) saturate
    too."""
    T, H, D = 4, 1024, 128
    x = rows(T, H, 41, dist="laplace").float()
    x[0, 5] = 300.0      # dominates its head: |x r| near sqrt(128)
    x[2, 900] = -400.0
    x = x.to(FP8)
    gh = weights(D, 42, 48.0, 64.0)
    say("fp8 headwise saturation")
    y, _ = qk.forward_headwise(gpu(x), None, gpu(gh), None, D, eps=1e-6)
    torch.cuda.synchronize()
    ref = oracle.headwise(x, gh, D, 1e-6)
    assert (np.abs(ref) >= 464).sum() >= 2
    assert_parity(y, ref, FP8, "headwise saturation")
    g = weights(H, 43, 12.0, 16.0)
    xd = gpu(x)
    K, w = 2, H // 2
    stats = torch.zeros((K, T), dtype=torch.float32, device=DEV)
    say("fp8 split-path saturation")
    for s_ in range(K):
        qk.partial_stats(xd[:, s_ * w:(s_ + 1) * w], s_, K, stats)
    ref, _ = oracle.forward(x, g, 1e-6, K)
    assert (np.abs(ref) >= 464).sum() >= 1
    gd = gpu(g)
    for s_ in range(K):
        ys = qk.apply_stats(xd[:, s_ * w:(s_ + 1) * w], gd[s_ * w:(s_ + 1) * w], stats, H, eps=1e-6)
        torch.cuda.synchronize()
        assert_parity(ys, ref[:, s_ * w:(s_ + 1) * w], FP8, "slice %d" % s_)
