"""Packed rows on the GPU: launches over many rows of at most 32 vectors (512
bytes), which put several rows in each slot of a wavefront, against the fp64
oracle, and bit for bit against the same calls with packing turned off (a
forced team of one wavefront keeps the one-row layout and its arithmetic).
Covered: the fused forward (both tensors, one tensor, in place, strided
inputs and outputs of different strides), the split path's statistics and
apply steps on a rank's shards, the inverse RMS, and FP8 rows that saturate
and are encoded again from the input with the clamp. Every case prints what
it runs before the GPU call."""
import os

import numpy as np
import pytest
import torch

import attention_qk_norm_amd as qk
import oracle
from attention_qk_norm_amd import workloads
from gpu_checks import assert_parity

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


def unpacked():
    return qk.Context(0, waves_per_row=1)


def bits(t):
    return t.contiguous().view(torch.uint8).cpu() if t.dtype == FP8 else t.cpu()


def gamma_dtype(dtype):
    return "bf16" if dtype == "fp8" else dtype


FORWARD = [
    # dtype, T, Hq, Hk (0: one tensor), layout; T * tensors >= 16 * 1024 rows,
    # so these launches pack (vectors per row in the comments)
    ("fp8", 16384, 512, 512, "plain"),       # C5-fp8's rank shards: 32 and 32, two rows per slot
    ("fp8", 16381, 320, 128, "plain"),       # 20 and 8: groups of 32 and 8 lanes; T ragged
    ("fp8", 9000, 16, 48, "in_place"),       # 1 and 3: 64 and 16 rows per slot
    ("bf16", 8200, 256, 64, "plain"),        # 32 and 8
    ("bf16", 10000, 200, 24, "views"),       # 25 and 3, column blocks of one buffer, in place
    ("bf16", 16384, 240, 0, "plain"),        # one tensor of 30
    ("f32", 8192, 128, 100, "out_views"),    # 32 and 25, outputs strided unlike the inputs
    ("f32", 20000, 4, 8, "plain"),           # 1 and 2
]


@pytest.mark.parametrize("dtype,T,Hq,Hk,layout", FORWARD)
def test_packed_forward(dtype, T, Hq, Hk, layout):
    q = workloads.random_rows(T, Hq, dtype, [T, Hq, 21], dist="laplace")
    k = workloads.random_rows(T, Hk, dtype, [T, Hk, 22]) if Hk else None
    gq = workloads.random_weights(Hq, gamma_dtype(dtype), [Hq, 23])
    gk = workloads.random_weights(Hk, gamma_dtype(dtype), [Hk, 24]) if Hk else None
    refq, _ = oracle.forward(q, gq, 1e-6, 1)
    refk = oracle.forward(k, gk, 1e-6, 1)[0] if Hk else None
    outs = []
    for ctx in (None, unpacked()):
        say("packed forward", dtype, T, Hq, Hk, layout, "packing" if ctx is None else "one row per slot")
        if layout == "views":
            pad = 64
            buf = torch.zeros((T, Hq + Hk + pad), dtype=q.dtype)
            buf[:, :Hq] = q
            buf[:, Hq:Hq + Hk] = k
            buf[:, Hq + Hk:] = 3.0
            bd = gpu(buf)
            qv, kv = bd[:, :Hq], bd[:, Hq:Hq + Hk]
            qk.forward(qv, kv, gpu(gq), gpu(gk), eps=1e-6, out_q=qv, out_k=kv, ctx=ctx)
            torch.cuda.synchronize()
            assert torch.equal(bits(bd[:, Hq + Hk:]), bits(buf[:, Hq + Hk:]))  # the other columns are untouched
            yq, yk = qv, kv
        elif layout == "out_views":
            ob = torch.full((T, Hq + Hk + 32), 5.0, dtype=q.dtype, device=DEV)
            oq, ok = ob[:, :Hq], ob[:, Hq:Hq + Hk]
            qk.forward(gpu(q), gpu(k), gpu(gq), gpu(gk), eps=1e-6, out_q=oq, out_k=ok, ctx=ctx)
            torch.cuda.synchronize()
            assert (ob[:, Hq + Hk:] == 5.0).all()
            yq, yk = oq, ok
        else:
            dq = gpu(q)
            dk = gpu(k) if Hk else None
            in_place = layout == "in_place"
            yq, yk = qk.forward(dq, dk, gpu(gq), gpu(gk) if Hk else None, eps=1e-6, ctx=ctx,
                                out_q=dq if in_place else None, out_k=dk if in_place else None)
            torch.cuda.synchronize()
        outs.append((yq, yk))
    (yq, yk), (yq1, yk1) = outs
    assert torch.equal(bits(yq), bits(yq1))
    assert_parity(yq, refq, q.dtype, "q")
    if Hk:
        assert torch.equal(bits(yk), bits(yk1))
        assert_parity(yk, refk, q.dtype, "k")


def test_packed_fp8_saturating_in_place():
    """FP8 rows whose results pass 448 (weights of +-(200..600)), with a NaN
    row and a zero row, in place: the saturating vectors are encoded again
    from the input with the clamp, as in the one-row layout."""
    T, Hq, Hk = 16384, 512, 256
    q = workloads.random_rows(T, Hq, "fp8", [T, 31], dist="laplace").float()
    k = workloads.random_rows(T, Hk, "fp8", [T, 32]).float()
    q[5, 100] = float("nan")
    q[6] = 0.0
    q, k = q.to(FP8), k.to(FP8)
    gq = workloads.random_weights(Hq, "bf16", 33, 200.0, 600.0).float()
    gq[::3] = -gq[::3]
    gq = gq.to(torch.bfloat16)
    gk = workloads.random_weights(Hk, "bf16", 34, 200.0, 600.0)
    keep = [t for t in range(T) if t != 5]
    rq, _ = oracle.forward(q[keep], gq, 1e-6, 1)
    rk, _ = oracle.forward(k, gk, 1e-6, 1)
    assert (np.abs(rq) >= 464).mean() > 0.05 and (np.abs(rk) >= 464).mean() > 0.05
    outs = []
    for ctx in (None, unpacked()):
        say("packed fp8 saturating", T, Hq, Hk, "packing" if ctx is None else "one row per slot")
        dq, dk = gpu(q), gpu(k)
        qk.forward(dq, dk, gpu(gq), gpu(gk), eps=1e-6, out_q=dq, out_k=dk, ctx=ctx)
        torch.cuda.synchronize()
        outs.append((dq, dk))
    (yq, yk), (yq1, yk1) = outs
    assert torch.equal(bits(yq), bits(yq1)) and torch.equal(bits(yk), bits(yk1))
    hq = yq.cpu().float()
    assert torch.isnan(hq[5]).all() and (hq[6] == 0).all()
    assert_parity(yq[keep], rq, FP8, "q")
    assert_parity(yk, rk, FP8, "k")


SPLIT = [
    # dtype, T, Hq, Hk, K: each rank's shards are [T, H / K] (vectors per row)
    ("fp8", 16384, 4096, 4096, 8),   # C5-fp8 on 8 ranks: 32 and 32
    ("fp8", 10001, 2560, 1024, 8),   # 20 and 8
    ("bf16", 12000, 2048, 512, 8),   # 32 and 8
    ("f32", 9000, 1024, 256, 8),     # 32 and 8
    ("bf16", 16384, 128, 64, 8),     # 2 and 1: the apply step's groups widen to 8 lanes, one per partial
    ("f32", 9000, 2048, 256, 64),    # 8 and 1, 64 partials: the apply step keeps one row per slot
]


@pytest.mark.parametrize("dtype,T,Hq,Hk,K", SPLIT)
def test_packed_split_path_on_rank_shards(dtype, T, Hq, Hk, K):
    """Every rank's statistics launch on its own contiguous shards, then the
    apply step of some ranks with all K partials: the oracle's partials and
    rows, and the bits of the same calls unpacked."""
    q = workloads.random_rows(T, Hq, dtype, [T, Hq, 41], dist="laplace")
    k = workloads.random_rows(T, Hk, dtype, [T, Hk, 42])
    gq = workloads.random_weights(Hq, gamma_dtype(dtype), [Hq, 43])
    gk = workloads.random_weights(Hk, gamma_dtype(dtype), [Hk, 44])
    refq, Pq = oracle.forward(q, gq, 1e-6, K)
    refk, Pk = oracle.forward(k, gk, 1e-6, K)
    wq, wk = Hq // K, Hk // K
    shards = [(gpu(q[:, r * wq:(r + 1) * wq]), gpu(k[:, r * wk:(r + 1) * wk])) for r in range(K)]
    dgq, dgk = gpu(gq), gpu(gk)
    res = []
    for ctx in (None, unpacked()):
        how = "packing" if ctx is None else "one row per slot"
        sq = torch.zeros((K, T), dtype=torch.float32, device=DEV)
        sk = torch.zeros((K, T), dtype=torch.float32, device=DEV)
        say("packed split partials", dtype, T, Hq, Hk, K, how)
        for r, (xq, xk) in enumerate(shards):
            qk.partial_stats_qk(xq, xk, r, K, sq, sk, ctx=ctx)
        torch.cuda.synchronize()
        ys = []
        for r in (0, 3, K - 1):
            say("packed split apply", dtype, T, Hq, Hk, K, "rank", r, how)
            xq, xk = shards[r]
            ys.append(qk.apply_stats_qk(xq, xk, dgq[r * wq:(r + 1) * wq], dgk[r * wk:(r + 1) * wk], sq, sk, Hq, Hk,
                                        eps=1e-6, ctx=ctx))
        torch.cuda.synchronize()
        res.append((sq, sk, ys))
    (sq, sk, ys), (sq1, sk1, ys1) = res
    assert torch.equal(sq, sq1) and torch.equal(sk, sk1)
    np.testing.assert_allclose(sq.cpu().numpy(), Pq, rtol=1e-5)
    np.testing.assert_allclose(sk.cpu().numpy(), Pk, rtol=1e-5)
    for (yq, yk), (yq1, yk1), r in zip(ys, ys1, (0, 3, K - 1)):
        assert torch.equal(bits(yq), bits(yq1)) and torch.equal(bits(yk), bits(yk1))
        assert_parity(yq, refq[:, r * wq:(r + 1) * wq], q.dtype, "q rank %d" % r)
        assert_parity(yk, refk[:, r * wk:(r + 1) * wk], q.dtype, "k rank %d" % r)


@pytest.mark.parametrize("dtype", ["fp8", "bf16", "f32"])
def test_packed_inv_rms(dtype):
    """The statistic-only output of narrow rows (30 and 4 vectors), packed:
    the oracle's inverse RMS, and the unpacked launch's bits."""
    T = 12345
    ve = {"fp8": 16, "bf16": 8, "f32": 4}[dtype]
    Hq, Hk = 30 * ve, 4 * ve
    q = workloads.random_rows(T, Hq, dtype, [T, 51], dist="laplace")
    k = workloads.random_rows(T, Hk, dtype, [T, 52])
    outs = []
    for ctx in (None, unpacked()):
        say("packed inv_rms", dtype, T, Hq, Hk, "packing" if ctx is None else "one row per slot")
        outs.append(qk.inv_rms(gpu(q), gpu(k), eps=1e-6, ctx=ctx))
        torch.cuda.synchronize()
    (rq, rk), (rq1, rk1) = outs
    assert torch.equal(rq, rq1) and torch.equal(rk, rk1)
    np.testing.assert_allclose(rq.cpu().double().numpy(), oracle.inv_rms(q, 1e-6), rtol=2e-6)
    np.testing.assert_allclose(rk.cpu().double().numpy(), oracle.inv_rms(k, 1e-6), rtol=2e-6)
