"""A seeded sweep of random shapes through every entry point, against the
fp64 oracle: element type, T, widths, padded row strides, slice count, head
width, in place or not. T spans the schedules: widened teams for small
batches, one round of one-wavefront rows (two rows per wavefront for FP8),
and several rounds. The shapes come from a fixed seed (QKNORM_RANDOM_SEED
picks another sequence), so a failing case replays exactly; each prints its
parameters before its GPU calls."""
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
VEC = {"f32": 4, "bf16": 8, "fp8": 16}
N_CASES = int(os.environ.get("QKNORM_RANDOM_CASES", "60"))  # more for a longer sweep
SEED = int(os.environ.get("QKNORM_RANDOM_SEED", "2024"))


@pytest.fixture(scope="module", autouse=True)
def _oracle_threads():
    oracle.set_threads(min(16, os.cpu_count() or 1))
    yield
    oracle.set_threads(1)


def draw_case(i):
    rng = np.random.default_rng([SEED, i])
    dtype = ["f32", "bf16", "fp8"][i % 3]
    ve = VEC[dtype]
    T = int(rng.choice([1, 2, 7, 64, 129, 300, 1000, 1100, 2048, 3001, 4500]))
    # slice count and head width first; both widths are multiples of the unit
    # that makes each cut whole vectors
    K = int(rng.choice([1, 2, 3, 4, 5, 8, 16, 64]))
    D = ve << int(rng.integers(0, 7))
    unit = int(np.lcm(K * ve, D))
    maxw = {"f32": 4096, "bf16": 6144, "fp8": 8192}[dtype]
    widths = []
    for _ in range(2):
        m = int(rng.integers(1, max(2, maxw // unit + 1)))
        widths.append(m * unit if m * unit <= qk_max(dtype) else unit)
    pad = ve * int(rng.integers(0, 4))
    in_place = bool(rng.integers(0, 2))
    return dict(dtype=dtype, T=T, Hq=widths[0], Hk=widths[1], K=K, D=D, pad=pad, in_place=in_place)


def qk_max(dtype):
    return {"f32": 32768, "bf16": 65536, "fp8": 65536}[dtype]


def padded(x, pad):
    """x laid out in a wider buffer (row stride width + pad), as a view."""
    T, H = x.shape
    buf = torch.zeros((T, H + pad), dtype=x.dtype, device=DEV)
    buf[:, :H] = x.to(DEV)
    return buf[:, :H]


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape(i):
    c = draw_case(i)
    dt, T, Hq, Hk, K, D = c["dtype"], c["T"], c["Hq"], c["Hk"], c["K"], c["D"]
    tdt = workloads.DTYPES[dt]
    gdt = "bf16" if dt == "fp8" else dt
    q = workloads.random_rows(T, Hq, dt, [i, 1], dist="laplace")
    k = workloads.random_rows(T, Hk, dt, [i, 2], scale=2.0)
    gq, gk = workloads.random_weights(Hq, gdt, [i, 3]), workloads.random_weights(Hk, gdt, [i, 4])
    print("[case]", i, c, flush=True)
    qd, kd = padded(q, c["pad"]), padded(k, c["pad"])
    yq, yk = qk.forward(qd, kd, gq.to(DEV), gk.to(DEV), eps=1e-6, num_slices=K,
                        out_q=qd if c["in_place"] else None, out_k=kd if c["in_place"] else None)
    torch.cuda.synchronize()
    assert_parity(yq, oracle.forward(q, gq, 1e-6, K)[0], tdt, "forward q")
    assert_parity(yk, oracle.forward(k, gk, 1e-6, K)[0], tdt, "forward k")
    qd, kd = padded(q, c["pad"]), padded(k, c["pad"])
    rq, rk = qk.inv_rms(qd, kd, eps=1e-6, num_slices=K)
    torch.cuda.synchronize()
    assert_parity(rq, oracle.inv_rms(q, 1e-6, K), torch.float32, "inv_rms q")
    assert_parity(rk, oracle.inv_rms(k, 1e-6, K), torch.float32, "inv_rms k")
    if D:
        hq, hk = workloads.random_weights(D, gdt, [i, 5]), workloads.random_weights(D, gdt, [i, 6])
        yq, yk = qk.forward_headwise(qd, kd, hq.to(DEV), hk.to(DEV), D, eps=1e-6)
        torch.cuda.synchronize()
        assert_parity(yq, oracle.headwise(q, hq, D, 1e-6), tdt, "headwise q")
        assert_parity(yk, oracle.headwise(k, hk, D, 1e-6), tdt, "headwise k")
    # split path over q: every slice's partial sums, then every slice's apply
    w = Hq // K
    stats = torch.zeros((K, T), dtype=torch.float32, device=DEV)
    for s in range(K):
        qk.partial_stats(qd[:, s * w:(s + 1) * w], s, K, stats)
    gqd = gq.to(DEV)
    ref = oracle.forward(q, gq, 1e-6, K)[0]
    for s in range(K):
        ys = qk.apply_stats(qd[:, s * w:(s + 1) * w], gqd[s * w:(s + 1) * w], stats, Hq, eps=1e-6)
        torch.cuda.synchronize()
        assert_parity(ys, ref[:, s * w:(s + 1) * w], tdt, "split slice %d" % s)
