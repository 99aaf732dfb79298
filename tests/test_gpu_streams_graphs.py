"""The library under a serving loop's conditions: calls captured in a HIP
graph and replayed, and calls on several streams at once. The library keeps
no state between calls and allocates nothing, so both must reproduce the
eager results bit for bit."""
import pytest
import torch

import attention_qk_norm_amd as qk
from attention_qk_norm_amd import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(*a):
    print("[case]", *a, flush=True)


def bits(t):
    return t.cpu().contiguous().view(torch.uint8)


def test_graph_capture_and_replay():
    """Fused forward (K = 4), headwise and inverse RMS captured in one graph,
    with a grouped-query pair large enough to take one launch per tensor;
    each replay, with unrelated eager work and a synchronisation in between,
    matches the eager call on fresh inputs copied into the captured buffers."""
    T, Hq, Hk = 96, 4096, 1024
    q = torch.empty((T, Hq), dtype=torch.bfloat16, device=DEV)
    k = torch.empty((T, Hk), dtype=torch.bfloat16, device=DEV)
    gq = workloads.random_weights(Hq, "bf16", 1).to(DEV)
    gk = workloads.random_weights(Hk, "bf16", 2).to(DEV)
    hg = workloads.random_weights(128, "bf16", 3).to(DEV)
    yq, yk = torch.empty_like(q), torch.empty_like(k)
    hq, hk = torch.empty_like(q), torch.empty_like(k)
    rq = torch.empty(T, device=DEV)
    rk = torch.empty(T, device=DEV)
    # 3700 x 16384/2048 in 8 slices: only the key rows need the narrow-slice
    # kernels, and the pair holds over 2^23 vectors
    TB, BQ, BK = 3700, 16384, 2048
    bq0 = workloads.random_rows(TB, BQ, "bf16", 20).to(DEV)
    bk0 = workloads.random_rows(TB, BK, "bf16", 21).to(DEV)
    bq, bk = torch.empty_like(bq0), torch.empty_like(bk0)
    gbq = workloads.random_weights(BQ, "bf16", 22).to(DEV)
    gbk = workloads.random_weights(BK, "bf16", 23).to(DEV)
    ybq, ybk = torch.empty_like(bq0), torch.empty_like(bk0)

    def calls(stream):
        qk.forward(q, k, gq, gk, eps=1e-6, num_slices=4, out_q=yq, out_k=yk, stream=stream)
        qk.forward_headwise(q, k, hg, hg, 128, eps=1e-6, out_q=hq, out_k=hk, stream=stream)
        qk.inv_rms(q, k, eps=1e-6, num_slices=4, out_q=rq, out_k=rk, stream=stream)
        qk.forward(bq, bk, gbq, gbk, eps=1e-6, num_slices=8, out_q=ybq, out_k=ybk, stream=stream)

    s = torch.cuda.Stream()
    q.copy_(workloads.random_rows(T, Hq, "bf16", 10).to(DEV))
    k.copy_(workloads.random_rows(T, Hk, "bf16", 11).to(DEV))
    bq.copy_(bq0)
    bk.copy_(bk0)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):  # warm the stream, as capture requires
        calls(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    say("capture")
    with torch.cuda.graph(g, stream=s):
        calls(s)
    torch.cuda.synchronize()
    for rep in range(4):
        q.copy_(workloads.random_rows(T, Hq, "bf16", 100 + rep).to(DEV))
        k.copy_(workloads.random_rows(T, Hk, "bf16", 200 + rep).to(DEV))
        bq.copy_(bq0.roll(rep + 1, dims=0))
        bk.copy_(bk0.roll(rep + 1, dims=0))
        torch.cuda.synchronize()
        say("replay", rep)
        g.replay()
        torch.cuda.synchronize()
        got = [bits(t) for t in (yq, yk, hq, hk, rq, rk, ybq, ybk)]
        junk = torch.randn(1 << 20, device=DEV).sum()  # unrelated eager work between replays
        calls(torch.cuda.current_stream())
        torch.cuda.synchronize()
        want = [bits(t) for t in (yq, yk, hq, hk, rq, rk, ybq, ybk)]
        for a, b in zip(got, want):
            assert torch.equal(a, b), rep
        del junk


def test_concurrent_streams():
    """Independent batches on four streams at once give the results each
    gives alone."""
    T, H = 300, 4096
    xs = [workloads.random_rows(T, H, "bf16", 30 + i).to(DEV) for i in range(4)]
    g = workloads.random_weights(H, "bf16", 40).to(DEV)
    alone = []
    for x in xs:
        y, _ = qk.forward(x, None, g, None, eps=1e-6, num_slices=8)
        torch.cuda.synchronize()
        alone.append(bits(y))
    streams = [torch.cuda.Stream() for _ in xs]
    outs = [torch.empty_like(x) for x in xs]
    torch.cuda.synchronize()
    say("four streams")
    for _ in range(3):
        for x, o, st in zip(xs, outs, streams):
            with torch.cuda.stream(st):
                qk.forward(x, None, g, None, eps=1e-6, num_slices=8, out_q=o, stream=st)
        torch.cuda.synchronize()
        for o, a in zip(outs, alone):
            assert torch.equal(bits(o), a)


def test_shared_context_from_threads():
    """One context shared by four host threads, each enqueueing on its own
    stream (validation and planning keep no mutable state): every thread's
    results equal the single-threaded ones, bit for bit."""
    import threading

    ctx = qk.Context(0)
    shapes = [(300, 4096, 1024, "bf16", 8), (2048, 5120, 1024, "fp8", 1), (64, 4096, 4096, "bf16", 1),
              (129, 1536, 512, "f32", 4)]
    cases = []
    for i, (T, hq, hk, dt, K) in enumerate(shapes):
        gdt = "bf16" if dt == "fp8" else dt
        q = workloads.random_rows(T, hq, dt, 50 + i).to(DEV)
        k = workloads.random_rows(T, hk, dt, 60 + i).to(DEV)
        gq = workloads.random_weights(hq, gdt, 70 + i).to(DEV)
        gk = workloads.random_weights(hk, gdt, 80 + i).to(DEV)
        say("single thread", T, hq, hk, dt, K)
        yq, yk = qk.forward(q, k, gq, gk, eps=1e-6, num_slices=K, ctx=ctx)
        torch.cuda.synchronize()
        cases.append(dict(q=q, k=k, gq=gq, gk=gk, K=K, want=(bits(yq), bits(yk)),
                          out=(torch.empty_like(q), torch.empty_like(k)), stream=torch.cuda.Stream()))
    torch.cuda.synchronize()
    failures = []

    def work(c):
        try:
            oq, ok = c["out"]
            for _ in range(20):
                qk.forward(c["q"], c["k"], c["gq"], c["gk"], eps=1e-6, num_slices=c["K"], out_q=oq, out_k=ok,
                           ctx=ctx, stream=c["stream"])
            c["stream"].synchronize()
        except Exception as e:  # reported by the main thread
            failures.append(repr(e))

    say("four threads, one context")
    threads = [threading.Thread(target=work, args=(c,)) for c in cases]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert not any(t.is_alive() for t in threads)
    torch.cuda.synchronize()
    assert not failures, failures
    for c in cases:
        assert torch.equal(bits(c["out"][0]), c["want"][0])
        assert torch.equal(bits(c["out"][1]), c["want"][1])
