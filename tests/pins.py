"""Pins for the fp64 oracle: facts fixed by the pages or by mathematics.

Each `pin_*` function raises AssertionError when the oracle disagrees with
something other than itself: a value printed on the pages, a closed form, an
exact-arithmetic computation, an invariant, or a library routine. The
mutation tests run all of them against deliberately broken copies of the
oracle and require every copy to fail at least one.
"""
import math

import numpy as np
import torch

import oracle
from oracle import exact
from attention_qk_norm_amd import workloads
from conftest import read_golden

F32 = np.float32


def _ex(x):
    return np.asarray(x, dtype=F32).reshape(1, -1)


def pin_worked_example_printed():
    """SwiftQK review section 4b, Eqs. (2)-(8), values as printed."""
    g = read_golden("swiftqk_worked_example.txt")
    x = _ex(g["x"])
    H = int(g["H_total"][0])
    K = int(g["num_slices"][0])
    eps = g["eps"][0]
    P = oracle.slice_sumsq(x, K)
    assert P[:, 0].tolist() == g["S_local"], ("Eqs. 3-4", P[:, 0])
    y, P2 = oracle.forward(x, np.asarray(g["gamma"], F32), eps, K)
    assert P2[:, 0].tolist() == g["S_local"]
    assert P2[:, 0].sum() == g["S_global"][0], "Eq. 5"
    assert P2[:, 0].sum() / H == g["mean"][0], "Eq. 6 mean"
    # gamma = 1, so y_j / x_j is the inverse RMS of Eq. 6
    r_tol = 0.5 * 10 ** -g["rms_inv_digits"][0]
    for j in range(H):
        r = y[0, j] / x[0, j]
        assert abs(r - g["rms_inv"][0]) <= r_tol, ("Eq. 6", j, r)
    # Eqs. 7-8 were printed after multiplying by the rounded 0.6065: allow the
    # printing error plus |x_j| times that rounding error
    y_tol = 0.5 * 10 ** -g["y_digits"][0]
    for j in range(H):
        tol = y_tol + abs(x[0, j]) * r_tol
        assert abs(y[0, j] - g["y"][j]) <= tol, ("Eqs. 7-8", j, y[0, j], g["y"][j])
    # the slice path and the one-slice path agree (section 4b "sanity check")
    y1, P1 = oracle.forward(x, np.asarray(g["gamma"], F32), eps, 1)
    assert P1[0, 0] == g["S_global"][0]
    assert np.array_equal(y1, y)
    # Eqs. 7-8 are the per-shard path: each shard is normalised on its own,
    # using the combined statistic and the full width H_total = 8
    w = H // K
    for r in range(K):
        xs = x[:, r * w:(r + 1) * w]
        Pr = oracle.slice_sumsq(xs, 1)
        assert Pr[0, 0] == g["S_local"][r], ("Eq. %d" % (3 + r))
        ys = oracle.apply(xs, P, np.asarray(g["gamma"][r * w:(r + 1) * w], F32), H, eps)
        for j in range(w):
            tol = y_tol + abs(xs[0, j]) * r_tol
            assert abs(ys[0, j] - g["y"][r * w + j]) <= tol, ("Eq. %d" % (7 + r), j)


def pin_worked_example_exact():
    """Same example against exact rational arithmetic (60 digits)."""
    g = read_golden("swiftqk_worked_example.txt")
    x = _ex(g["x"])
    gam = np.asarray(g["gamma"], F32)
    eps = oracle.eps_as_gpu_sees_it(g["eps"][0])
    y, _ = oracle.forward(x, gam, eps, 2)
    ref = [float(v) for v in exact.rmsnorm_row(x[0], gam, eps)]
    np.testing.assert_allclose(y[0], ref, rtol=1e-15, atol=0)


def pin_four_element_closed_form():
    """The first shard of the worked example as a whole row (H = 4):
    sum of squares 6.25, mean 1.5625, RMS exactly 1.25."""
    x = _ex([1.0, 2.0, -1.0, 0.5])
    one = np.ones(4, F32)
    y, P = oracle.forward(x, one, 0.0, 1)
    assert P[0, 0] == 6.25
    np.testing.assert_allclose(y[0], [0.8, 1.6, -0.8, 0.4], rtol=1e-15, atol=0)
    # weights act per column, in column order
    y, _ = oracle.forward(x, np.asarray([1.0, 0.5, 2.0, 4.0], F32), 0.0, 1)
    np.testing.assert_allclose(y[0], [0.8, 0.8, -1.6, 1.6], rtol=1e-15, atol=0)
    # eps is added to the mean inside the square root
    eps = oracle.eps_as_gpu_sees_it(1e-6)
    r = 1.0 / math.sqrt(1.5625 + eps)
    y, _ = oracle.forward(x, one, 1e-6, 1)
    np.testing.assert_allclose(y[0], x[0].astype(np.float64) * r, rtol=2e-16, atol=0)
    # and that is distinguishable from eps added outside the root
    assert abs(r - 1.0 / (1.25 + eps)) / r > 1e-7
    # with K = 2 slices of 2 the result is the same: the mean divides by H = 4
    y2, P2 = oracle.forward(x, one, 1e-6, 2)
    assert P2[:, 0].tolist() == [5.0, 1.25]
    np.testing.assert_allclose(y2[0], x[0].astype(np.float64) * r, rtol=2e-16, atol=0)


def pin_exact_sums_any_slicing():
    """On rows of n/16 values every partial sum is exact, so all slicings give
    the same statistic, equal to the integer sum of n^2 over 256."""
    for T, H, seed in ((8, 1024, 11), (1, 16384, 12), (3, 96, 13)):
        x = workloads.exact_sum_rows(T, H, "f32", seed).numpy()
        n = np.rint(x.astype(np.float64) * 16).astype(np.int64)
        full = (n * n).sum(axis=1) / 256.0
        y1, P1 = oracle.forward(x, np.ones(H, F32), 1e-6, 1)
        assert np.array_equal(P1[0], full)
        for K in (2, 3, 4, 8, 16):
            if H % K:
                continue
            w = H // K
            yK, PK = oracle.forward(x, np.ones(H, F32), 1e-6, K)
            for s in range(K):
                ns = n[:, s * w:(s + 1) * w]
                assert np.array_equal(PK[s], (ns * ns).sum(axis=1) / 256.0), (K, s)
            assert np.array_equal(PK.sum(axis=0), full)
            assert np.array_equal(yK, y1), K


def pin_slicing_general_inputs():
    """On general inputs the slice path differs from the one-slice path only
    by rounding order."""
    x = workloads.random_rows(16, 1280, "f32", 21).numpy()
    g = workloads.random_weights(1280, "f32", 22).numpy()
    y1, P1 = oracle.forward(x, g, 1e-6, 1)
    for K in (2, 4, 5, 10):
        yK, PK = oracle.forward(x, g, 1e-6, K)
        np.testing.assert_allclose(PK.sum(axis=0), P1[0], rtol=1e-13)
        np.testing.assert_allclose(yK, y1, rtol=1e-13)


def pin_scale_invariance():
    """y(c x; c^2 eps) = y(x; eps) for c > 0, and y(-x) = -y(x). Powers of
    two scale exactly in binary floating point, so those cases are bitwise."""
    x = workloads.random_rows(6, 256, "f32", 31).numpy()
    g = workloads.random_weights(256, "f32", 32).numpy()
    eps = oracle.eps_as_gpu_sees_it(1e-6)
    y, _ = oracle.forward(x, g, eps, 4)
    for j in (-3, 5):
        c = 2.0 ** j
        yc, _ = oracle.forward((x * F32(c)).astype(F32), g, eps * (c * c), 4)
        assert np.array_equal(yc, y), j
    yn, _ = oracle.forward(-x, g, eps, 4)
    assert np.array_equal(yn, -y)
    # non-power-of-two scale on values where c*x stays exact in fp32
    xs = workloads.exact_sum_rows(4, 64, "f32", 33).numpy()
    y0, _ = oracle.forward(xs, np.ones(64, F32), 0.0, 2)
    y3, _ = oracle.forward((xs * F32(3)).astype(F32), np.ones(64, F32), 0.0, 2)
    np.testing.assert_allclose(y3, y0, rtol=1e-15, atol=0)
    # with eps fixed the output still barely moves for c >= 1
    yb, _ = oracle.forward((x * F32(4)).astype(F32), g, eps, 4)
    np.testing.assert_allclose(yb, y, rtol=1e-5)


def pin_unit_rms():
    """With gamma = 1 the output's mean square is m / (m + eps), m = mean(x^2)."""
    for seed, H in ((41, 4096), (42, 8), (43, 1000)):
        x = workloads.random_rows(5, H, "f32", seed, scale=0.01).numpy()
        eps = oracle.eps_as_gpu_sees_it(1e-6)
        y, _ = oracle.forward(x, np.ones(H, F32), eps, 1)
        xd = x.astype(np.float64)
        m = (xd * xd).mean(axis=1)
        np.testing.assert_allclose((y * y).mean(axis=1), m / (m + eps), rtol=1e-13)
        y0, _ = oracle.forward(x, np.ones(H, F32), 0.0, 1)
        np.testing.assert_allclose((y0 * y0).mean(axis=1), 1.0, rtol=1e-13)


def pin_special_cases():
    """A constant row, a one-column row, and the slice-wise split path."""
    eps = oracle.eps_as_gpu_sees_it(1e-6)
    g = workloads.random_weights(32, "f32", 51).numpy()
    for a in (0.75, -3.0, 0.0):
        x = np.full((1, 32), a, F32)
        y, _ = oracle.forward(x, g, eps, 4)
        np.testing.assert_allclose(y[0], a / math.sqrt(a * a + eps) * g.astype(np.float64),
                                   rtol=1e-15, atol=0)
    x1 = np.asarray([[2.5], [-0.125], [7.0]], F32)
    g1 = np.asarray([1.5], F32)
    y1, _ = oracle.forward(x1, g1, eps, 1)
    for t in range(3):
        v = float(x1[t, 0])
        assert abs(y1[t, 0] - v * 1.5 / math.sqrt(v * v + eps)) <= 1e-15 * abs(y1[t, 0])
    # split path: slice statistics, then each slice normalised on its own with
    # the full width as the denominator, reproduce the whole-row forward
    x = workloads.random_rows(7, 96, "f32", 52).numpy()
    gw = workloads.random_weights(96, "f32", 53).numpy()
    yf, _ = oracle.forward(x, gw, eps, 1)
    K, w = 3, 32
    P = np.stack([oracle.slice_sumsq(x[:, s * w:(s + 1) * w], 1)[0] for s in range(K)])
    for s in range(K):
        ys = oracle.apply(x[:, s * w:(s + 1) * w], P, gw[s * w:(s + 1) * w], 96, eps)
        np.testing.assert_allclose(ys, yf[:, s * w:(s + 1) * w], rtol=1e-15, atol=0)
    # one slice: apply over the whole row is the forward
    P1 = oracle.slice_sumsq(x, 1)
    np.testing.assert_array_equal(oracle.apply(x, P1, gw, 96, eps), yf)


def pin_brute_force_rows():
    """Several distinct rows (T != H) against exact arithmetic row by row:
    catches row-stride, transposition and column-order mistakes."""
    T, H = 3, 12
    x = workloads.random_rows(T, H, "f32", 61).numpy()
    g = workloads.random_weights(H, "f32", 62).numpy()
    eps = oracle.eps_as_gpu_sees_it(1e-6)
    for K in (1, 3):
        y, P = oracle.forward(x, g, eps, K)
        for t in range(T):
            ref = [float(v) for v in exact.rmsnorm_row(x[t], g, eps)]
            np.testing.assert_allclose(y[t], ref, rtol=1e-15, atol=0)
            assert abs(P[:, t].sum() - float(exact.sum_of_squares(x[t]))) <= 1e-15 * P[:, t].sum()


def pin_tiny_workload_exact():
    """The tiny fp32 workload (4 tokens, rows of 256) row by row against exact
    arithmetic, for both of its slice counts and both tensors."""
    d = workloads.generate("c1")
    w = d["w"]
    eps = oracle.eps_as_gpu_sees_it(w.eps)
    for which in ("q", "k"):
        x = oracle.as_f32(d[which])
        g = oracle.as_f32(d["gamma_" + which])
        refs = [[float(v) for v in exact.rmsnorm_row(x[t], g, eps)] for t in range(w.T)]
        for K in w.slices:
            y, _ = oracle.forward(x, g, w.eps, K)
            for t in range(w.T):
                np.testing.assert_allclose(y[t], refs[t], rtol=1e-15, atol=0)


def pin_library_rms_norm():
    """torch.nn.functional.rms_norm in float64 is an independent textbook
    implementation of Eq. 1."""
    for name in ("c1", "c3"):
        d = workloads.generate(name)
        w = d["w"]
        for which in ("q", "k"):
            x = d[which][:64]
            g = d["gamma_" + which]
            y, _ = oracle.forward(x, g, w.eps, w.slices[0])
            ref = torch.nn.functional.rms_norm(
                x.double(), (x.shape[1],), g.double(), oracle.eps_as_gpu_sees_it(w.eps)).numpy()
            np.testing.assert_allclose(y, ref, rtol=1e-14, atol=0)


def pin_headwise_closed_form():
    """Headwise statistics on the worked example's row (H = 8) cut into two
    heads of 4: the first head's sum of squares is 6.25, so with eps = 0 its
    RMS is exactly 1.25; the second head's is 15.5 (mean 3.875). Each head is
    normalised by its own statistic, and the 4 weights apply to both heads."""
    x = _ex([1.0, 2.0, -1.0, 0.5, 3.0, -2.0, 1.5, 0.5])
    g = np.asarray([1.0, 0.5, 2.0, 4.0], F32)
    y = oracle.headwise(x, np.ones(4, F32), 4, 0.0)
    np.testing.assert_allclose(y[0, :4], [0.8, 1.6, -0.8, 0.4], rtol=1e-15, atol=0)
    r1 = 1.0 / math.sqrt(3.875)
    np.testing.assert_allclose(y[0, 4:], [3.0 * r1, -2.0 * r1, 1.5 * r1, 0.5 * r1], rtol=2e-16, atol=0)
    y = oracle.headwise(x, g, 4, 0.0)
    np.testing.assert_allclose(y[0, :4], [0.8, 0.8, -1.6, 1.6], rtol=1e-15, atol=0)
    np.testing.assert_allclose(y[0, 4:], [3.0 * r1, -1.0 * r1, 3.0 * r1, 2.0 * r1], rtol=2e-16, atol=0)
    # eps joins each head's own mean inside the root
    eps = oracle.eps_as_gpu_sees_it(1e-6)
    y = oracle.headwise(x, np.ones(4, F32), 4, 1e-6)
    np.testing.assert_allclose(y[0, :4], x[0, :4].astype(np.float64) / math.sqrt(1.5625 + eps), rtol=2e-16)
    np.testing.assert_allclose(y[0, 4:], x[0, 4:].astype(np.float64) / math.sqrt(3.875 + eps), rtol=2e-16)
    # heads of 2: sums 5, 1.25, 13, 2.5 (means 2.5, 0.625, 6.5, 1.25)
    y = oracle.headwise(x, np.ones(2, F32), 2, 0.0)
    for h, m in enumerate((2.5, 0.625, 6.5, 1.25)):
        np.testing.assert_allclose(y[0, 2 * h:2 * h + 2],
                                   x[0, 2 * h:2 * h + 2].astype(np.float64) / math.sqrt(m), rtol=2e-16)


def pin_headwise_exact_rows():
    """Distinct rows and heads against exact arithmetic, head by head, with
    the shared weights: catches head-offset, weight-index and stride mistakes."""
    T, D, nh = 3, 8, 4
    x = workloads.random_rows(T, D * nh, "f32", 71).numpy()
    g = workloads.random_weights(D, "f32", 72).numpy()
    eps = oracle.eps_as_gpu_sees_it(1e-6)
    y = oracle.headwise(x, g, D, eps)
    for t in range(T):
        for h in range(nh):
            ref = [float(v) for v in exact.rmsnorm_row(x[t, h * D:(h + 1) * D], g, eps)]
            np.testing.assert_allclose(y[t, h * D:(h + 1) * D], ref, rtol=1e-15, atol=0)


def pin_headwise_reductions():
    """One head spanning the row is the layerwise norm; heads are independent
    of each other; torch's rms_norm over the rows reshaped to one head per row
    (float64) is an independent library implementation."""
    eps = oracle.eps_as_gpu_sees_it(1e-6)
    x = workloads.random_rows(5, 512, "f32", 81).numpy()
    g = workloads.random_weights(512, "f32", 82).numpy()
    y1, _ = oracle.forward(x, g, eps, 1)
    assert np.array_equal(oracle.headwise(x, g, 512, eps), y1)
    D = 128
    gh = workloads.random_weights(D, "f32", 83).numpy()
    y = oracle.headwise(x, gh, D, eps)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x).double().reshape(-1, D), (D,),
                                       torch.from_numpy(gh).double(), eps).reshape(5, 512).numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-14, atol=0)
    # scaling head 2 changes head 2 only; with eps = 0 not even head 2
    x2 = x.copy()
    x2[:, 2 * D:3 * D] *= F32(4)
    y2 = oracle.headwise(x2, gh, D, eps)
    keep = np.r_[0:2 * D, 3 * D:4 * D]
    assert np.array_equal(y2[:, keep], y[:, keep])
    assert not np.array_equal(y2[:, 2 * D:3 * D], y[:, 2 * D:3 * D])
    assert np.array_equal(oracle.headwise(x2, gh, D, 0.0), oracle.headwise(x, gh, D, 0.0))
    # unit mean square per head when the weights are 1 and eps = 0
    y0 = oracle.headwise(x, np.ones(D, F32), D, 0.0).reshape(5, 4, D)
    np.testing.assert_allclose((y0 * y0).mean(axis=2), 1.0, rtol=1e-13)


def pin_inv_rms():
    """The inverse RMS on its own: Eq. 6's printed 0.6065 (and the exact
    value from rational arithmetic) for the worked example with K = 2 and 1,
    exactly 0.8 for the four-element shard with eps = 0, and, on general
    rows, the factor that turns x * gamma into the forward's output."""
    g = read_golden("swiftqk_worked_example.txt")
    x = _ex(g["x"])
    eps = oracle.eps_as_gpu_sees_it(g["eps"][0])
    exact_r = float(1 / exact._dec(exact.sum_of_squares(x[0]) / 8 + exact.Fraction(eps)).sqrt())
    for K in (2, 1):
        r = oracle.inv_rms(x, g["eps"][0], K)
        assert abs(r[0] - g["rms_inv"][0]) <= 0.5 * 10 ** -g["rms_inv_digits"][0], ("Eq. 6", K, r[0])
        assert abs(r[0] - exact_r) <= 1e-16, (K, r[0], exact_r)
    assert oracle.inv_rms(_ex([1.0, 2.0, -1.0, 0.5]), 0.0, 1)[0] == 0.8
    assert oracle.inv_rms(_ex([1.0, 2.0, -1.0, 0.5]), 0.0, 2)[0] == 0.8
    xs = workloads.random_rows(9, 640, "f32", 91).numpy()
    gs = workloads.random_weights(640, "f32", 92).numpy()
    y, _ = oracle.forward(xs, gs, 1e-6, 5)
    r = oracle.inv_rms(xs, 1e-6, 5)
    np.testing.assert_allclose(y, xs.astype(np.float64) * r[:, None] * gs.astype(np.float64), rtol=1e-15)
    # a constant row a: 1 / sqrt(a^2 + eps)
    assert abs(oracle.inv_rms(np.full((1, 64), 0.75, F32), 1e-6, 4)[0] - 1 / math.sqrt(0.5625 + eps)) < 1e-15


ALL_PINS = [
    pin_worked_example_printed,
    pin_worked_example_exact,
    pin_four_element_closed_form,
    pin_exact_sums_any_slicing,
    pin_slicing_general_inputs,
    pin_scale_invariance,
    pin_unit_rms,
    pin_special_cases,
    pin_brute_force_rows,
    pin_tiny_workload_exact,
    pin_library_rms_norm,
    pin_headwise_closed_form,
    pin_headwise_exact_rows,
    pin_headwise_reductions,
    pin_inv_rms,
]
