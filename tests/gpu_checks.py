"""Comparison helpers for the GPU parity tests (host-side numpy only).

Acceptance bars:
  fp32 output: |y - y_ref| <= 1e-5 * |y_ref| elementwise (zero stays zero);
  bf16 output: |y - y_ref| <= one bf16 ulp of y_ref, i.e. the kernel's result
  is the round-to-nearest-even of the exact value or its neighbour, which
  bounds the relative error by 2^-7 = 7.8e-3;
  fp8 (e4m3) output: the same one-ulp rule in e4m3 (3 fraction bits) against
  y_ref saturated at +-448, and exactly +-448 where |y_ref| >= 464.
y_ref is the fp64 oracle. Error summaries (max-abs, MAE, RMSE) are the ones
the SwiftQK review reports against its fp64 gold RMSNorm (Fig. 2(b)).
"""
import numpy as np
import torch

F32_RTOL = 1e-5


def bf16_ulp(ref):
    """Spacing of bf16 values at |ref| (8 significant bits; subnormals below 2^-126)."""
    a = np.abs(ref)
    _, e = np.frexp(a)                   # a = m * 2^e, m in [0.5, 1)
    e = np.maximum(e - 8, -133)          # ulp = 2^(floor(log2 a) - 7) = 2^(e - 8)
    return np.ldexp(1.0, e)


E4M3_MAX = 448.0


def e4m3_ulp(ref):
    """Spacing of OCP FP8 E4M3 values at |ref|: 3 fraction bits, normal down
    to 2^-6, subnormal spacing 2^-9 below that."""
    a = np.abs(ref)
    _, e = np.frexp(np.maximum(a, 2.0 ** -6))  # floor(log2 a) = e - 1 for a >= 2^-6
    return np.ldexp(1.0, e - 1 - 3)


def e4m3_expected(ref):
    """The exact value the output approximates: the fp64 result, saturated at
    +-448 (NaN stays NaN)."""
    return np.clip(ref, -E4M3_MAX, E4M3_MAX)


def host64(t):
    """GPU or CPU tensor (fp32 / bf16) -> float64 numpy, exactly."""
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)


def errors(y, ref):
    d = np.abs(y - ref)
    return {"max_abs": float(d.max()) if d.size else 0.0,
            "mae": float(d.mean()) if d.size else 0.0,
            "rmse": float(np.sqrt((d * d).mean())) if d.size else 0.0,
            "max_rel": float((d / np.maximum(np.abs(ref), 1e-300)).max()) if d.size else 0.0}


def assert_parity(y_gpu, ref, dtype, what=""):
    """y_gpu: torch tensor (any device); ref: float64 numpy of the same shape."""
    y = host64(y_gpu)
    assert y.shape == ref.shape, (what, y.shape, ref.shape)
    assert np.isfinite(y).all() == np.isfinite(ref).all(), what
    if dtype == torch.float8_e4m3fn:
        # past the rounding boundary above 448 the result is exactly +-448
        over = np.abs(ref) >= 464.0
        assert (y[over] == np.sign(ref[over]) * E4M3_MAX).all(), (what, "saturation")
        ref = e4m3_expected(ref)
        bound = e4m3_ulp(ref)
    elif dtype == torch.float32:
        bound = F32_RTOL * np.abs(ref)
    else:
        bound = bf16_ulp(ref)
    d = np.abs(y - ref)
    bad = d > bound
    if bad.any():
        idx = np.argwhere(bad)[:5]
        detail = [(tuple(int(v) for v in i), float(y[tuple(i)]), float(ref[tuple(i)])) for i in idx]
        raise AssertionError("%s: %d of %d outside tolerance, first %s" % (what, int(bad.sum()), bad.size,
                                                                           detail))
    return errors(y, ref)


def assert_near_each_other(a, b, dtype, what=""):
    """Two GPU results that each meet the bar against the exact value differ
    by rounding only: at most 2e-5 relative (fp32) or one bf16 ulp of the
    larger (bf16: both round values within ~1e-6 of each other). Returns the
    fraction of bitwise-equal elements."""
    x, y = host64(a), host64(b)
    d = np.abs(x - y)
    big = np.maximum(np.abs(x), np.abs(y))
    if dtype == torch.float32:
        bound = 2 * F32_RTOL * big
    elif dtype == torch.float8_e4m3fn:
        bound = e4m3_ulp(big)
    else:
        bound = bf16_ulp(big)
    bad = d > bound
    assert not bad.any(), "%s: %d elements differ by more than rounding" % (what, int(bad.sum()))
    return float((x == y).mean()) if x.size else 1.0
