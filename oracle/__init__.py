"""fp64 CPU oracle for layerwise QK-Norm -- TEST INFRASTRUCTURE ONLY.

Only `tests/`, the smoke check and the benchmark's CPU-baseline leg may import
this package. It shares no code with the HIP path: it reads plain numpy arrays
and calls the C reference in `qknorm_oracle.c` (SwiftQK technical review,
Eq. 1, with the sum of squares split into contiguous column slices as in the
section 4b worked example, Eqs. 3-6).

Inputs are handed to the C code as float32 arrays. Both fp32 data and bf16
data widen to float32 exactly, so the C code sees exactly the values the GPU
sees; it widens them to double before doing any arithmetic.
"""
import contextlib
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None
_dp = ctypes.POINTER(ctypes.c_double)
_fp = ctypes.POINTER(ctypes.c_float)


def load(path):
    """Open a compiled oracle shared object and declare its signatures."""
    L = ctypes.CDLL(path)
    i64 = ctypes.c_int64
    L.oracle_set_threads.argtypes = [ctypes.c_int]
    L.oracle_set_threads.restype = ctypes.c_int
    L.oracle_get_threads.argtypes = []
    L.oracle_get_threads.restype = ctypes.c_int
    L.oracle_slice_sumsq.argtypes = [_fp, i64, i64, i64, ctypes.c_int, _dp]
    L.oracle_slice_sumsq.restype = None
    L.oracle_apply.argtypes = [_fp, i64, i64, i64, _dp, ctypes.c_int, _fp,
                               i64, ctypes.c_double, _dp, i64]
    L.oracle_apply.restype = None
    L.oracle_forward.argtypes = [_fp, i64, i64, i64, _fp, ctypes.c_double,
                                 ctypes.c_int, _dp, _dp, i64]
    L.oracle_forward.restype = None
    L.oracle_headwise.argtypes = [_fp, i64, i64, i64, i64, _fp, ctypes.c_double, _dp, i64]
    L.oracle_headwise.restype = None
    L.oracle_inv_rms.argtypes = [_fp, i64, i64, i64, ctypes.c_int, ctypes.c_double, _dp, _dp]
    L.oracle_inv_rms.restype = None
    return L


def lib():
    """Load the C oracle, building it first when the shared object is missing
    or older than its source."""
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB) or os.path.getmtime(_build.LIB) < os.path.getmtime(_build.SRC):
            _build.build()
        _lib = load(_build.LIB)
    return _lib


@contextlib.contextmanager
def using(path):
    """Temporarily route every oracle call through another compiled copy of
    the oracle (the mutation tests plant mistakes in such copies)."""
    global _lib
    saved = lib()
    _lib = load(path)
    try:
        yield _lib
    finally:
        _lib = saved


def set_threads(n):
    """Threads the oracle's token loops use; returns the count in force."""
    return lib().oracle_set_threads(int(n))


def as_f32(a):
    """Exact float32 view of the values in `a` (numpy array or CPU torch tensor
    of dtype float32, bfloat16 or float8_e4m3fn). Each widens to fp32
    exactly."""
    if hasattr(a, "detach"):  # torch tensor
        import torch
        t = a.detach().to("cpu")
        if t.dtype in (torch.bfloat16, torch.float8_e4m3fn):
            t = t.to(torch.float32)  # exact widening
        if t.dtype != torch.float32:
            raise TypeError("oracle takes float32, bfloat16 or float8_e4m3fn data, got %s" % t.dtype)
        return np.ascontiguousarray(t.numpy())
    a = np.asarray(a)
    if a.dtype != np.float32:
        if a.dtype == np.float64 and np.array_equal(a, a.astype(np.float32).astype(np.float64)):
            return np.ascontiguousarray(a.astype(np.float32))
        raise TypeError("oracle takes values exactly representable in float32")
    return np.ascontiguousarray(a)


def eps_as_gpu_sees_it(eps):
    """The library receives eps as a C float: use that exact value in fp64."""
    return float(np.float32(eps))


def _rows(x):
    x = as_f32(x)
    if x.ndim != 2:
        raise ValueError("rows must be a 2-D array [T, W]")
    return x


def slice_sumsq(x, num_slices):
    """Per-slice sums of squares (review Eqs. 3-4).

    x: [T, W] values; the W columns are cut into `num_slices` equal contiguous
    slices. Returns P: float64 [num_slices, T], P[s, t] = sum_{j in slice s} x[t, j]^2.
    """
    x = _rows(x)
    T, W = x.shape
    K = int(num_slices)
    if K < 1 or W % K:
        raise ValueError("width %d is not cut evenly into %d slices" % (W, K))
    P = np.empty((K, T), dtype=np.float64)
    lib().oracle_slice_sumsq(x.ctypes.data_as(_fp), T, W, W, K, P.ctypes.data_as(_dp))
    return P


def apply(x, P, gamma, H_total, eps):
    """Combine K slice statistics per token and normalise (Eqs. 5-6, Eq. 1).

    x: [T, W] columns to normalise (a whole row or one slice of it);
    P: [K, T] partial sums covering the FULL row of width H_total;
    gamma: [W]. Returns y: float64 [T, W].
    """
    x = _rows(x)
    T, W = x.shape
    P = np.ascontiguousarray(np.asarray(P, dtype=np.float64))
    if P.ndim != 2 or P.shape[1] != T:
        raise ValueError("P must be [K, T]")
    g = as_f32(gamma).reshape(-1)
    if g.shape[0] != W:
        raise ValueError("gamma must have one weight per column")
    y = np.empty((T, W), dtype=np.float64)
    lib().oracle_apply(x.ctypes.data_as(_fp), T, W, W, P.ctypes.data_as(_dp),
                       P.shape[0], g.ctypes.data_as(_fp), int(H_total),
                       eps_as_gpu_sees_it(eps), y.ctypes.data_as(_dp), W)
    return y


def forward(x, gamma, eps, num_slices=1):
    """RMSNorm of every row of x (Eq. 1) via K slice statistics.

    Returns (y float64 [T, H], P float64 [K, T]).
    """
    x = _rows(x)
    T, H = x.shape
    K = int(num_slices)
    if K < 1 or H % K:
        raise ValueError("width %d is not cut evenly into %d slices" % (H, K))
    g = as_f32(gamma).reshape(-1)
    if g.shape[0] != H:
        raise ValueError("gamma must have one weight per column")
    P = np.empty((K, T), dtype=np.float64)
    y = np.empty((T, H), dtype=np.float64)
    lib().oracle_forward(x.ctypes.data_as(_fp), T, H, H, g.ctypes.data_as(_fp),
                         eps_as_gpu_sees_it(eps), K, P.ctypes.data_as(_dp),
                         y.ctypes.data_as(_dp), H)
    return y, P


def qk_forward(q, k, gamma_q, gamma_k, eps, num_slices=1):
    """Layerwise QK-Norm: the projected query rows and the projected key rows
    are normalised separately, each with its own width and weights
    (review, "Layerwise vs. headwise QK-Norm"; Fig. 1(a): two RMSNorm layers).
    Returns (y_q, y_k) in float64."""
    yq, _ = forward(q, gamma_q, eps, num_slices)
    yk, _ = forward(k, gamma_k, eps, num_slices)
    return yq, yk


def headwise(x, gamma, head_dim, eps):
    """Headwise RMSNorm (review, "Layerwise vs. headwise QK-Norm"): every
    head of `head_dim` contiguous columns is normalised with its own
    statistic, and the `head_dim` weights of gamma are shared by all heads.

    x: [T, H] with H a multiple of head_dim; gamma: [head_dim].
    Returns y float64 [T, H]."""
    x = _rows(x)
    T, H = x.shape
    D = int(head_dim)
    if D < 1 or H % D:
        raise ValueError("width %d is not a whole number of %d-column heads" % (H, D))
    g = as_f32(gamma).reshape(-1)
    if g.shape[0] != D:
        raise ValueError("gamma must have head_dim weights")
    y = np.empty((T, H), dtype=np.float64)
    lib().oracle_headwise(x.ctypes.data_as(_fp), T, H, H, D, g.ctypes.data_as(_fp),
                          eps_as_gpu_sees_it(eps), y.ctypes.data_as(_dp), H)
    return y


def qk_headwise(q, k, gamma_q, gamma_k, head_dim, eps):
    """Headwise QK-Norm of the query rows and the key rows, each tensor with
    its own head_dim-long weights. Returns (y_q, y_k) in float64."""
    return headwise(q, gamma_q, head_dim, eps), headwise(k, gamma_k, head_dim, eps)


def inv_rms(x, eps, num_slices=1):
    """Per-token inverse RMS 1 / sqrt(S / H + eps) (review Eq. 6), with S the
    ascending sum of `num_slices` slice sums. x: [T, H]. Returns float64 [T]."""
    x = _rows(x)
    T, H = x.shape
    K = int(num_slices)
    if K < 1 or H % K:
        raise ValueError("width %d is not cut evenly into %d slices" % (H, K))
    P = np.empty((K, T), dtype=np.float64)
    r = np.empty(T, dtype=np.float64)
    lib().oracle_inv_rms(x.ctypes.data_as(_fp), T, H, H, K, eps_as_gpu_sees_it(eps),
                         P.ctypes.data_as(_dp), r.ctypes.data_as(_dp))
    return r
