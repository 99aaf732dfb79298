"""Layerwise QK-Norm for AMD Instinct MI355X (gfx950).

A thin ctypes binding over the C ABI of `libqknorm.so` (declared in
`include/qknorm.h`). It only marshals arguments: every step of the
normalisation runs in the library's HIP kernels. PyTorch supplies device
memory (tensors) and the stream (torch's current stream). There is no CPU
fallback: when the library is missing or no gfx950 device is present the
calls raise.

    y_q, y_k = forward(q, k, gamma_q, gamma_k, eps=1e-6, num_slices=1)

normalises every row of q [T, Hq] and of k [T, Hk] over its full width
(SwiftQK technical review, Eq. 1), forming each row's sum of squares as the
ascending sum of `num_slices` per-slice partials (section 4b, Eqs. 3-6).
The other entry points:

    forward_headwise(q, k, hgamma_q, hgamma_k, head_dim)   one statistic per head
    inv_rms(q, k)                                           the per-token 1 / RMS alone
    partial_stats(x_slice, slice_index, num_slices)         split path, step 1
    apply_stats(x_slice, gamma_slice, stats, h_total)       split path, step 2
    partial_stats_qk / apply_stats_qk                       both steps for a query and a
                                                            key slice in one launch each

Rows are float32, bfloat16 or float8_e4m3fn (with bfloat16 weights); q and
k may be strided views, such as the column blocks of a packed QKV tensor.
"""
import ctypes
import os
import threading

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libqknorm.so")

F32, BF16, FP8_E4M3 = 0, 1, 2
OK = 0
ERR_NULL, ERR_SHAPE, ERR_SLICES, ERR_ALIGN, ERR_DTYPE, ERR_EPS, ERR_ALIAS, ERR_DEVICE, ERR_CONTEXT = (
    -1, -2, -3, -4, -5, -6, -7, -8, -9)

# Every symbol include/qknorm.h declares.
EXPORTS = ("qknorm_create", "qknorm_create_ex", "qknorm_destroy", "qknorm_forward",
           "qknorm_forward_headwise", "qknorm_inv_rms", "qknorm_partial_stats",
           "qknorm_apply_stats", "qknorm_partial_stats_qk", "qknorm_apply_stats_qk",
           "qknorm_status_string", "qknorm_max_width")


class Rows(ctypes.Structure):
    """qknorm_rows: one tensor's rows (device pointers, sizes in elements)."""
    _fields_ = [("x", ctypes.c_void_p), ("y", ctypes.c_void_p), ("width", ctypes.c_int64),
                ("x_stride", ctypes.c_int64), ("y_stride", ctypes.c_int64)]


class Options(ctypes.Structure):
    """qknorm_options: schedule overrides (0 = automatic)."""
    _fields_ = [("waves_per_row", ctypes.c_int), ("max_workgroups", ctypes.c_int),
                ("cached_rows", ctypes.c_int)]


class QKNormError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__("%s: %s (status %d)" % (where, status_string(status), status))


_lib = None
_lib_lock = threading.Lock()


def lib():
    """The loaded C library, with argument types declared. Raises if it has not
    been built (build it with attention_qk_norm_amd.build.build())."""
    global _lib
    with _lib_lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError("libqknorm.so is not built (expected at %s); run "
                                   "attention_qk_norm_amd.build.build()" % LIB_PATH)
            L = ctypes.CDLL(LIB_PATH)
            vp, i64, ci, cf = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
            L.qknorm_create.argtypes = [ctypes.POINTER(vp), ci]
            L.qknorm_create_ex.argtypes = [ctypes.POINTER(vp), ci, ctypes.POINTER(Options)]
            L.qknorm_destroy.argtypes = [vp]
            L.qknorm_forward.argtypes = [vp, ci, i64, ctypes.POINTER(Rows), ctypes.POINTER(Rows),
                                         vp, vp, cf, ci, vp]
            L.qknorm_forward_headwise.argtypes = [vp, ci, i64, ctypes.POINTER(Rows), ctypes.POINTER(Rows),
                                                  vp, vp, i64, cf, vp]
            L.qknorm_inv_rms.argtypes = [vp, ci, i64, ctypes.POINTER(Rows), ctypes.POINTER(Rows), cf, ci,
                                         vp, vp, vp]
            L.qknorm_partial_stats.argtypes = [vp, ci, i64, vp, i64, i64, ci, ci, vp, vp]
            L.qknorm_apply_stats.argtypes = [vp, ci, i64, ctypes.POINTER(Rows), vp, vp, ci, i64,
                                             cf, vp]
            L.qknorm_partial_stats_qk.argtypes = [vp, ci, i64, ctypes.POINTER(Rows), ctypes.POINTER(Rows),
                                                  ci, ci, vp, vp, vp]
            L.qknorm_apply_stats_qk.argtypes = [vp, ci, i64, ctypes.POINTER(Rows), ctypes.POINTER(Rows),
                                                vp, vp, vp, vp, ci, i64, i64, cf, vp]
            L.qknorm_status_string.argtypes = [ci]
            L.qknorm_status_string.restype = ctypes.c_char_p
            L.qknorm_max_width.argtypes = [ci]
            L.qknorm_max_width.restype = i64
            for name in ("qknorm_create", "qknorm_create_ex", "qknorm_destroy", "qknorm_forward",
                         "qknorm_forward_headwise", "qknorm_inv_rms", "qknorm_partial_stats",
                         "qknorm_apply_stats", "qknorm_partial_stats_qk", "qknorm_apply_stats_qk"):
                getattr(L, name).restype = ci
            _lib = L
        return _lib


def status_string(status):
    return lib().qknorm_status_string(int(status)).decode()


def max_width(dtype):
    return int(lib().qknorm_max_width(int(dtype)))


def _check(status, where):
    if status != OK:
        raise QKNormError(status, where)


class Context:
    """Owns a qknorm_ctx for one device (immutable, shareable by threads)."""

    def __init__(self, device=0, waves_per_row=0, max_workgroups=0, cached_rows=0):
        self.device = int(device)
        self.options = Options(int(waves_per_row), int(max_workgroups), int(cached_rows))
        h = ctypes.c_void_p()
        _check(lib().qknorm_create_ex(ctypes.byref(h), self.device, ctypes.byref(self.options)),
               "qknorm_create_ex")
        self.handle = h

    def close(self):
        if getattr(self, "handle", None) is not None and self.handle.value:
            lib().qknorm_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


_default = {}


def default_context(device=0):
    """One shared default Context per device index."""
    ctx = _default.get(device)
    if ctx is None:
        ctx = _default[device] = Context(device)
    return ctx


# ---- torch-facing wrappers (argument marshalling only) ----------------------

def _torch():
    import torch
    return torch


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float8_e4m3fn:
        return FP8_E4M3
    raise TypeError("qknorm supports float32, bfloat16 and float8_e4m3fn tensors, got %s" % t.dtype)


def gamma_dtype(row_dtype):
    """The weights' dtype for rows of `row_dtype`: bfloat16 for FP8 rows,
    else the rows' own dtype."""
    torch = _torch()
    return torch.bfloat16 if row_dtype == torch.float8_e4m3fn else row_dtype


def _rows_of(x, y):
    """Describe 2-D row tensors x (input) and y (output) as a Rows struct.
    The C ABI sees only pointers, so the output's shape and dtype are checked
    here: a smaller or differently typed y would be written past its end."""
    if x.dim() != 2 or (y is not None and y.dim() != 2):
        raise ValueError("rows must be 2-D [T, width] tensors")
    if y is not None and (tuple(y.shape) != tuple(x.shape) or y.dtype != x.dtype):
        raise ValueError("the output must have the input's shape %s and dtype %s, got %s %s"
                         % (tuple(x.shape), x.dtype, tuple(y.shape), y.dtype))
    if x.stride(1) != 1 or (y is not None and y.stride(1) != 1):
        raise ValueError("each row must be contiguous (stride 1 along the width)")
    yy = y if y is not None else x
    return Rows(x.data_ptr(), yy.data_ptr(), x.shape[1], x.stride(0) if x.shape[0] > 1 else x.shape[1],
                yy.stride(0) if yy.shape[0] > 1 else yy.shape[1])


def _on_one_gpu(*tensors):
    """Every tensor a call hands to the library must be GPU memory of one
    device: the kernels dereference the pointers on that device."""
    ts = [t for t in tensors if t is not None]
    dev = ts[0].device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU (device type 'cuda'), got %s" % dev)
    for t in ts[1:]:
        if t.device != dev:
            raise ValueError("all tensors of a call must be on %s, got one on %s" % (dev, t.device))


def _stream_of(t, stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return ctypes.c_void_p(stream.cuda_stream)


def _ctx_of(t, ctx):
    return ctx if ctx is not None else default_context(t.device.index or 0)


def _qk_rows(q, k, gamma_q, gamma_k, gamma_width, out_q, out_k):
    """Marshal the query and key tensors of a fused call: (dtype, T, rows of q,
    rows of k or None, y_q, y_k). gamma_width(x) is the weight count for rows x."""
    torch = _torch()
    dt = _dtype_code(q)
    T = q.shape[0]
    if out_q is None:
        out_q = torch.empty_like(q, memory_format=torch.contiguous_format)
    rq = _rows_of(q, out_q)
    rk = None
    if k is not None:
        if k.shape[0] != T:
            raise ValueError("q and k must have the same number of rows")
        if k.dtype != q.dtype:
            raise TypeError("q and k must share a dtype")
        if out_k is None:
            out_k = torch.empty_like(k, memory_format=torch.contiguous_format)
        rk = _rows_of(k, out_k)
    for g, x in ((gamma_q, q), (gamma_k, k)):
        if x is None:
            continue
        if g.dtype != gamma_dtype(x.dtype) or g.dim() != 1 or g.shape[0] != gamma_width(x) or \
                not g.is_contiguous():
            raise ValueError("gamma must be a contiguous 1-D %s tensor with %d weights"
                             % (gamma_dtype(x.dtype), gamma_width(x)))
    _on_one_gpu(q, out_q, gamma_q, k, out_k, gamma_k if k is not None else None)
    return dt, T, rq, rk, out_q, out_k


def forward(q, k, gamma_q, gamma_k, eps=1e-6, num_slices=1, out_q=None, out_k=None,
            ctx=None, stream=None):
    """Layerwise QK-Norm of q [T, Hq] and k [T, Hk] (k may be None) in one launch.

    Outputs are new tensors unless out_q / out_k are given; passing the input
    itself (out_q=q) normalises in place. Returns (y_q, y_k)."""
    dt, T, rq, rk, out_q, out_k = _qk_rows(q, k, gamma_q, gamma_k, lambda x: x.shape[1], out_q, out_k)
    c = _ctx_of(q, ctx)
    st = lib().qknorm_forward(c.handle, dt, T, ctypes.byref(rq),
                              ctypes.byref(rk) if rk is not None else None,
                              gamma_q.data_ptr(), gamma_k.data_ptr() if k is not None else None,
                              float(eps), int(num_slices), _stream_of(q, stream))
    _check(st, "qknorm_forward")
    return out_q, out_k


def forward_headwise(q, k, gamma_q, gamma_k, head_dim, eps=1e-6, out_q=None, out_k=None,
                     ctx=None, stream=None):
    """Headwise QK-Norm of q [T, Hq] and k [T, Hk] (k may be None) in one
    launch: every head of `head_dim` columns has its own statistic, and
    gamma_q / gamma_k hold `head_dim` weights shared by the heads of their
    tensor. Outputs as for forward(). Returns (y_q, y_k)."""
    dt, T, rq, rk, out_q, out_k = _qk_rows(q, k, gamma_q, gamma_k, lambda x: int(head_dim), out_q, out_k)
    c = _ctx_of(q, ctx)
    st = lib().qknorm_forward_headwise(c.handle, dt, T, ctypes.byref(rq),
                                       ctypes.byref(rk) if rk is not None else None,
                                       gamma_q.data_ptr(), gamma_k.data_ptr() if k is not None else None,
                                       int(head_dim), float(eps), _stream_of(q, stream))
    _check(st, "qknorm_forward_headwise")
    return out_q, out_k


def inv_rms(q, k=None, eps=1e-6, num_slices=1, out_q=None, out_k=None, ctx=None, stream=None):
    """Per-token inverse RMS 1 / sqrt(S / width + eps) of the rows of q
    [T, Hq] and k [T, Hk] (k may be None), in one launch: the factor
    forward() scales each row by, for a consumer that applies it itself.
    Returns (r_q, r_k), float32 [T] each (new tensors unless out_* given)."""
    torch = _torch()
    dt = _dtype_code(q)
    T = q.shape[0]
    rq = _rows_of(q, None)
    rk = None
    if k is not None:
        if k.shape[0] != T or k.dtype != q.dtype:
            raise ValueError("q and k must share T and dtype")
        rk = _rows_of(k, None)
    outs = []
    for o, x in ((out_q, q), (out_k, k)):
        if x is None:
            outs.append(None)
            continue
        if o is None:
            o = torch.empty(T, dtype=torch.float32, device=x.device)
        if o.dtype != torch.float32 or o.shape != (T,) or not o.is_contiguous():
            raise ValueError("inverse-RMS outputs are contiguous float32 [T] tensors")
        outs.append(o)
    _on_one_gpu(q, k, outs[0], outs[1])
    c = _ctx_of(q, ctx)
    st = lib().qknorm_inv_rms(c.handle, dt, T, ctypes.byref(rq), ctypes.byref(rk) if rk is not None else None,
                              float(eps), int(num_slices), outs[0].data_ptr(),
                              outs[1].data_ptr() if outs[1] is not None else None, _stream_of(q, stream))
    _check(st, "qknorm_inv_rms")
    return outs[0], outs[1]


def partial_stats(x_slice, slice_index, num_slices, stats=None, ctx=None, stream=None):
    """Sum of squares of each row of x_slice [T, w] into stats[slice_index]
    (stats is float32 [num_slices, T]; allocated when None). Returns stats."""
    torch = _torch()
    dt = _dtype_code(x_slice)
    T = x_slice.shape[0]
    if x_slice.dim() != 2 or x_slice.stride(1) != 1:
        raise ValueError("x_slice must be 2-D with contiguous rows")
    if stats is None:
        stats = torch.zeros((num_slices, T), dtype=torch.float32, device=x_slice.device)
    if stats.dtype != torch.float32 or stats.shape != (num_slices, T) or not stats.is_contiguous():
        raise ValueError("stats must be a contiguous float32 [num_slices, T] tensor")
    _on_one_gpu(x_slice, stats)
    c = _ctx_of(x_slice, ctx)
    st = lib().qknorm_partial_stats(c.handle, dt, T, x_slice.data_ptr(),
                                    x_slice.stride(0) if T > 1 else x_slice.shape[1],
                                    x_slice.shape[1], int(slice_index), int(num_slices),
                                    stats.data_ptr(), _stream_of(x_slice, stream))
    _check(st, "qknorm_partial_stats")
    return stats


def apply_stats(x_slice, gamma_slice, stats, h_total, eps=1e-6, out=None, ctx=None, stream=None):
    """Normalise the rows of x_slice [T, w] with the K partials in stats
    [K, T] and the full width h_total. Returns the output (out=x_slice: in place)."""
    torch = _torch()
    dt = _dtype_code(x_slice)
    T = x_slice.shape[0]
    if out is None:
        out = torch.empty_like(x_slice, memory_format=torch.contiguous_format)
    r = _rows_of(x_slice, out)
    if stats.dtype != torch.float32 or stats.dim() != 2 or stats.shape[1] != T or not stats.is_contiguous():
        raise ValueError("stats must be a contiguous float32 [K, T] tensor")
    if gamma_slice.dtype != gamma_dtype(x_slice.dtype) or gamma_slice.dim() != 1 or \
            gamma_slice.shape[0] != x_slice.shape[1] or not gamma_slice.is_contiguous():
        raise ValueError("gamma_slice must be a contiguous 1-D %s tensor with %d weights"
                         % (gamma_dtype(x_slice.dtype), x_slice.shape[1]))
    _on_one_gpu(x_slice, out, gamma_slice, stats)
    c = _ctx_of(x_slice, ctx)
    st = lib().qknorm_apply_stats(c.handle, dt, T, ctypes.byref(r), gamma_slice.data_ptr(),
                                  stats.data_ptr(), stats.shape[0], int(h_total), float(eps),
                                  _stream_of(x_slice, stream))
    _check(st, "qknorm_apply_stats")
    return out


def _stats_out(st, x, num_slices):
    torch = _torch()
    T = x.shape[0]
    if st is None:
        st = torch.zeros((num_slices, T), dtype=torch.float32, device=x.device)
    if st.dtype != torch.float32 or st.shape != (num_slices, T) or not st.is_contiguous():
        raise ValueError("stats must be a contiguous float32 [num_slices, T] tensor")
    return st


def partial_stats_qk(q_slice, k_slice, slice_index, num_slices, stats_q=None, stats_k=None, ctx=None,
                     stream=None):
    """partial_stats of a query slice and a key slice of the same T tokens in
    one launch (k_slice may be None). Returns (stats_q, stats_k)."""
    dt = _dtype_code(q_slice)
    T = q_slice.shape[0]
    rq = _rows_of(q_slice, None)
    rk = None
    if k_slice is not None:
        if k_slice.shape[0] != T or k_slice.dtype != q_slice.dtype:
            raise ValueError("q_slice and k_slice must share T and dtype")
        rk = _rows_of(k_slice, None)
    stats_q = _stats_out(stats_q, q_slice, num_slices)
    stats_k = _stats_out(stats_k, k_slice, num_slices) if k_slice is not None else None
    _on_one_gpu(q_slice, k_slice, stats_q, stats_k)
    c = _ctx_of(q_slice, ctx)
    st = lib().qknorm_partial_stats_qk(c.handle, dt, T, ctypes.byref(rq),
                                       ctypes.byref(rk) if rk is not None else None,
                                       int(slice_index), int(num_slices), stats_q.data_ptr(),
                                       stats_k.data_ptr() if stats_k is not None else None,
                                       _stream_of(q_slice, stream))
    _check(st, "qknorm_partial_stats_qk")
    return stats_q, stats_k


def apply_stats_qk(q_slice, k_slice, gamma_q_slice, gamma_k_slice, stats_q, stats_k, hq_total, hk_total,
                   eps=1e-6, out_q=None, out_k=None, ctx=None, stream=None):
    """apply_stats of a query slice and a key slice of the same T tokens in
    one launch (k_slice may be None; out_*=x_slice: in place). Returns
    (y_q, y_k)."""
    torch = _torch()
    dt, T, rq, rk, out_q, out_k = _qk_rows(q_slice, k_slice, gamma_q_slice, gamma_k_slice,
                                           lambda x: x.shape[1], out_q, out_k)
    K = stats_q.shape[0] if stats_q.dim() == 2 else -1
    for st_, x in ((stats_q, q_slice), (stats_k, k_slice)):
        if x is None:
            continue
        if st_.dtype != torch.float32 or st_.dim() != 2 or st_.shape != (K, T) or not st_.is_contiguous():
            raise ValueError("stats must be contiguous float32 [K, T] tensors of one K")
    _on_one_gpu(q_slice, stats_q, stats_k if k_slice is not None else None)
    c = _ctx_of(q_slice, ctx)
    st = lib().qknorm_apply_stats_qk(c.handle, dt, T, ctypes.byref(rq), ctypes.byref(rk) if rk is not None else None,
                                     gamma_q_slice.data_ptr(),
                                     gamma_k_slice.data_ptr() if k_slice is not None else None,
                                     stats_q.data_ptr(), stats_k.data_ptr() if k_slice is not None else None,
                                     K, int(hq_total), int(hk_total) if k_slice is not None else 0, float(eps),
                                     _stream_of(q_slice, stream))
    _check(st, "qknorm_apply_stats_qk")
    return out_q, out_k
