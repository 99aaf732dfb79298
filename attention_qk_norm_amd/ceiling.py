"""ctypes binding of libqkceil (include/qkceil.h): the streaming copy,
read-only, write-only and empty kernels the benchmark times beside the
QK-Norm kernels as the practical bandwidth ceiling. Measurement only; no
part of the normalisation runs here."""
import ctypes
import os
import threading

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libqkceil.so")

OK, ERR_NULL, ERR_SIZE, ERR_ALIGN, ERR_CONFIG, ERR_DEVICE = 0, -1, -2, -3, -4, -5
EXPORTS = ("qkceil_copy", "qkceil_read", "qkceil_write", "qkceil_empty", "qkceil_clock")
VECTORS_PER_LANE = (1, 2, 4, 8)

_lib = None
_lock = threading.Lock()


def lib():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError("libqkceil.so is not built (expected at %s); run "
                                   "attention_qk_norm_amd.build.build_ceiling()" % LIB_PATH)
            L = ctypes.CDLL(LIB_PATH)
            vp, u64, ci, cu = ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int, ctypes.c_uint
            L.qkceil_copy.argtypes = [vp, vp, u64, ci, vp]
            L.qkceil_read.argtypes = [vp, u64, ci, vp, vp]
            L.qkceil_write.argtypes = [vp, u64, ci, vp]
            L.qkceil_empty.argtypes = [cu, vp]
            L.qkceil_clock.argtypes = [vp, vp]
            for name in EXPORTS:
                getattr(L, name).restype = ci
            _lib = L
        return _lib


def _check(status, where):
    if status != OK:
        raise RuntimeError("%s failed with status %d" % (where, status))


def copy(src_ptr, dst_ptr, nbytes, vectors_per_lane, stream_ptr):
    _check(lib().qkceil_copy(src_ptr, dst_ptr, nbytes, vectors_per_lane, stream_ptr), "qkceil_copy")


def read(src_ptr, nbytes, vectors_per_lane, sink_ptr, stream_ptr):
    _check(lib().qkceil_read(src_ptr, nbytes, vectors_per_lane, sink_ptr, stream_ptr), "qkceil_read")


def write(dst_ptr, nbytes, vectors_per_lane, stream_ptr):
    _check(lib().qkceil_write(dst_ptr, nbytes, vectors_per_lane, stream_ptr), "qkceil_write")


def empty(workgroups, stream_ptr):
    _check(lib().qkceil_empty(workgroups, stream_ptr), "qkceil_empty")


def clock(out_ptr, stream_ptr):
    """Queue a sample of the shader clock into two uint64 at out_ptr."""
    _check(lib().qkceil_clock(out_ptr, stream_ptr), "qkceil_clock")
