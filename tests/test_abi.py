"""The C ABI without a GPU: the library loads, exports what include/qknorm.h
declares, and rejects every invalid argument on the host before touching any
pointer (validation precedes the context check, so ctx = NULL is enough)."""
import ctypes
import os
import re

import pytest

import attention_qk_norm_amd as qk
from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "qknorm.h")
A = 0x7F0000000000  # fake, 16-byte aligned device addresses: never dereferenced
MB = 1 << 20


@pytest.fixture(scope="module")
def L():
    return qk.lib()


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|int64_t|const char \*)\s*\*?\s*(qknorm_\w+)\s*\(",
                                 text, re.M)))


def header_enum(name):
    text = open(HEADER).read()
    return int(re.search(r"\b%s\s*=\s*(-?\d+)" % name, text).group(1))


def test_exports_every_declared_symbol(L):
    declared = header_functions()
    assert sorted(qk.EXPORTS) == declared
    for name in declared:
        assert hasattr(L, name), name


def test_binding_constants_match_header():
    for pyname, cname in (("F32", "QKNORM_F32"), ("BF16", "QKNORM_BF16"), ("FP8_E4M3", "QKNORM_FP8_E4M3"),
                          ("OK", "QKNORM_OK"),
                          ("ERR_NULL", "QKNORM_ERR_NULL"), ("ERR_SHAPE", "QKNORM_ERR_SHAPE"),
                          ("ERR_SLICES", "QKNORM_ERR_SLICES"), ("ERR_ALIGN", "QKNORM_ERR_ALIGN"),
                          ("ERR_DTYPE", "QKNORM_ERR_DTYPE"), ("ERR_EPS", "QKNORM_ERR_EPS"),
                          ("ERR_ALIAS", "QKNORM_ERR_ALIAS"), ("ERR_DEVICE", "QKNORM_ERR_DEVICE"),
                          ("ERR_CONTEXT", "QKNORM_ERR_CONTEXT")):
        assert getattr(qk, pyname) == header_enum(cname), pyname


def test_status_strings():
    codes = [qk.OK, qk.ERR_NULL, qk.ERR_SHAPE, qk.ERR_SLICES, qk.ERR_ALIGN, qk.ERR_DTYPE,
             qk.ERR_EPS, qk.ERR_ALIAS, qk.ERR_DEVICE, qk.ERR_CONTEXT]
    texts = [qk.status_string(c) for c in codes]
    assert len(set(texts)) == len(codes)
    assert qk.status_string(12345) == "unknown status"


def test_max_width():
    assert qk.max_width(qk.BF16) == 65536
    assert qk.max_width(qk.F32) == 32768
    assert qk.max_width(qk.FP8_E4M3) == 65536
    assert qk.max_width(7) == 0


def _fwd(L, dtype=qk.BF16, T=64, q=None, k="default", gq=A + 60 * MB, gk=A + 61 * MB,
         eps=1e-6, K=1):
    if q is None:
        q = qk.Rows(A, A + 8 * MB, 4096, 4096, 4096)
    if k == "default":
        k = qk.Rows(A + 16 * MB, A + 24 * MB, 1024, 1024, 1024)
    return L.qknorm_forward(None, dtype, T, ctypes.byref(q), ctypes.byref(k) if k is not None else None,
                            gq, gk, eps, K, None)


def test_forward_valid_arguments_reach_the_context_check(L):
    assert _fwd(L) == qk.ERR_CONTEXT
    assert _fwd(L, k=None) == qk.ERR_CONTEXT
    assert _fwd(L, dtype=qk.F32) == qk.ERR_CONTEXT


def test_forward_empty_is_ok(L):
    assert _fwd(L, T=0) == qk.OK
    assert _fwd(L, T=0, q=qk.Rows(0, 0, 0, 0, 0)) == qk.OK  # nothing to check, nothing to do


def test_forward_rejects(L):
    R = qk.Rows
    cases = [
        (dict(dtype=3), qk.ERR_DTYPE),
        (dict(T=-1), qk.ERR_SHAPE),
        (dict(T=1 << 31), qk.ERR_SHAPE),
        (dict(q=R(0, A + 8 * MB, 4096, 4096, 4096)), qk.ERR_NULL),
        (dict(q=R(A, 0, 4096, 4096, 4096)), qk.ERR_NULL),
        (dict(gq=None), qk.ERR_NULL),
        (dict(gk=None), qk.ERR_NULL),
        (dict(q=R(A, A + 8 * MB, 0, 4096, 4096)), qk.ERR_SHAPE),
        (dict(q=R(A, A + 8 * MB, 4096, 4088, 4096)), qk.ERR_SHAPE),
        (dict(q=R(A, A + 8 * MB, 4096, 4096, 4000)), qk.ERR_SHAPE),
        (dict(q=R(A, A + 8 * MB, 65536 + 8, 70000, 70000)), qk.ERR_SHAPE),
        (dict(q=R(A, A + 8 * MB, 4092, 4096, 4096)), qk.ERR_ALIGN),  # not whole bf16 vectors
        (dict(q=R(A, A + 8 * MB, 4096, 4100, 4096)), qk.ERR_ALIGN),
        (dict(q=R(A + 2, A + 8 * MB, 4096, 4096, 4096)), qk.ERR_ALIGN),
        (dict(q=R(A, A + 8 * MB + 8, 4096, 4096, 4096)), qk.ERR_ALIGN),
        (dict(gq=A + 60 * MB + 4), qk.ERR_ALIGN),
        (dict(K=0), qk.ERR_SLICES),
        (dict(K=65), qk.ERR_SLICES),
        (dict(K=3), qk.ERR_SLICES),  # 4096 not cut evenly into 3
        (dict(K=256), qk.ERR_SLICES),
        (dict(K=1024), qk.ERR_SLICES),
        (dict(eps=-1e-6), qk.ERR_EPS),
        (dict(eps=float("nan")), qk.ERR_EPS),
        (dict(eps=float("inf")), qk.ERR_EPS),
        # output overlapping its own input without being it
        (dict(q=R(A, A + 16, 4096, 4096, 4096)), qk.ERR_ALIAS),
        # in place needs the same stride
        (dict(q=R(A, A, 4096, 4096, 8192)), qk.ERR_ALIAS),
        # q's output over k's input, or over a gamma
        (dict(q=R(A, A + 16 * MB, 4096, 4096, 4096)), qk.ERR_ALIAS),
        (dict(q=R(A, A + 60 * MB, 4096, 4096, 4096)), qk.ERR_ALIAS),
    ]
    for kw, want in cases:
        assert _fwd(L, **kw) == want, kw


def test_forward_slice_width_must_be_whole_vectors(L):
    R = qk.Rows
    # bf16 4096 / 64 = 64 elements = 8 vectors; fp32 256 / 64 = 4 elements = 1 vector
    assert _fwd(L, K=64) == qk.ERR_CONTEXT
    q, k = R(A, A + 8 * MB, 256, 256, 256), R(A + 16 * MB, A + 24 * MB, 256, 256, 256)
    assert _fwd(L, dtype=qk.F32, q=q, k=k, K=64) == qk.ERR_CONTEXT
    # bf16 96 / 12 = 8 elements: one vector; 96 / 24 = 4 elements: half a vector
    q = R(A, A + 8 * MB, 96, 96, 96)
    assert _fwd(L, q=q, k=None, K=12) == qk.ERR_CONTEXT
    assert _fwd(L, q=q, k=None, K=24) == qk.ERR_SLICES
    # fp32 8 / 8 = 1 element
    q = R(A, A + 8 * MB, 8, 8, 8)
    assert _fwd(L, dtype=qk.F32, q=q, k=None, K=2) == qk.ERR_CONTEXT
    assert _fwd(L, dtype=qk.F32, q=q, k=None, K=8) == qk.ERR_SLICES


def test_fp8_rows(L):
    """FP8 rows move 16 elements per vector; their weights are bf16, so a
    weight vector is twice the row's bytes."""
    R = qk.Rows
    q, k = R(A, A + 8 * MB, 4096, 4096, 4096), R(A + 16 * MB, A + 24 * MB, 1024, 1024, 1024)
    assert _fwd(L, dtype=qk.FP8_E4M3, q=q, k=k, K=8) == qk.ERR_CONTEXT
    # 4096 / 512 = 8 fp8 elements: half a vector
    assert _fwd(L, dtype=qk.FP8_E4M3, q=q, k=k, K=512) == qk.ERR_SLICES
    assert _fwd(L, dtype=qk.FP8_E4M3, q=R(A, A + 8 * MB, 4104, 4104, 4104), k=k) == qk.ERR_ALIGN
    assert _fwd(L, dtype=qk.FP8_E4M3, q=R(A, A + 8 * MB, 65536, 65536, 65536), k=None) == qk.ERR_CONTEXT
    assert _fwd(L, dtype=qk.FP8_E4M3, q=R(A, A + 8 * MB, 65536 + 16, 65552, 65552), k=None) == qk.ERR_SHAPE
    # the query output placed right after 4096 bf16 weights (8 KiB) is clear
    # of them; 4 KiB after them (the fp8 row length) is not
    q2 = R(A, A + 60 * MB + 8192, 4096, 4096, 4096)
    assert _fwd(L, dtype=qk.FP8_E4M3, q=q2, k=None) == qk.ERR_CONTEXT
    q3 = R(A, A + 60 * MB + 4096, 4096, 4096, 4096)
    assert _fwd(L, dtype=qk.FP8_E4M3, q=q3, k=None) == qk.ERR_ALIAS
    # headwise: heads are a power of two of 16-byte vectors, 16 ... 1024 fp8 columns
    for D, want in ((16, qk.ERR_CONTEXT), (128, qk.ERR_CONTEXT), (1024, qk.ERR_CONTEXT), (8, qk.ERR_SLICES),
                    (2048, qk.ERR_SLICES), (48, qk.ERR_SLICES)):
        assert _head(L, dtype=qk.FP8_E4M3, D=D) == want, D


def test_forward_in_place_and_packed_qkv_are_accepted(L):
    R = qk.Rows
    # in place, same stride
    assert _fwd(L, q=R(A, A, 4096, 4096, 4096), k=R(A + 16 * MB, A + 16 * MB, 1024, 1024, 1024)) \
        == qk.ERR_CONTEXT
    # query and key columns of one packed [T, Hq + Hk + Hv] buffer, normalised in place
    H = 4096 + 1024 + 1024
    q = R(A, A, 4096, H, H)
    k = R(A + 4096 * 2, A + 4096 * 2, 1024, H, H)
    assert _fwd(L, q=q, k=k) == qk.ERR_CONTEXT
    # ...but key columns that reach into the query columns are refused
    k_bad = R(A + 4000 * 2, A + 4000 * 2, 1024, H, H)
    assert _fwd(L, q=q, k=k_bad) == qk.ERR_ALIAS


def _head(L, dtype=qk.BF16, T=64, q=None, k="default", gq=A + 60 * MB, gk=A + 61 * MB, D=128, eps=1e-6):
    if q is None:
        q = qk.Rows(A, A + 8 * MB, 4096, 4096, 4096)
    if k == "default":
        k = qk.Rows(A + 16 * MB, A + 24 * MB, 1024, 1024, 1024)
    return L.qknorm_forward_headwise(None, dtype, T, ctypes.byref(q),
                                     ctypes.byref(k) if k is not None else None, gq, gk, D, eps, None)


def test_headwise_validation(L):
    R = qk.Rows
    assert _head(L) == qk.ERR_CONTEXT
    assert _head(L, k=None) == qk.ERR_CONTEXT
    assert _head(L, T=0) == qk.OK
    # valid head widths: a power of two of 16-byte vectors, at most 64 of them
    for dtype, D in ((qk.BF16, 8), (qk.BF16, 64), (qk.BF16, 256), (qk.BF16, 512),
                     (qk.F32, 4), (qk.F32, 128), (qk.F32, 256)):
        assert _head(L, dtype=dtype, D=D) == qk.ERR_CONTEXT, (dtype, D)
    for dtype, D in ((qk.BF16, 0), (qk.BF16, -128), (qk.BF16, 4), (qk.BF16, 96), (qk.BF16, 1024),
                     (qk.BF16, 2048), (qk.F32, 2), (qk.F32, 512), (qk.F32, 192)):
        assert _head(L, dtype=dtype, D=D) == qk.ERR_SLICES, (dtype, D)
    # every width must be whole heads: 1024 / 512 is, 1152 / 256 is not
    assert _head(L, D=512) == qk.ERR_CONTEXT
    assert _head(L, D=256, k=R(A + 16 * MB, A + 24 * MB, 1152, 1152, 1152)) == qk.ERR_SLICES
    cases = [
        (dict(dtype=3), qk.ERR_DTYPE),
        (dict(T=-1), qk.ERR_SHAPE),
        (dict(gq=None), qk.ERR_NULL),
        (dict(q=R(A, A + 8 * MB, 4096, 4088, 4096)), qk.ERR_SHAPE),
        (dict(q=R(A + 2, A + 8 * MB, 4096, 4096, 4096)), qk.ERR_ALIGN),
        (dict(eps=-1.0), qk.ERR_EPS),
        (dict(q=R(A, A + 16, 4096, 4096, 4096)), qk.ERR_ALIAS),
        # gamma holds head_dim weights: an output starting just past 128 bf16
        # weights does not overlap them, one starting inside does
        (dict(gq=A + 8 * MB - 256), qk.ERR_CONTEXT),
        (dict(gq=A + 8 * MB - 240), qk.ERR_ALIAS),
    ]
    for kw, want in cases:
        assert _head(L, **kw) == want, kw


def _rinv(L, dtype=qk.BF16, T=64, q=None, k="default", rq=A + 40 * MB, rk=A + 41 * MB, eps=1e-6, K=1):
    if q is None:
        q = qk.Rows(A, 0, 4096, 4096, 4096)
    if k == "default":
        k = qk.Rows(A + 16 * MB, 0, 1024, 1024, 1024)
    return L.qknorm_inv_rms(None, dtype, T, ctypes.byref(q), ctypes.byref(k) if k is not None else None,
                            eps, K, rq, rk, None)


def test_inv_rms_validation(L):
    R = qk.Rows
    assert _rinv(L) == qk.ERR_CONTEXT
    assert _rinv(L, k=None, rk=None) == qk.ERR_CONTEXT
    assert _rinv(L, K=64) == qk.ERR_CONTEXT
    assert _rinv(L, T=0) == qk.OK
    cases = [
        (dict(dtype=5), qk.ERR_DTYPE),
        (dict(T=-2), qk.ERR_SHAPE),
        (dict(rq=None), qk.ERR_NULL),
        (dict(rk=None), qk.ERR_NULL),
        (dict(q=R(0, 0, 4096, 4096, 4096)), qk.ERR_NULL),
        (dict(q=R(A, 0, 4096, 4000, 4096)), qk.ERR_SHAPE),
        (dict(q=R(A + 8, 0, 4096, 4096, 4096)), qk.ERR_ALIGN),
        (dict(rq=A + 40 * MB + 2), qk.ERR_ALIGN),
        (dict(K=3), qk.ERR_SLICES),
        (dict(eps=float("nan")), qk.ERR_EPS),
        # an output inside the query rows, inside the key rows, or over the other output
        (dict(rq=A + 1024), qk.ERR_ALIAS),
        (dict(rk=A + 16 * MB + 4), qk.ERR_ALIAS),
        (dict(rk=A + 40 * MB + 64), qk.ERR_ALIAS),
        (dict(rk=A + 40 * MB + 256), qk.ERR_CONTEXT),  # just past T = 64 floats
    ]
    for kw, want in cases:
        assert _rinv(L, **kw) == want, kw


def _stats(L, dtype=qk.BF16, T=256, x=A, stride=5120, w=1280, s=0, K=4, st=A + 64 * MB):
    return L.qknorm_partial_stats(None, dtype, T, x, stride, w, s, K, st, None)


def test_partial_stats_validation(L):
    assert _stats(L) == qk.ERR_CONTEXT
    assert _stats(L, T=0) == qk.OK
    for kw, want in [
        (dict(dtype=9), qk.ERR_DTYPE), (dict(T=-3), qk.ERR_SHAPE),
        (dict(x=None), qk.ERR_NULL), (dict(st=None), qk.ERR_NULL),
        (dict(w=0), qk.ERR_SHAPE), (dict(stride=1000), qk.ERR_SHAPE),
        (dict(w=1276, stride=5120), qk.ERR_ALIGN), (dict(x=A + 8), qk.ERR_ALIGN),
        (dict(st=A + 64 * MB + 2), qk.ERR_ALIGN),
        (dict(s=4), qk.ERR_SLICES), (dict(s=-1), qk.ERR_SLICES), (dict(K=0), qk.ERR_SLICES),
        (dict(K=65, s=0), qk.ERR_SLICES),
        (dict(st=A + 100), qk.ERR_ALIAS),
    ]:
        assert _stats(L, **kw) == want, kw
    # stats rows of other slices may sit anywhere; only row s must miss x
    assert _stats(L, st=A + 64 * MB + 4) == qk.ERR_CONTEXT


def _apply(L, dtype=qk.BF16, T=256, r=None, g=A + 60 * MB, st=A + 64 * MB, K=4, h=5120, eps=1e-6):
    if r is None:
        r = qk.Rows(A, A + 8 * MB, 1280, 5120, 1280)
    return L.qknorm_apply_stats(None, dtype, T, ctypes.byref(r), g, st, K, h, eps, None)


def test_apply_stats_validation(L):
    R = qk.Rows
    assert _apply(L) == qk.ERR_CONTEXT
    assert _apply(L, r=R(A, A, 1280, 5120, 5120)) == qk.ERR_CONTEXT  # in place
    assert _apply(L, T=0) == qk.OK
    for kw, want in [
        (dict(dtype=-1), qk.ERR_DTYPE), (dict(T=-1), qk.ERR_SHAPE),
        (dict(st=None), qk.ERR_NULL), (dict(g=None), qk.ERR_NULL),
        (dict(r=R(A, None, 1280, 5120, 1280)), qk.ERR_NULL),
        (dict(h=1000), qk.ERR_SHAPE), (dict(h=(1 << 24) + 8), qk.ERR_SHAPE),
        (dict(r=R(A, A + 8 * MB, 1280, 1000, 1280)), qk.ERR_SHAPE),
        (dict(st=A + 64 * MB + 1), qk.ERR_ALIGN),
        (dict(g=A + 60 * MB + 8), qk.ERR_ALIGN),
        (dict(K=0), qk.ERR_SLICES), (dict(K=65), qk.ERR_SLICES),
        (dict(eps=-0.5), qk.ERR_EPS),
        (dict(r=R(A, A, 1280, 5120, 2560)), qk.ERR_ALIAS),
        (dict(r=R(A, A + 64 * MB, 1280, 5120, 1280)), qk.ERR_ALIAS),  # output over stats
        (dict(r=R(A, A + 60 * MB, 1280, 5120, 1280)), qk.ERR_ALIAS),  # output over gamma
    ]:
        assert _apply(L, **kw) == want, kw


def _stats_qk(L, dtype=qk.BF16, T=256, q="default", k="default", s=1, K=4, sq=A + 64 * MB, sk=A + 65 * MB):
    # slice 1 of 4 of a packed [T, 5120 + 1024] buffer: query columns 1280-2559, key columns 5376-5631
    if q == "default":
        q = qk.Rows(A + 2 * 1280, None, 1280, 6144, 1280)
    if k == "default":
        k = qk.Rows(A + 2 * (5120 + 256), None, 256, 6144, 256)
    return L.qknorm_partial_stats_qk(None, dtype, T, ctypes.byref(q) if q is not None else None,
                                     ctypes.byref(k) if k is not None else None, s, K, sq, sk, None)


def test_partial_stats_qk_validation(L):
    R = qk.Rows
    assert _stats_qk(L) == qk.ERR_CONTEXT
    assert _stats_qk(L, k=None) == qk.ERR_CONTEXT
    assert _stats_qk(L, k=None, sk=None) == qk.ERR_CONTEXT  # stats_k unused without k
    assert _stats_qk(L, T=0) == qk.OK
    for kw, want in [
        (dict(dtype=9), qk.ERR_DTYPE), (dict(T=-3), qk.ERR_SHAPE),
        (dict(q=None), qk.ERR_NULL), (dict(sq=None), qk.ERR_NULL), (dict(sk=None), qk.ERR_NULL),
        (dict(q=R(None, None, 1280, 6144, 1280)), qk.ERR_NULL),
        (dict(q=R(A, None, 0, 6144, 0)), qk.ERR_SHAPE), (dict(k=R(A, None, 256, 100, 256)), qk.ERR_SHAPE),
        (dict(k=R(A + 8, None, 256, 6144, 256)), qk.ERR_ALIGN), (dict(sk=A + 65 * MB + 2), qk.ERR_ALIGN),
        (dict(k=R(A, None, 252, 6144, 252)), qk.ERR_ALIGN),
        (dict(s=4), qk.ERR_SLICES), (dict(s=-1), qk.ERR_SLICES), (dict(K=0), qk.ERR_SLICES),
        (dict(sq=A + 2 * 1280 + 100 - 256 * 4), qk.ERR_ALIAS),  # row 1 of stats_q over the rows
        (dict(sk=A + 64 * MB), qk.ERR_ALIAS),               # the two written rows coincide
    ]:
        assert _stats_qk(L, **kw) == want, kw
    # different rows of one [2][K][T] block are fine
    assert _stats_qk(L, sk=A + 64 * MB + 4 * 256 * 4) == qk.ERR_CONTEXT


def _apply_qk(L, dtype=qk.BF16, T=256, q="default", k="default", gq=A + 60 * MB, gk=A + 61 * MB,
              sq=A + 64 * MB, sk=A + 65 * MB, K=4, hq=5120, hk=1024, eps=1e-6):
    if q == "default":
        q = qk.Rows(A, A + 8 * MB, 1280, 5120, 1280)
    if k == "default":
        k = qk.Rows(A + 16 * MB, A + 24 * MB, 256, 1024, 256)
    return L.qknorm_apply_stats_qk(None, dtype, T, ctypes.byref(q) if q is not None else None,
                                   ctypes.byref(k) if k is not None else None, gq, gk, sq, sk, K, hq, hk,
                                   eps, None)


def test_apply_stats_qk_validation(L):
    R = qk.Rows
    assert _apply_qk(L) == qk.ERR_CONTEXT
    assert _apply_qk(L, k=None, gk=None, sk=None) == qk.ERR_CONTEXT
    assert _apply_qk(L, q=R(A, A, 1280, 5120, 5120), k=R(A + 16 * MB, A + 16 * MB, 256, 1024, 1024)) == \
        qk.ERR_CONTEXT  # both in place
    assert _apply_qk(L, T=0) == qk.OK
    for kw, want in [
        (dict(dtype=-1), qk.ERR_DTYPE), (dict(T=-1), qk.ERR_SHAPE),
        (dict(q=None), qk.ERR_NULL), (dict(sq=None), qk.ERR_NULL), (dict(sk=None), qk.ERR_NULL),
        (dict(gk=None), qk.ERR_NULL), (dict(k=R(A + 16 * MB, None, 256, 1024, 256)), qk.ERR_NULL),
        (dict(hq=1000), qk.ERR_SHAPE), (dict(hk=128), qk.ERR_SHAPE), (dict(hk=(1 << 24) + 8), qk.ERR_SHAPE),
        (dict(sk=A + 65 * MB + 1), qk.ERR_ALIGN), (dict(gk=A + 61 * MB + 8), qk.ERR_ALIGN),
        (dict(K=0), qk.ERR_SLICES), (dict(K=65), qk.ERR_SLICES),
        (dict(eps=float("nan")), qk.ERR_EPS),
        (dict(k=R(A + 16 * MB, A + 65 * MB, 256, 1024, 256)), qk.ERR_ALIAS),   # y_k over stats_k
        (dict(k=R(A + 16 * MB, A + 64 * MB, 256, 1024, 256)), qk.ERR_ALIAS),   # y_k over stats_q
        (dict(k=R(A + 16 * MB, A + 60 * MB, 256, 1024, 256)), qk.ERR_ALIAS),   # y_k over gamma_q
        (dict(k=R(A + 16 * MB, A + 1024, 256, 1024, 256)), qk.ERR_ALIAS),      # y_k over x_q
        (dict(k=R(A + 16 * MB, A + 8 * MB, 256, 1024, 256)), qk.ERR_ALIAS),    # y_k over y_q
    ]:
        assert _apply_qk(L, **kw) == want, kw


def test_create_validation(L):
    h = ctypes.c_void_p()
    assert L.qknorm_create(None, 0) == qk.ERR_NULL
    assert L.qknorm_create_ex(ctypes.byref(h), 0, ctypes.byref(qk.Options(3, 0, 0))) == qk.ERR_SHAPE
    assert L.qknorm_create_ex(ctypes.byref(h), 0, ctypes.byref(qk.Options(0, -1, 0))) == qk.ERR_SHAPE
    assert L.qknorm_create_ex(ctypes.byref(h), 0, ctypes.byref(qk.Options(0, 0, 2))) == qk.ERR_SHAPE
    assert L.qknorm_create(ctypes.byref(h), -1) == qk.ERR_DEVICE
    assert L.qknorm_destroy(None) == qk.OK


def test_no_device_means_loud_failure():
    """Without a gfx950 device the product path raises; it never computes on
    the CPU."""
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present")
    h = ctypes.c_void_p()
    assert qk.lib().qknorm_create(ctypes.byref(h), 0) == qk.ERR_DEVICE
    with pytest.raises(qk.QKNormError) as e:
        qk.Context(0)
    assert e.value.status == qk.ERR_DEVICE
    x = torch.zeros(4, 256)
    with pytest.raises(ValueError, match="GPU"):
        qk.forward(x, x, torch.ones(256), torch.ones(256))


def test_binding_checks_what_the_c_abi_cannot_see():
    """The C ABI takes bare pointers, so the binding checks sizes and types
    of the caller's outputs and weights before any call: a too-small or
    differently typed output, or a short weight vector, would be written or
    read past its end. CPU tensors pass these checks and then fail the
    device check, so no case here reaches the library."""
    import torch
    bf = torch.bfloat16
    q, k = torch.zeros(8, 256, dtype=bf), torch.zeros(8, 64, dtype=bf)
    gq, gk = torch.ones(256, dtype=bf), torch.ones(64, dtype=bf)
    for kw, msg in [
        (dict(out_q=torch.zeros(1, 256, dtype=bf)), "shape"),          # one row for T rows
        (dict(out_k=torch.zeros(8, 32, dtype=bf)), "shape"),
        (dict(out_q=torch.zeros(8, 256, dtype=torch.float32)), "dtype"),
        (dict(gamma_q=torch.ones(128, dtype=bf)), "weights"),          # short weights
        (dict(gamma_k=torch.ones(64, dtype=torch.float32)), "weights"),
        (dict(), "GPU"),                                               # all valid, but host memory
    ]:
        args = dict(gamma_q=gq, gamma_k=gk)
        args.update(kw)
        with pytest.raises(ValueError, match=msg):
            qk.forward(q, k, args.pop("gamma_q"), args.pop("gamma_k"), **args)
    with pytest.raises(ValueError, match="shape"):
        qk.forward_headwise(q, k, torch.ones(64, dtype=bf), torch.ones(64, dtype=bf), 64,
                            out_q=torch.zeros(4, 256, dtype=bf))
    with pytest.raises(ValueError, match="weights"):
        qk.forward_headwise(q, k, torch.ones(32, dtype=bf), torch.ones(64, dtype=bf), 64)
    with pytest.raises(ValueError, match="float32"):
        qk.inv_rms(q, k, out_q=torch.zeros(4, dtype=torch.float32))
    with pytest.raises(ValueError, match="GPU"):
        qk.inv_rms(q, k)
    xs = q[:, :64]
    st = torch.zeros(4, 8, dtype=torch.float32)
    with pytest.raises(ValueError, match="stats"):
        qk.partial_stats(xs, 0, 4, stats=torch.zeros(4, 4, dtype=torch.float32))
    with pytest.raises(ValueError, match="GPU"):
        qk.partial_stats(xs, 0, 4, stats=st)
    with pytest.raises(ValueError, match="64 weights"):
        qk.apply_stats(xs, torch.ones(32, dtype=bf), st, 256)     # short gamma_slice
    with pytest.raises(ValueError, match="shape"):
        qk.apply_stats(xs, torch.ones(64, dtype=bf), st, 256, out=torch.zeros(8, 32, dtype=bf))
    with pytest.raises(ValueError, match="stats"):
        qk.apply_stats(xs, torch.ones(64, dtype=bf), torch.zeros(4, 7, dtype=torch.float32), 256)
    with pytest.raises(ValueError, match="GPU"):
        qk.apply_stats(xs, torch.ones(64, dtype=bf), st, 256)
