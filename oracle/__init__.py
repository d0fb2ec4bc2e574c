"""CPU oracle for single-precision GEMM — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The GPU library (``precision_gemm_amd``)
never imports it and shares no code with it; this package never imports the
GPU library.

It wraps the plain C triple loop in ``sgemm_oracle.c`` (the GEMM definition of
"From 1% to 94% of cuBLAS, one kernel at a time", accumulated in double
precision) and provides the acceptance check

    |C_gpu - ref| <= 2e-6 * max(K, 1) * (|alpha| * S + |beta| * |C_in|)

elementwise, where S = sum_k |opA[i,k]| * |opB[k,j]|. A NaN or Inf in the GPU
result always fails.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

from . import build as _build

_lib = None
_i64 = ctypes.c_longlong
_dp = ctypes.POINTER(ctypes.c_double)
_fp = ctypes.POINTER(ctypes.c_float)
_ip = ctypes.POINTER(ctypes.c_longlong)

TOL_PER_K = 2e-6


def _load():
    global _lib
    if _lib is None:
        path = _build.LIB
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_build.SRC):
            _build.build()
        lib = ctypes.CDLL(path)
        lib.oracle_sgemm_rows.restype = ctypes.c_int
        lib.oracle_sgemm_rows.argtypes = [
            ctypes.c_int, ctypes.c_int, _i64, _i64, _i64,
            ctypes.c_double, _fp, _i64, _i64,
            _fp, _i64, _i64,
            ctypes.c_double, _fp, _i64, _i64,
            _i64, _i64, _i64, _i64,
            _dp, _dp, ctypes.c_int]
        lib.oracle_sgemm_elements.restype = None
        lib.oracle_sgemm_elements.argtypes = [
            ctypes.c_int, ctypes.c_int, _i64,
            ctypes.c_double, _fp, _i64, _i64,
            _fp, _i64, _i64,
            ctypes.c_double, _fp, _i64, _i64,
            _i64, _ip, _ip, _ip, _dp, _dp]
        _lib = lib
    return _lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _fbuf(x) -> tuple[np.ndarray, ctypes._Pointer]:
    a = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
    if a.size == 0:
        a = np.zeros(1, np.float32)
    return a, a.ctypes.data_as(_fp)


def sgemm_rows(trans_a, trans_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
               batch=1, stride_a=0, stride_b=0, stride_c=0,
               rows=None, batches=None, threads=None, want_S=True):
    """Oracle rows of the (strided-batched) GEMM over flat float32 buffers.

    Arguments mirror the library's C ABI. ``rows=(r0, r1)`` and
    ``batches=(b0, b1)`` restrict the output to those rows / batch items.
    Returns ``(ref, S)`` as float64 arrays of shape (nb, nr, N); S is None if
    ``want_S`` is false.
    """
    r0, r1 = rows if rows is not None else (0, M)
    b0, b1 = batches if batches is not None else (0, batch)
    nb, nr = max(0, b1 - b0), max(0, r1 - r0)
    ref = np.zeros((nb, nr, N), np.float64)
    S = np.zeros((nb, nr, N), np.float64) if want_S else None
    if nb == 0 or nr == 0 or N == 0:
        return ref, S
    a, pa = _fbuf(A)
    b, pb = _fbuf(B)
    c, pc = _fbuf(C)
    rc = _load().oracle_sgemm_rows(
        int(trans_a), int(trans_b), M, N, K,
        float(alpha), pa, lda, stride_a, pb, ldb, stride_b,
        float(beta), pc, ldc, stride_c,
        b0, b1, r0, r1,
        ref.ctypes.data_as(_dp), S.ctypes.data_as(_dp) if S is not None else None,
        int(threads or default_threads()))
    if rc != 0:
        raise RuntimeError("oracle_sgemm_rows failed")
    return ref, S


def sgemm_elements(trans_a, trans_b, K, alpha, A, lda, B, ldb, beta, C, ldc,
                   bs, is_, js, stride_a=0, stride_b=0, stride_c=0):
    """Oracle value and magnitude sum of individual elements (b, i, j)."""
    bs = np.ascontiguousarray(bs, dtype=np.int64)
    is_ = np.ascontiguousarray(is_, dtype=np.int64)
    js = np.ascontiguousarray(js, dtype=np.int64)
    n = bs.size
    ref = np.zeros(n, np.float64)
    S = np.zeros(n, np.float64)
    if n == 0:
        return ref, S
    a, pa = _fbuf(A)
    b, pb = _fbuf(B)
    c, pc = _fbuf(C)
    _load().oracle_sgemm_elements(
        int(trans_a), int(trans_b), K, float(alpha), pa, lda, stride_a,
        pb, ldb, stride_b, float(beta), pc, ldc, stride_c,
        n, bs.ctypes.data_as(_ip), is_.ctypes.data_as(_ip), js.ctypes.data_as(_ip),
        ref.ctypes.data_as(_dp), S.ctypes.data_as(_dp))
    return ref, S


@dataclass
class BoundReport:
    ok: bool
    n: int
    n_bad: int
    n_nonfinite: int
    max_norm_err: float     # max |d| / (max(K,1) * (|alpha| S + |beta| |c|))
    p999_norm_err: float
    worst_index: int

    def __str__(self):
        return (f"ok={self.ok} n={self.n} bad={self.n_bad} nonfinite={self.n_nonfinite} "
                f"max_norm_err={self.max_norm_err:.3e} (limit {TOL_PER_K:.1e}) "
                f"p99.9={self.p999_norm_err:.3e} worst@{self.worst_index}")


def bound_check(c_gpu, ref, S, c_in, alpha, beta, K, tol_per_k=TOL_PER_K) -> BoundReport:
    """Elementwise acceptance bound; all arrays share one shape.

    The scale uses max(K, 1) so that a K == 0 call (C = beta*C, rounded to
    float32 once) is held to a bound that is not identically zero.
    """
    g = np.asarray(c_gpu, dtype=np.float64).reshape(-1)
    r = np.asarray(ref, dtype=np.float64).reshape(-1)
    s = np.asarray(S, dtype=np.float64).reshape(-1)
    ci = np.asarray(c_in, dtype=np.float64).reshape(-1) if beta != 0 else np.zeros_like(r)
    n = r.size
    if n == 0:
        return BoundReport(True, 0, 0, 0, 0.0, 0.0, -1)
    scale = max(K, 1) * (abs(alpha) * s + abs(beta) * np.abs(ci))
    finite = np.isfinite(g)
    diff = np.abs(g - r)
    limit = tol_per_k * scale
    bad = ~finite | (diff > limit)
    with np.errstate(divide="ignore", invalid="ignore"):
        norm = np.where(scale > 0, diff / np.where(scale > 0, scale, 1.0),
                        np.where(diff > 0, np.inf, 0.0))
    norm = np.where(finite, norm, np.inf)
    worst = int(np.argmax(norm))
    return BoundReport(bool(not bad.any()), n, int(bad.sum()), int((~finite).sum()),
                       float(norm.max()),
                       float(np.quantile(np.minimum(norm, np.finfo(np.float64).max), 0.999)), worst)
