"""precision_gemm_amd — single-precision GEMM on MI355X (gfx950).

A thin ctypes binding over ``libsgemm.so`` (built from ``csrc/sgemm.hip``;
its C ABI is declared in ``include/sgemm.h``). The functions have the C
names and argument order; they only marshal arguments (tensor -> device
pointer, torch's current stream -> hipStream_t) and raise on a nonzero
status. All arithmetic runs in the library's HIP kernels; there is no CPU or
PyTorch fallback, and a missing library is an error.

    C = alpha * op(A) @ op(B) + beta * C            (fp32, row-major)
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "SgemmError", "sgemm", "sgemm_strided_batched", "sgemm_strided_batched_variant",
    "sgemm_batched", "sgemm_batched_variant", "sgemm_colmajor",
    "sgemm_colmajor_strided_batched", "pointer_array", "sgemm_ws", "sgemm_strided_batched_ws",
    "sgemm_strided_batched_ws_variant", "sgemm_workspace_size", "sgemm_select_splits",
    "sgemm_status_string", "sgemm_select_variant", "sgemm_window_ranges",
    "sgemm_strided_batched_noalloc", "NOALLOC_SCRATCH_BYTES", "matmul",
    "sgemm_set_dispatch_overrides", "sgemm_dispatch_override_count", "load_dispatch_overrides",
    "MAX_DISPATCH_OVERRIDES",
    "library_path",
    "VARIANT_AUTO", "VARIANT_L256x128", "VARIANT_M128x128", "VARIANT_S64x64",
    "VARIANT_S64x64_V1", "VARIANT_T64x64", "VARIANT_L256x256", "VARIANT_S64x64_K2",
    "VARIANT_M128x128_DMA", "VARIANT_T32x64", "VARIANT_T64x32", "VARIANT_GEMV",
    "VARIANT_W64x64", "VARIANT_W64x64_V1", "VARIANT_P128x128", "VARIANT_P64x64",
    "VARIANT_COUNT", "VARIANT_NAMES",
]

VARIANT_AUTO = -1
VARIANT_L256x128 = 0
VARIANT_M128x128 = 1
VARIANT_S64x64 = 2
VARIANT_S64x64_V1 = 3
VARIANT_T64x64 = 4
VARIANT_L256x256 = 5
VARIANT_S64x64_K2 = 6
VARIANT_M128x128_DMA = 7
VARIANT_T32x64 = 8
VARIANT_T64x32 = 9
VARIANT_GEMV = 10
VARIANT_W64x64 = 11
VARIANT_W64x64_V1 = 12
VARIANT_P128x128 = 13
VARIANT_P64x64 = 14
VARIANT_COUNT = 15
VARIANT_NAMES = {0: "L256x128", 1: "M128x128", 2: "S64x64", 3: "S64x64_V1", 4: "T64x64",
                 5: "L256x256", 6: "S64x64_K2", 7: "M128x128_DMA",
                 8: "T32x64", 9: "T64x32", 10: "GEMV", 11: "W64x64", 12: "W64x64_V1",
                 13: "P128x128", 14: "P64x64"}

# SGEMM_NOALLOC_SCRATCH_BYTES of the C header: the fixed device array of the
# entry point that allocates nothing
NOALLOC_SCRATCH_BYTES = 32 << 20

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None


def library_path() -> str:
    """The in-tree library; SGEMM_LIBRARY may name another build of the same
    source (used when comparing tuning builds side by side)."""
    return os.environ.get("SGEMM_LIBRARY") or os.path.join(_HERE, "libsgemm.so")


class SgemmError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"sgemm status {status}: {message}")
        self.status = status


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: the HIP library must be built first "
            "(python -c 'import __graft_entry__ as g; g.build()')")
    # The library links the HIP runtime by its soname. Loaded after torch, it
    # binds to the runtime torch already loaded, and both share one view of
    # the devices. Loaded first, it brings in a second runtime next to
    # torch's, and its device calls then fail. So torch, when installed, is
    # imported first.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    i, f, p, ll = ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_longlong
    lib.sgemm.restype = i
    lib.sgemm.argtypes = [i, i, i, i, i, f, p, i, p, i, f, p, i, p]
    lib.sgemm_strided_batched.restype = i
    lib.sgemm_strided_batched.argtypes = [i, i, i, i, i, f, p, i, p, i, f, p, i, i, ll, ll, ll, p]
    lib.sgemm_strided_batched_variant.restype = i
    lib.sgemm_strided_batched_variant.argtypes = [i, i, i, i, i, f, p, i, p, i, f, p, i, i,
                                                  ll, ll, ll, i, p]
    lib.sgemm_status_string.restype = ctypes.c_char_p
    lib.sgemm_status_string.argtypes = [i]
    lib.sgemm_select_variant.restype = i
    lib.sgemm_select_variant.argtypes = [i, i, i, i, i, i, i, i]
    lib.sgemm_batched.restype = i
    lib.sgemm_batched.argtypes = [i, i, i, i, i, f, p, i, p, i, f, p, i, i, p]
    lib.sgemm_batched_variant.restype = i
    lib.sgemm_batched_variant.argtypes = [i, i, i, i, i, f, p, i, p, i, f, p, i, i, i, p]
    sz = ctypes.c_size_t
    lib.sgemm_ws.restype = i
    lib.sgemm_ws.argtypes = [i, i, i, i, i, f, p, i, p, i, f, p, i, p, sz, p]
    lib.sgemm_strided_batched_ws.restype = i
    lib.sgemm_strided_batched_ws.argtypes = [i, i, i, i, i, f, p, i, p, i, f, p, i, i, ll, ll, ll,
                                             p, sz, p]
    lib.sgemm_strided_batched_ws_variant.restype = i
    lib.sgemm_strided_batched_ws_variant.argtypes = [i, i, i, i, i, f, p, i, p, i, f, p, i, i, ll,
                                                     ll, ll, i, i, p, sz, p]
    lib.sgemm_workspace_size.restype = sz
    lib.sgemm_workspace_size.argtypes = [i, i, i, i, i, i]
    lib.sgemm_select_splits.restype = i
    lib.sgemm_select_splits.argtypes = [i, i, i, i, i, i, i, i]
    lib.sgemm_colmajor.restype = i
    lib.sgemm_colmajor.argtypes = [i, i, i, i, i, f, p, i, p, i, f, p, i, p]
    lib.sgemm_colmajor_strided_batched.restype = i
    lib.sgemm_colmajor_strided_batched.argtypes = [i, i, i, i, i, f, p, i, p, i, f, p, i, i,
                                                   ll, ll, ll, p]
    lib.sgemm_strided_batched_noalloc.restype = i
    lib.sgemm_strided_batched_noalloc.argtypes = [i, i, i, i, i, f, p, i, p, i, f, p, i, i, ll,
                                                  ll, ll, i, p]
    lib.sgemm_window_ranges.restype = i
    lib.sgemm_window_ranges.argtypes = [ll, i, i, ctypes.POINTER(ctypes.c_uint)]
    lib.sgemm_set_dispatch_overrides.restype = i
    lib.sgemm_set_dispatch_overrides.argtypes = [ctypes.POINTER(ctypes.c_int), i]
    lib.sgemm_dispatch_override_count.restype = i
    lib.sgemm_dispatch_override_count.argtypes = []
    _lib = lib
    return lib


def _ptr(x):
    """Device pointer of a float32 GPU tensor, or an int / None passed through."""
    if x is None or isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        if not x.is_cuda:
            raise TypeError("sgemm operands must be GPU tensors")
        import torch
        if x.dtype != torch.float32:
            raise TypeError(f"sgemm operands must be float32, got {x.dtype}")
        return x.data_ptr()
    raise TypeError(f"cannot take a device pointer of {type(x).__name__}")


def _ptr_array(x):
    """Device address of a pointer array: an int64 GPU tensor of device
    addresses (see pointer_array), or an int / None passed through."""
    if x is None or isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        import torch
        if not x.is_cuda or x.dtype != torch.int64 or not x.is_contiguous():
            raise TypeError("a pointer array must be a contiguous int64 GPU tensor")
        return x.data_ptr()
    raise TypeError(f"cannot take a device pointer of {type(x).__name__}")


def pointer_array(tensors, device=None):
    """An int64 GPU tensor holding the device addresses of `tensors` (float32
    GPU tensors, or ints taken as addresses), for the pointer-array form. The
    caller keeps the tensors alive while the work runs."""
    import torch
    addrs = [t if isinstance(t, int) else _ptr(t) for t in tensors]
    if device is None:
        device = next((t.device for t in tensors if hasattr(t, "device")), "cuda")
    return torch.tensor(addrs, dtype=torch.int64).to(device)


def _stream(stream, *tensors):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    for t in tensors:
        if hasattr(t, "data_ptr"):
            import torch
            return torch.cuda.current_stream(t.device).cuda_stream
    return None


def _check(status: int, check: bool) -> int:
    if status != 0 and check:
        raise SgemmError(status, sgemm_status_string(status))
    return status


def sgemm_status_string(status: int) -> str:
    return _load().sgemm_status_string(int(status)).decode()


def sgemm(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=None,
          check=True) -> int:
    """C ABI ``sgemm``; A, B, C are float32 GPU tensors (or raw pointers)."""
    st = _load().sgemm(int(transA), int(transB), M, N, K, float(alpha), _ptr(A), lda,
                       _ptr(B), ldb, float(beta), _ptr(C), ldc, _stream(stream, A, B, C))
    return _check(st, check)


def sgemm_strided_batched(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                          batch, strideA, strideB, strideC, stream=None, check=True) -> int:
    """C ABI ``sgemm_strided_batched``."""
    st = _load().sgemm_strided_batched(int(transA), int(transB), M, N, K, float(alpha),
                                       _ptr(A), lda, _ptr(B), ldb, float(beta), _ptr(C), ldc,
                                       batch, strideA, strideB, strideC,
                                       _stream(stream, A, B, C))
    return _check(st, check)


def sgemm_strided_batched_variant(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C,
                                  ldc, batch, strideA, strideB, strideC, variant,
                                  stream=None, check=True) -> int:
    """C ABI ``sgemm_strided_batched_variant`` (kernel variant forced)."""
    st = _load().sgemm_strided_batched_variant(
        int(transA), int(transB), M, N, K, float(alpha), _ptr(A), lda, _ptr(B), ldb,
        float(beta), _ptr(C), ldc, batch, strideA, strideB, strideC, int(variant),
        _stream(stream, A, B, C))
    return _check(st, check)


def _workspace(ws):
    """(device address, bytes) of a workspace: a GPU tensor of any dtype (its
    whole storage), an (address, bytes) pair, or None (no workspace)."""
    if ws is None:
        return None, 0
    if isinstance(ws, tuple):
        return ws[0], int(ws[1])
    if hasattr(ws, "data_ptr"):
        if not ws.is_cuda:
            raise TypeError("a workspace must be a GPU tensor")
        return ws.data_ptr(), ws.numel() * ws.element_size()
    raise TypeError(f"cannot use {type(ws).__name__} as a workspace")


def sgemm_ws(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, workspace,
             stream=None, check=True) -> int:
    """C ABI ``sgemm_ws`` (split-K with a caller workspace, see _workspace)."""
    wp, wb = _workspace(workspace)
    st = _load().sgemm_ws(int(transA), int(transB), M, N, K, float(alpha), _ptr(A), lda,
                          _ptr(B), ldb, float(beta), _ptr(C), ldc, wp, wb,
                          _stream(stream, A, B, C))
    return _check(st, check)


def sgemm_strided_batched_ws(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                             batch, strideA, strideB, strideC, workspace, stream=None,
                             check=True) -> int:
    """C ABI ``sgemm_strided_batched_ws``."""
    wp, wb = _workspace(workspace)
    st = _load().sgemm_strided_batched_ws(int(transA), int(transB), M, N, K, float(alpha),
                                          _ptr(A), lda, _ptr(B), ldb, float(beta), _ptr(C), ldc,
                                          batch, strideA, strideB, strideC, wp, wb,
                                          _stream(stream, A, B, C))
    return _check(st, check)


def sgemm_strided_batched_ws_variant(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C,
                                     ldc, batch, strideA, strideB, strideC, variant, splits,
                                     workspace, stream=None, check=True) -> int:
    """C ABI ``sgemm_strided_batched_ws_variant`` (variant and split count forced)."""
    wp, wb = _workspace(workspace)
    st = _load().sgemm_strided_batched_ws_variant(
        int(transA), int(transB), M, N, K, float(alpha), _ptr(A), lda, _ptr(B), ldb,
        float(beta), _ptr(C), ldc, batch, strideA, strideB, strideC, int(variant), int(splits),
        wp, wb, _stream(stream, A, B, C))
    return _check(st, check)


def sgemm_strided_batched_noalloc(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                                  batch, strideA, strideB, strideC, splits=0, stream=None,
                                  check=True) -> int:
    """C ABI ``sgemm_strided_batched_noalloc`` (split-K partials in the
    library's fixed device array; allocates nothing)."""
    st = _load().sgemm_strided_batched_noalloc(
        int(transA), int(transB), M, N, K, float(alpha), _ptr(A), lda, _ptr(B), ldb,
        float(beta), _ptr(C), ldc, batch, strideA, strideB, strideC, int(splits),
        _stream(stream, A, B, C))
    return _check(st, check)


def sgemm_workspace_size(transA, transB, M, N, K, batch=1) -> int:
    """C ABI ``sgemm_workspace_size`` (bytes, for the current device)."""
    return int(_load().sgemm_workspace_size(int(transA), int(transB), M, N, K, batch))


def sgemm_select_splits(transA, transB, M, N, K, batch, variant, num_cus) -> int:
    """C ABI ``sgemm_select_splits`` (host-side split decision)."""
    return _load().sgemm_select_splits(int(transA), int(transB), M, N, K, batch, int(variant),
                                       num_cus)


def sgemm_batched(transA, transB, M, N, K, alpha, A_array, lda, B_array, ldb, beta, C_array,
                  ldc, batch, stream=None, check=True) -> int:
    """C ABI ``sgemm_batched``; the arrays are int64 GPU tensors of device
    addresses (see pointer_array) or raw device pointers."""
    st = _load().sgemm_batched(int(transA), int(transB), M, N, K, float(alpha),
                               _ptr_array(A_array), lda, _ptr_array(B_array), ldb, float(beta),
                               _ptr_array(C_array), ldc, batch,
                               _stream(stream, A_array, B_array, C_array))
    return _check(st, check)


def sgemm_batched_variant(transA, transB, M, N, K, alpha, A_array, lda, B_array, ldb, beta,
                          C_array, ldc, batch, variant, stream=None, check=True) -> int:
    """C ABI ``sgemm_batched_variant`` (kernel variant forced)."""
    st = _load().sgemm_batched_variant(int(transA), int(transB), M, N, K, float(alpha),
                                       _ptr_array(A_array), lda, _ptr_array(B_array), ldb,
                                       float(beta), _ptr_array(C_array), ldc, batch,
                                       int(variant), _stream(stream, A_array, B_array, C_array))
    return _check(st, check)


def sgemm_colmajor(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream=None,
                   check=True) -> int:
    """C ABI ``sgemm_colmajor`` (BLAS column-major storage)."""
    st = _load().sgemm_colmajor(int(transA), int(transB), M, N, K, float(alpha), _ptr(A), lda,
                                _ptr(B), ldb, float(beta), _ptr(C), ldc,
                                _stream(stream, A, B, C))
    return _check(st, check)


def sgemm_colmajor_strided_batched(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                                   batch, strideA, strideB, strideC, stream=None,
                                   check=True) -> int:
    """C ABI ``sgemm_colmajor_strided_batched``."""
    st = _load().sgemm_colmajor_strided_batched(int(transA), int(transB), M, N, K, float(alpha),
                                                _ptr(A), lda, _ptr(B), ldb, float(beta),
                                                _ptr(C), ldc, batch, strideA, strideB, strideC,
                                                _stream(stream, A, B, C))
    return _check(st, check)


def sgemm_select_variant(transA, transB, M, N, K, batch, vec4_ok, num_cus) -> int:
    """C ABI ``sgemm_select_variant`` (host-side dispatch decision)."""
    return _load().sgemm_select_variant(int(transA), int(transB), M, N, K, batch,
                                        int(bool(vec4_ok)), num_cus)


MAX_DISPATCH_OVERRIDES = 1 << 20  # SGEMM_MAX_DISPATCH_OVERRIDES


def sgemm_set_dispatch_overrides(records, check=True) -> int:
    """C ABI ``sgemm_set_dispatch_overrides``: install per-shape overrides of
    the automatic choice, replacing any installed table. `records` is an
    iterable of (transA, transB, M, N, K, batch, variant), the variant a
    number or a name of VARIANT_NAMES; an empty iterable clears the table."""
    by_name = {n: v for v, n in VARIANT_NAMES.items()}
    flat = []
    for rec in records:
        if len(rec) != 7:
            raise ValueError(f"an override record has 7 fields, got {rec!r}")
        variant = by_name[rec[6]] if isinstance(rec[6], str) else int(rec[6])
        flat.extend([int(x) for x in rec[:6]] + [variant])
    n = len(flat) // 7
    arr = (ctypes.c_int * len(flat))(*flat) if flat else None
    return _check(_load().sgemm_set_dispatch_overrides(arr, n), check)


def sgemm_dispatch_override_count() -> int:
    """C ABI ``sgemm_dispatch_override_count``."""
    return _load().sgemm_dispatch_override_count()


def load_dispatch_overrides(path, check=True) -> int:
    """Install the overrides a tuning sweep wrote (``python -m
    precision_gemm_amd.tune --write-overrides PATH``): a JSON list of records
    as sgemm_set_dispatch_overrides takes them."""
    import json
    with open(path) as f:
        return sgemm_set_dispatch_overrides(json.load(f), check=check)


def sgemm_window_ranges(left_bytes, step_bytes, nsteps):
    """C ABI ``sgemm_window_ranges``: the buffer ranges the kernels give the
    successive load windows of an operand (host-side, no device call). Returns
    a list of nsteps ints; raises SgemmError on invalid arguments."""
    out = (ctypes.c_uint * max(1, nsteps))()
    st = _load().sgemm_window_ranges(int(left_bytes), int(step_bytes), int(nsteps), out)
    _check(st, True)
    return list(out[:nsteps])


def matmul(A, B, C, alpha=1.0, beta=0.0, transA=False, transB=False, stream=None):
    """In-place ``C = alpha*op(A)@op(B) + beta*C`` on 2-D (or 3-D, batched)
    float32 GPU tensors whose last dimension is contiguous; the leading
    dimensions are the tensors' row strides. Returns C."""
    if A.dim() != B.dim() or A.dim() != C.dim() or A.dim() not in (2, 3):
        raise ValueError("matmul takes three 2-D or three 3-D tensors")
    for t in (A, B, C):
        if t.stride(-1) != 1:
            raise ValueError("the last dimension of every operand must be contiguous")
    M, N = C.shape[-2], C.shape[-1]
    K = A.shape[-2] if transA else A.shape[-1]
    if (A.shape[-1] if transA else A.shape[-2]) != M:
        raise ValueError("op(A) rows must equal C rows")
    if (B.shape[-1] if transB else B.shape[-2]) != K or \
            (B.shape[-2] if transB else B.shape[-1]) != N:
        raise ValueError("op(B) must be K x N")
    lda, ldb, ldc = (max(1, t.stride(-2)) for t in (A, B, C))
    if A.dim() == 2:
        sgemm(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream)
    else:
        batch = C.shape[0]
        if A.shape[0] != batch or B.shape[0] != batch:
            raise ValueError("batch sizes differ")
        sgemm_strided_batched(transA, transB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                              batch, A.stride(0), B.stride(0), C.stride(0), stream)
    return C
