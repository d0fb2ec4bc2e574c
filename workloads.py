"""Seeded synthetic inputs for single-precision GEMM, shared by the tests, the
benchmark and the smoke check.

This module holds no GEMM arithmetic: it only names the workloads and draws
their operands. Both the GPU library and the CPU oracle consume what it
returns; neither is imported here.

Workloads (sizes, value distributions and alpha/beta) follow the single
workload of "From 1% to 94% of cuBLAS, one kernel at a time" (the 4092-cubed
SGEMM it benchmarks, with the alpha/beta epilogue of its kernels) widened to
the batched, transposed, ragged and memory-bound shapes the library must also
serve.

RNG reading (the pages fix none): ``numpy.random.default_rng(seed)`` (PCG64);
the stored buffers are drawn in the order A, B, C, each in memory order;
U(-1,1) is ``rng.uniform(-1, 1, n)`` in float64 rounded to float32 and N(0,1) is
``rng.standard_normal(n)`` rounded to float32. C is drawn even when beta is 0
so the operands do not change when beta does.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    """One strided-batched GEMM call ``C = alpha*op(A)@op(B) + beta*C``.

    Dimensions are those of the product (op(A) is M x K, op(B) is K x N);
    ``lda/ldb/ldc`` are row strides of the stored row-major buffers and
    ``stride_*`` the element distance between consecutive batch items.
    """

    name: str
    trans_a: int
    trans_b: int
    M: int
    N: int
    K: int
    alpha: float
    beta: float
    seed: int
    dist: str = "uniform"  # "uniform" = U(-1,1), "normal" = N(0,1)
    batch: int = 1
    lda: int | None = None
    ldb: int | None = None
    ldc: int | None = None
    stride_a: int | None = None
    stride_b: int | None = None
    stride_c: int | None = None
    note: str = field(default="", compare=False)

    # Stored shapes of the row-major buffers (rows, cols) per batch item.
    @property
    def a_stored(self) -> tuple[int, int]:
        return (self.K, self.M) if self.trans_a else (self.M, self.K)

    @property
    def b_stored(self) -> tuple[int, int]:
        return (self.N, self.K) if self.trans_b else (self.K, self.N)

    @property
    def c_stored(self) -> tuple[int, int]:
        return (self.M, self.N)

    @property
    def LDA(self) -> int:
        return self.lda if self.lda is not None else max(1, self.a_stored[1])

    @property
    def LDB(self) -> int:
        return self.ldb if self.ldb is not None else max(1, self.b_stored[1])

    @property
    def LDC(self) -> int:
        return self.ldc if self.ldc is not None else max(1, self.c_stored[1])

    @property
    def SA(self) -> int:
        return self.stride_a if self.stride_a is not None else _extent(self.a_stored, self.LDA)

    @property
    def SB(self) -> int:
        return self.stride_b if self.stride_b is not None else _extent(self.b_stored, self.LDB)

    @property
    def SC(self) -> int:
        return self.stride_c if self.stride_c is not None else _extent(self.c_stored, self.LDC)

    def buffer_lengths(self) -> tuple[int, int, int]:
        """Elements each flat buffer must hold (covering every batch item)."""
        def span(stored, ld, stride):
            one = _extent(stored, ld)
            if one == 0 or self.batch == 0:
                return 0
            return (self.batch - 1) * stride + one
        return (span(self.a_stored, self.LDA, self.SA),
                span(self.b_stored, self.LDB, self.SB),
                span(self.c_stored, self.LDC, self.SC))

    def flops(self) -> int:
        """2*M*N*K per GEMM, times the batch (epilogue flops not counted)."""
        return 2 * self.M * self.N * self.K * self.batch

    def algorithmic_bytes(self) -> int:
        """Each operand read once, C written once and read once iff beta != 0."""
        c_passes = 2 if self.beta != 0.0 else 1
        return 4 * self.batch * (self.M * self.K + self.K * self.N + c_passes * self.M * self.N)


def _extent(stored: tuple[int, int], ld: int) -> int:
    rows, cols = stored
    if rows == 0 or cols == 0:
        return 0
    return (rows - 1) * ld + cols


def draw(n: int, rng: np.random.Generator, dist: str) -> np.ndarray:
    if dist == "uniform":
        return rng.uniform(-1.0, 1.0, n).astype(np.float32)
    if dist == "normal":
        return rng.standard_normal(n).astype(np.float32)
    if dist.startswith("int"):
        # "int3": integers in [-3, 3]; every partial sum of a short dot product
        # of such values is exactly representable in float32.
        lim = int(dist[3:])
        return rng.integers(-lim, lim + 1, n).astype(np.float32)
    raise ValueError(f"unknown distribution {dist!r}")


def make_inputs(w: Workload) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Flat float32 buffers A, B, C for ``w``, drawn A then B then C."""
    rng = np.random.default_rng(w.seed)
    la, lb, lc = w.buffer_lengths()
    A = draw(la, rng, w.dist)
    B = draw(lb, rng, w.dist)
    C = draw(lc, rng, w.dist)
    return A, B, C


# The five workloads the library is measured and checked on.
CONFIGS: list[Workload] = [
    Workload("sgemm_128", 0, 0, 128, 128, 128, 1.0, 0.0, seed=1,
             note="small square, alpha=1 beta=0"),
    Workload("sgemm_1024", 0, 0, 1024, 1024, 1024, 0.5, 3.0, seed=2,
             note="beta*C read-modify-write epilogue"),
    Workload("sgemm_4092", 0, 0, 4092, 4092, 4092, 1.0, 0.5, seed=3,
             note="4092-cubed: ragged M/N edges and a masked K tail for BK>=8"),
    Workload("bmm_64x512x512x520_tn", 1, 0, 512, 512, 520, 1.0, 0.0, seed=4,
             dist="normal", batch=64,
             note="strided batched, A stored K x M, K % tile != 0"),
    Workload("skinny_16384x64x4096_nt", 0, 1, 16384, 64, 4096, 1.0, 1.0, seed=5,
             note="memory-streaming shape, B stored N x K"),
]

# Matrix-vector products, measured and profiled beside the five (not part of
# them): y = A x with A's rows contiguous in k, and y = A^T x with A stored
# K x M (contiguous along the outputs).
EXTRA: list[Workload] = [
    Workload("gemv_16384x1x4096_nt", 0, 1, 16384, 1, 4096, 1.0, 0.0, seed=6,
             note="matrix-vector product, matrix rows contiguous in k"),
    Workload("gemv_16384x1x4096_tt", 1, 1, 16384, 1, 4096, 1.0, 0.0, seed=7,
             note="matrix-vector product, matrix contiguous along the outputs"),
]

BY_NAME = {w.name: w for w in CONFIGS + EXTRA}
HEADLINE = BY_NAME["sgemm_4092"]
