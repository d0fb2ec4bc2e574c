"""Roofline arithmetic for the benchmark report.

The roofline model follows "Custom GPU kernels & Triton", section 2 (roofline
and arithmetic intensity): intensity is FLOPs per byte moved from HBM, the
ridge is peak FLOP/s over bandwidth, the attainable rate is the smaller of the
peak and intensity times bandwidth, and an operation below the ridge is
memory-bound.

The block-tile intensity BM*BN / (2*(BM+BN)) FLOP per byte of fp32 loaded into
shared memory is the one "From 1% to 94% of cuBLAS, one kernel at a time"
derives for its 2-D blocktiling kernel (kernel 5, "Counting again").

MI355X figures are AMD's published ones: 256 CUs at 2.4 GHz, dense FP32 matrix
(MFMA) 157.3 TFLOP/s, FP32 vector 157.3 TFLOP/s with packed math (half of it
without), HBM3E 8.0 TB/s.
"""
from __future__ import annotations

from dataclasses import dataclass

MI355X_FP32_MFMA_PEAK = 157.3e12  # FLOP/s, dense
MI355X_HBM_BW = 8.0e12            # B/s
MI355X_CUS = 256
MI355X_SCLK = 2.4e9


@dataclass(frozen=True)
class Roof:
    intensity: float    # FLOP per byte
    ridge: float        # FLOP per byte where the bound flips
    attainable: float   # FLOP/s
    bound: str          # "memory-bound" or "compute-bound"
    peak: float         # FLOP/s

    @property
    def frac_of_peak(self) -> float:
        return self.attainable / self.peak


def roofline(flops: float, bytes_moved: float, peak_flops: float, bw_bytes_per_s: float) -> Roof:
    ai = flops / bytes_moved
    ridge = peak_flops / bw_bytes_per_s
    attainable = min(peak_flops, ai * bw_bytes_per_s)
    bound = "memory-bound" if ai < ridge else "compute-bound"
    return Roof(ai, ridge, attainable, bound, peak_flops)


def block_tile_intensity(bm: int, bn: int) -> float:
    """FLOPs per byte of fp32 A/B staged per K-step by a BM x BN block tile."""
    return bm * bn / (2.0 * (bm + bn))


def gemm_flops(M: int, N: int, K: int, batch: int = 1) -> int:
    return 2 * M * N * K * batch


def naive_kernel_read_bytes(M: int, N: int, K: int) -> int:
    """Bytes a kernel with no on-chip reuse reads: two fp32 loads per multiply-add."""
    return 2 * 4 * M * N * K
