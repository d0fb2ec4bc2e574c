"""Roofline arithmetic for the benchmark report.

The roofline model is the one "Custom GPU kernels & Triton" sets out in
section 2 (roofline and arithmetic intensity): a kernel is limited either by
its arithmetic or by the bytes it moves from HBM, its intensity (FLOPs per HBM
byte) says which, and the ridge is the intensity at which the two limits meet.

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
    intensity: float    # FLOP per byte moved from HBM
    ridge: float        # FLOP per byte at which both floors are equal
    attainable: float   # FLOP/s the slower of the two resources allows
    bound: str          # "memory-bound" or "compute-bound"
    peak: float         # FLOP/s

    @property
    def frac_of_peak(self) -> float:
        return self.attainable / self.peak


def place_on_roofline(flops: float, hbm_bytes: float, peak_flops: float,
                      hbm_bw: float) -> Roof:
    """Where a kernel doing `flops` and moving `hbm_bytes` sits on the roofline.

    Each resource sets a floor on the kernel's time: the math at the peak rate
    and the traffic at the HBM rate. The larger floor is the bound, and the work
    over that floor is the best rate the kernel can reach. A tie (a kernel on the
    ridge) counts as compute-bound.
    """
    t_math = flops / peak_flops
    t_hbm = hbm_bytes / hbm_bw
    limited_by_hbm = t_hbm > t_math
    return Roof(intensity=flops / hbm_bytes, ridge=peak_flops / hbm_bw,
                attainable=flops / (t_hbm if limited_by_hbm else t_math),
                bound="memory-bound" if limited_by_hbm else "compute-bound",
                peak=peak_flops)


def block_tile_intensity(bm: int, bn: int) -> float:
    """FLOPs per byte of fp32 A/B staged per K-step by a BM x BN block tile."""
    return bm * bn / (2.0 * (bm + bn))


def gemm_flops(M: int, N: int, K: int, batch: int = 1) -> int:
    return 2 * M * N * K * batch


def naive_kernel_read_bytes(M: int, N: int, K: int) -> int:
    """Bytes a kernel with no on-chip reuse reads: two fp32 loads per multiply-add."""
    return 2 * 4 * M * N * K
