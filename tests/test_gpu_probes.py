"""GPU probes of the hardware behaviour the kernels are built on (test-only
kernels in tests/probes, built by __graft_entry__.build()).

- The FP32 MFMA lane layout: the epilogue of every tile kernel assumes that
  for v_mfma_f32_32x32x2_f32 lane l supplies A[l % 32][l / 32] and
  B[l / 32][l % 32] (a 32x2 by 2x32 product) and that accumulator register v
  of lane l holds output row 8*(v/4) + 4*(l/32) + v%4, column l % 32. The
  probe runs one MFMA on integer operands and checks every register.
- The FP32 MFMA issue rate: long runs of independent MFMAs with no memory
  traffic, reported against the 157.3 TFLOP/s dense FP32-MFMA peak.
- Both FP32 MFMA shapes (32x32x2 and 16x16x4), with four independent
  accumulators per wave and with one dependent chain: the rates each shape
  sustains and what a dependent chain costs.
"""
import ctypes
import os
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "probes", "libprobes.so")


@pytest.fixture(scope="module")
def probes():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    if not os.path.exists(LIB):
        pytest.fail("tests/probes/libprobes.so is not built (run __graft_entry__.build())")
    lib = ctypes.CDLL(LIB)
    p = ctypes.c_void_p
    lib.probe_mfma_layout.restype = ctypes.c_int
    lib.probe_mfma_layout.argtypes = [p, p, p]
    lib.probe_mfma_tflops.restype = ctypes.c_int
    lib.probe_mfma_tflops.argtypes = [ctypes.c_int, ctypes.c_int, p,
                                      ctypes.POINTER(ctypes.c_double)]
    lib.probe_mfma_shape_tflops.restype = ctypes.c_int
    lib.probe_mfma_shape_tflops.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                            p, ctypes.POINTER(ctypes.c_double)]
    return torch, lib


def test_mfma_32x32x2_lane_layout(probes):
    torch, lib = probes
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(11)
    for trial in range(4):
        A = rng.integers(-8, 9, (32, 2)).astype(np.float32)   # op(A) 32 x 2
        B = rng.integers(-8, 9, (2, 32)).astype(np.float32)   # op(B) 2 x 32
        lanes = np.arange(64)
        a = A[lanes % 32, lanes // 32]
        b = B[lanes // 32, lanes % 32]
        da, db = torch.from_numpy(a).to(dev), torch.from_numpy(b).to(dev)
        dd = torch.zeros(64 * 16, dtype=torch.float32, device=dev)
        assert lib.probe_mfma_layout(da.data_ptr(), db.data_ptr(), dd.data_ptr()) == 0
        got = dd.cpu().numpy().reshape(64, 16)
        D = A.astype(np.float64) @ B.astype(np.float64)
        v = np.arange(16)
        rows = 8 * (v[None, :] // 4) + 4 * (lanes[:, None] // 32) + v[None, :] % 4
        cols = np.broadcast_to(lanes[:, None] % 32, (64, 16))
        want = D[rows, cols].astype(np.float32)
        assert np.array_equal(got, want), f"trial {trial}: layout differs at " \
            f"{np.argwhere(got != want)[:4].tolist()}"


def test_mfma_issue_rate(probes):
    torch, lib = probes
    dev = torch.device("cuda:0")
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    out = torch.empty(2 * cus * 256, dtype=torch.float32, device=dev)
    tf = ctypes.c_double(0.0)
    # two workgroups of four waves per CU: two waves per SIMD
    assert lib.probe_mfma_tflops(2 * cus, 4096, out.data_ptr(), ctypes.byref(tf)) == 0
    sys.stdout.write(f"FP32 MFMA rate {tf.value:.1f} TFLOP/s "
                     f"({100 * tf.value / 157.3:.1f} % of 157.3) on {cus} CUs\n")
    sys.stdout.flush()
    # a sanity floor only: the rate depends on the clock the device runs at
    assert tf.value > 0.5 * 157.3 * cus / 256


def test_mfma_shapes(probes):
    torch, lib = probes
    dev = torch.device("cuda:0")
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    out = torch.empty(cus * 256, dtype=torch.float32, device=dev)
    rates = {}
    # one workgroup of four waves per CU: one wave per SIMD, so a dependent
    # chain is not hidden behind another wave
    for shape in (32, 16):
        for chains in (4, 1):
            tf = ctypes.c_double(0.0)
            assert lib.probe_mfma_shape_tflops(shape, chains, cus, 4096 if shape == 32 else 8192,
                                               out.data_ptr(), ctypes.byref(tf)) == 0
            rates[shape, chains] = tf.value
            sys.stdout.write(f"{shape}x{shape}x{128 // shape / 2:.0f} MFMA, {chains} chain(s): "
                             f"{tf.value:.1f} TFLOP/s ({100 * tf.value / 157.3:.1f} % of 157.3)\n")
    sys.stdout.flush()
    assert lib.probe_mfma_shape_tflops(8, 4, 1, 1, out.data_ptr(), ctypes.byref(tf)) == -1
    for v in rates.values():
        assert v > 0.1 * 157.3 * cus / 256


def test_no_schedule_cliff_across_transposes():
    """The 128 x 128 tile runs the same work at about the same speed for every
    transpose pair and for K with or without a partial K-step (4096^2 x K).
    A kernel whose compiled schedule falls off a cliff for one of them (an
    earlier build ran NT with K = 4092 24 % slower) fails this; the margin,
    12 % over the median, is far above run-to-run noise."""
    import statistics
    import time

    import torch

    import precision_gemm_amd as pg
    dev = torch.device("cuda:0")
    s = torch.cuda.current_stream(dev)
    n = 4096
    A, B, C = (torch.rand(n * n, device=dev) for _ in range(3))
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 0.3:  # clock ramp
        pg.sgemm(0, 0, n, n, n, 1.0, A, n, B, n, 0.0, C, n)
        torch.cuda.synchronize(dev)

    def timed(tA, tB, K):
        def call():
            pg.sgemm_strided_batched_variant(tA, tB, n, n, K, 1.0, A, n, B, n, 0.0, C, n, 1, 0, 0,
                                             0, pg.VARIANT_M128x128)
        for _ in range(3):
            call()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        for _ in range(8):
            call()
        e1.record(s)
        e1.synchronize()
        return e0.elapsed_time(e1) / 8

    cases = [(tA, tB, K) for tA in (0, 1) for tB in (0, 1) for K in (4096, 4092)]
    times = {c: statistics.median(timed(*c) for _ in range(3)) for c in cases}
    med = statistics.median(times.values())
    sys.stdout.write("transpose/K times (ms): " +
                     ", ".join(f"{'NT'[a]}{'NT'[b]} K{k}={t:.3f}" for (a, b, k), t in times.items())
                     + "\n")
    slow = {c: t for c, t in times.items() if t > 1.12 * med}
    assert not slow, f"schedule cliff: {slow} against a median of {med:.3f} ms"
