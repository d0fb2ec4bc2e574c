"""Per-shape dispatch overrides on the GPU: an automatic call whose shape has
an installed record runs the record's variant. On U(-1, 1) inputs different
kernels round differently, so the check is that the automatic call's output
equals the forced variant's bit for bit (and lies within the oracle's bound),
for the plain, the split-K and the pointer-array entry points."""
import sys

import numpy as np
import pytest

import oracle
import workloads
from workloads import Workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import precision_gemm_amd as pg
    pg._load()
    pg.sgemm_set_dispatch_overrides([])
    yield torch, pg
    pg.sgemm_set_dispatch_overrides([])  # the table is process-wide


def log(msg):
    sys.stdout.write(msg + "\n")
    sys.stdout.flush()


def bits_of(env, w, variant=-1, ws=False):
    torch, pg = env
    dev = torch.device("cuda:0")
    A, B, C = workloads.make_inputs(w)
    dA, dB, dC = (torch.from_numpy(x).to(dev) for x in (A, B, C))
    args = (w.trans_a, w.trans_b, w.M, w.N, w.K, w.alpha, dA, w.LDA, dB, w.LDB, w.beta, dC,
            w.LDC, w.batch, w.SA, w.SB, w.SC)
    if ws:
        # split-K form with the split held at one slice (a split would change
        # the summation order): its automatic choice consults the table too
        work = torch.empty(64 << 20, dtype=torch.uint8, device=dev)
        pg.sgemm_strided_batched_ws_variant(*args, variant, 1, work)
    else:
        pg.sgemm_strided_batched_variant(*args, variant)
    torch.cuda.synchronize(dev)
    return A, B, C, dC.cpu().numpy()


@pytest.mark.parametrize("shape,forced", [
    ((0, 0, 1000, 1000, 1000, 1), "M128x128"),    # the model's K-split tile otherwise
    ((1, 0, 512, 512, 520, 8), "T64x64"),         # the model's 64 x 64 tile otherwise
    ((0, 1, 700, 300, 2048, 1), "S64x64_K2"),     # the model's streaming 64 x 32 tile otherwise
])
def test_automatic_call_runs_the_override(env, shape, forced):
    torch, pg = env
    tA, tB, M, N, K, batch = shape
    w = Workload("ovr", tA, tB, M, N, K, 1.0, 0.5, seed=M + K, batch=batch)
    model = pg.VARIANT_NAMES[pg.sgemm_select_variant(tA, tB, M, N, K, batch, 1, 256)]
    assert model != forced, (shape, model)
    A, B, C, want = bits_of(env, w, variant=getattr(pg, f"VARIANT_{forced}"))
    _, _, _, before = bits_of(env, w)
    pg.sgemm_set_dispatch_overrides([(*shape, forced)])
    try:
        _, _, _, got = bits_of(env, w)
        _, _, _, got_ws = bits_of(env, w, ws=True)
    finally:
        pg.sgemm_set_dispatch_overrides([])
    differ = int(np.count_nonzero(before.view(np.uint32) != want.view(np.uint32)))
    log(f"  {shape}: {model} -> {forced}; elements whose bits differ between the two: {differ}")
    # the two variants sum in different orders, so their bits tell them apart
    assert differ > 0
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    assert np.array_equal(got_ws.view(np.uint32), want.view(np.uint32))
    ref, S = oracle.sgemm_rows(tA, tB, M, N, K, 1.0, A, w.LDA, B, w.LDB, 0.5, C, w.LDC,
                               batch=batch, stride_a=w.SA, stride_b=w.SB, stride_c=w.SC)
    cin = C.reshape(batch, M, N)
    assert oracle.bound_check(got.reshape(batch, M, N), ref, S, cin, 1.0, 0.5, K).ok


def test_pointer_array_call_runs_the_override(env):
    torch, pg = env
    dev = torch.device("cuda:0")
    M, N, K, batch = 600, 400, 900, 3
    rng = np.random.default_rng(5)
    As = [torch.from_numpy(rng.uniform(-1, 1, (M, K)).astype(np.float32)).to(dev) for _ in range(batch)]
    Bs = [torch.from_numpy(rng.uniform(-1, 1, (K, N)).astype(np.float32)).to(dev) for _ in range(batch)]
    C0 = rng.uniform(-1, 1, (M, N)).astype(np.float32)

    def run(variant):
        Cs = [torch.from_numpy(C0).to(dev) for _ in range(batch)]
        pa, pb, pc = (pg.pointer_array(x) for x in (As, Bs, Cs))
        pg.sgemm_batched_variant(0, 0, M, N, K, 1.0, pa, K, pb, N, 1.0, pc, N, batch, variant)
        torch.cuda.synchronize(dev)
        return np.stack([c.cpu().numpy() for c in Cs])

    model = pg.sgemm_select_variant(0, 0, M, N, K, batch, 1, 256)
    forced = pg.VARIANT_L256x128 if model != pg.VARIANT_L256x128 else pg.VARIANT_S64x64
    want = run(forced)
    assert not np.array_equal(run(-1).view(np.uint32), want.view(np.uint32))
    pg.sgemm_set_dispatch_overrides([(0, 0, M, N, K, batch, forced)])
    try:
        got = run(-1)
    finally:
        pg.sgemm_set_dispatch_overrides([])
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_misaligned_call_ignores_a_four_float_override(env):
    """A record whose variant needs 16-byte loads does not apply to a call that
    cannot use them: the call runs the 1-float variant and is still right."""
    torch, pg = env
    w = Workload("ovr_v1", 0, 0, 257, 129, 65, 1.0, 0.0, seed=3)  # K % 4 != 0: no 4-float path
    A, B, C, want = bits_of(env, w, variant=pg.VARIANT_S64x64_V1)
    pg.sgemm_set_dispatch_overrides([(0, 0, 257, 129, 65, 1, "M128x128")])
    try:
        _, _, _, got = bits_of(env, w)
    finally:
        pg.sgemm_set_dispatch_overrides([])
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_library_loaded_before_torch(env):
    """Installing overrides (or any call of the binding) before torch is
    imported must not leave the process with a second HIP runtime: in a fresh
    process, load the library first, then import torch and run a GEMM."""
    import os
    import subprocess
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = "\n".join([
        "import precision_gemm_amd as pg",
        "assert pg.sgemm_dispatch_override_count() == 0  # the library is loaded here",
        "import torch",
        "x = torch.ones(64 * 64, device='cuda')",
        "y = torch.zeros(64 * 64, device='cuda')",
        "pg.sgemm(0, 0, 64, 64, 64, 1.0, x, 64, x, 64, 0.0, y, 64)",
        "torch.cuda.synchronize()",
        "assert float(y[0]) == 64.0 and float(y[-1]) == 64.0",
        "print('ok')",
    ])
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=240,
                       cwd=root)
    assert r.returncode == 0 and "ok" in r.stdout, r.stderr[-2000:]
