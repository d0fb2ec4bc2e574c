"""GPU parity of the persistent tile kernels (P128x128, P64x64): one
workgroup per compute unit, three wave groups, whole tiles and a K range
split in thirds over the last tile of each unit. Integer inputs make every
order of summation exact, so the results must equal the oracle bit for bit;
on grids with no split tile the persistent kernels multiply in the same order
as the plain tiles and must give their bits on fp32 inputs too."""
import itertools
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
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    return torch, pg, cus


def log(msg):
    sys.stdout.write(msg + "\n")
    sys.stdout.flush()


def run(env, w, A, B, C, variant):
    torch, pg, _ = env
    dev = torch.device("cuda:0")
    dA, dB, dC = (torch.from_numpy(x).to(dev) for x in (A, B, C))
    st = pg.sgemm_strided_batched_variant(w.trans_a, w.trans_b, w.M, w.N, w.K, w.alpha, dA,
                                          w.LDA, dB, w.LDB, w.beta, dC, w.LDC, w.batch, w.SA,
                                          w.SB, w.SC, variant, check=False)
    torch.cuda.synchronize(dev)
    return st, dC.cpu().numpy()


def items(flat, w):
    return np.stack([np.lib.stride_tricks.as_strided(flat[b * w.SC:], (w.M, w.N),
                                                     (4 * w.LDC, 4)) for b in range(w.batch)])


def check_exact(w, A, B, C, got, batches, rows):
    ref, _ = oracle.sgemm_rows(w.trans_a, w.trans_b, w.M, w.N, w.K, w.alpha, A, w.LDA, B,
                               w.LDB, w.beta, C, w.LDC, batch=w.batch, stride_a=w.SA,
                               stride_b=w.SB, stride_c=w.SC, rows=rows, batches=batches,
                               want_S=False)
    want = ref.astype(np.float32)
    assert np.array_equal(ref, want.astype(np.float64))
    g = items(got, w)[batches[0]:batches[1], rows[0]:rows[1]]
    bad = np.argwhere(g != want)
    assert bad.size == 0, f"{w.name}: {len(bad)} mismatches, first {bad[:3].tolist()}"


def grid_shape(cus, bm, bn, ragged):
    """M, N whose bm x bn tiles number exactly `cus` (16 tile rows)."""
    tiles_n = cus // 16
    M, N = 16 * bm, tiles_n * bn
    return (M - ragged, N - 2 * ragged) if ragged else (M, N)


@pytest.mark.parametrize("variant,bm", [(13, 128), (14, 64)])
@pytest.mark.parametrize("per_cu", [1, 3, 4, 7])
def test_persistent_bitwise(env, variant, bm, per_cu):
    """n tiles per compute unit (1 and 4 and 7 split one tile in thirds, 3
    does not), every transpose pair, ragged M and N, K with a partial first
    step in every third; the batch makes up the tile count."""
    torch, pg, cus = env
    assert pg.VARIANT_NAMES[variant] == f"P{bm}x{bm}"
    if cus % 16:
        pytest.skip("shapes below assume a multiple of 16 compute units")
    M, N = grid_shape(cus, bm, bm, ragged=4)
    for (tA, tB), K in zip(itertools.product([0, 1], repeat=2), (200, 388, 196, 520)):
        w = Workload(f"p{per_cu}", tA, tB, M, N, K, 2.0, -1.0, seed=per_cu * 10 + 2 * tA + tB,
                     dist="int3", batch=per_cu, lda=(M if tA else K) + 4,
                     ldb=(K if tB else N) + 8, ldc=N + 4)
        A, B, C = workloads.make_inputs(w)
        log(f"[persistent] {pg.VARIANT_NAMES[variant]} n={per_cu} tA={tA} tB={tB} "
            f"{M}x{N}x{K} batch {per_cu}")
        st, got = run(env, w, A, B, C, variant)
        assert st == 0, st
        # every item's first and last rows (each tile row band of both ends)
        for b in sorted({0, per_cu - 1}):
            for rows in ((0, bm + 8), (M - bm - 8, M)):
                check_exact(w, A, B, C, got, (b, b + 1), rows)


@pytest.mark.parametrize("variant,plain", [(13, 1), (14, 2)])
def test_persistent_equals_plain_tile_without_split(env, variant, plain):
    """Three tiles per compute unit: every group takes whole tiles, which it
    multiplies in the plain tile's order, so fp32 results match its bits."""
    torch, pg, cus = env
    bm = 128 if variant == 13 else 64
    M, N = grid_shape(cus, bm, bm, ragged=0)
    for tA, tB in itertools.product([0, 1], repeat=2):
        w = Workload("peq", tA, tB, M, N, 300, 0.75, 1.5, seed=5 + 2 * tA + tB,
                     dist="normal", batch=3)
        A, B, C = workloads.make_inputs(w)
        st1, got1 = run(env, w, A, B, C, variant)
        st2, got2 = run(env, w, A, B, C, plain)
        assert st1 == 0 and st2 == 0
        assert np.array_equal(got1.view(np.uint32), got2.view(np.uint32)), (tA, tB)


def test_persistent_fp32_bound(env):
    """fp32 inputs through the split tiles: within the acceptance bound."""
    torch, pg, cus = env
    M, N = grid_shape(cus, 128, 128, ragged=4)
    w = Workload("pf", 1, 0, M, N, 1000, 1.0, 0.5, seed=3, dist="normal", batch=4)
    A, B, C = workloads.make_inputs(w)
    st, got = run(env, w, A, B, C, 13)
    assert st == 0
    for b in (0, 3):
        ref, S = oracle.sgemm_rows(w.trans_a, w.trans_b, w.M, w.N, w.K, w.alpha, A, w.LDA, B,
                                   w.LDB, w.beta, C, w.LDC, batch=w.batch, stride_a=w.SA,
                                   stride_b=w.SB, stride_c=w.SC, rows=(0, 200),
                                   batches=(b, b + 1))
        g = items(got, w)[b:b + 1, 0:200]
        cin = items(C, w)[b:b + 1, 0:200]
        rep = oracle.bound_check(g, ref, S, cin, w.alpha, w.beta, w.K)
        assert rep.ok, rep


def test_persistent_refusals(env):
    """Grids the persistent kernels cannot run are refused (-18), as is a
    split-K request (-19); nothing is written."""
    torch, pg, cus = env
    dev = torch.device("cuda:0")
    M, N = grid_shape(cus, 128, 128, ragged=0)
    A = torch.zeros(5 * M * 512, device=dev)
    B = torch.zeros(5 * 512 * N, device=dev)
    C = torch.full((5 * M * N,), 7.0, device=dev)
    # 2 and 5 tiles per compute unit (n % 3 == 2), a tile count that does not
    # divide, a K too short for thirds
    for batch, m, k in ((2, M, 512), (5, M, 512), (1, M - 128, 512), (1, M, 128)):
        st = pg.sgemm_strided_batched_variant(0, 0, m, N, k, 1.0, A, k, B, N, 0.0, C, N, batch,
                                              m * k, k * N, m * N, 13, check=False)
        assert st == -18, (batch, m, k, st)
    st = pg.sgemm_strided_batched_ws_variant(0, 0, M, N, 512, 1.0, A, 512, B, N, 0.0, C, N, 1,
                                             0, 0, 0, 13, 2, torch.empty(4 * M * N, device=dev),
                                             check=False)
    assert st == -19
    torch.cuda.synchronize(dev)
    assert bool(torch.all(C == 7.0))


def test_persistent_batched_workload(env):
    """The full-size batched workload (64 x 512 x 512 x 520, A transposed):
    four tiles per compute unit on 256 of them, one split in thirds."""
    torch, pg, cus = env
    w = workloads.BY_NAME["bmm_64x512x512x520_tn"]
    if (w.batch * 16) % cus:
        pytest.skip("the workload's 1024 tiles do not split evenly over this GPU")
    A, B, C = workloads.make_inputs(w)
    st, got = run(env, w, A, B, C, 13)
    assert st == 0
    for b in (0, 37, w.batch - 1):
        ref, S = oracle.sgemm_rows(w.trans_a, w.trans_b, w.M, w.N, w.K, w.alpha, A, w.LDA, B,
                                   w.LDB, w.beta, C, w.LDC, batch=w.batch, stride_a=w.SA,
                                   stride_b=w.SB, stride_c=w.SC, batches=(b, b + 1))
        rep = oracle.bound_check(items(got, w)[b:b + 1], ref, S, items(C, w)[b:b + 1], w.alpha,
                                 w.beta, w.K)
        log(f"  batch {b}: {rep}")
        assert rep.ok
