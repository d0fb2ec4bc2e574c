"""The entry point that allocates nothing (sgemm_strided_batched_noalloc),
through the C ABI, against the split-K entry point it mirrors
(sgemm_strided_batched_ws_variant with the automatic variant and a caller
workspace of the same size): the same bits on two calls in a row, the second
smaller, so the second reuses the array the first left behind. Also checked
against the oracle's bound, and a forced split too large for the array is
refused before anything runs."""
import sys

import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu


def log(msg):
    sys.stdout.write(msg + "\n")
    sys.stdout.flush()


@pytest.fixture(scope="module")
def env():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import precision_gemm_amd as pg
    pg._load()
    return torch, pg


def one_call(env, rng, tA, tB, M, N, K, batch, alpha, beta, splits):
    torch, pg = env
    dev = torch.device("cuda:0")
    lda, ldb, ldc = (M if tA else K), (K if tB else N), N
    sa, sb, sc = M * K, K * N, M * N
    A = rng.uniform(-1, 1, batch * sa).astype(np.float32)
    B = rng.uniform(-1, 1, batch * sb).astype(np.float32)
    C = rng.uniform(-1, 1, batch * sc).astype(np.float32)
    dA, dB = torch.from_numpy(A).to(dev), torch.from_numpy(B).to(dev)
    c_noalloc = torch.from_numpy(C).to(dev)
    c_ws = torch.from_numpy(C).to(dev)
    ws = torch.empty(pg.NOALLOC_SCRATCH_BYTES // 4, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    log(f"[noalloc] tA={tA} tB={tB} {M}x{N}x{K} batch={batch} splits={splits}")
    st = pg.sgemm_strided_batched_noalloc(tA, tB, M, N, K, alpha, dA, lda, dB, ldb, beta,
                                          c_noalloc, ldc, batch, sa, sb, sc, splits,
                                          stream=stream, check=False)
    assert st == 0, (st, pg.sgemm_status_string(st))
    st = pg.sgemm_strided_batched_ws_variant(tA, tB, M, N, K, alpha, dA, lda, dB, ldb, beta,
                                             c_ws, ldc, batch, sa, sb, sc, pg.VARIANT_AUTO,
                                             splits, ws, stream=stream, check=False)
    assert st == 0, st
    torch.cuda.synchronize(dev)
    got, want = c_noalloc.cpu().numpy(), c_ws.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), "bits differ"
    ref, S = oracle.sgemm_rows(tA, tB, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc,
                               batch=batch, stride_a=sa, stride_b=sb, stride_c=sc)
    rep = oracle.bound_check(got.reshape(batch, M, N), ref, S, C.reshape(batch, M, N), alpha,
                             beta, K)
    assert rep.ok, rep


def test_noalloc_matches_the_workspace_form(env):
    rng = np.random.default_rng(77)
    # six slices of 1024 x 1024 partial tiles: 24 MiB of the array
    one_call(env, rng, 0, 0, 1024, 1024, 3000, 1, 1.0, 0.5, 6)
    # right after, a smaller call over the array the first one left behind:
    # two slices of 768 x 768, other transposes, beta = 0
    one_call(env, rng, 1, 0, 768, 768, 1500, 1, -0.75, 0.0, 2)
    # and a smaller one again whose split the library picks (small grid, deep
    # K), batched
    one_call(env, rng, 0, 1, 256, 256, 16384, 2, 1.0, 2.0, 0)


def test_noalloc_refuses_a_split_beyond_its_array(env):
    torch, pg = env
    dev = torch.device("cuda:0")
    # 1024 x 1024 partials are 4 MiB a slice: 16 slices need 64 MiB
    A = torch.zeros(1024 * 8192, device=dev)
    B = torch.zeros(8192 * 1024, device=dev)
    C = torch.zeros(1024 * 1024, device=dev)
    st = pg.sgemm_strided_batched_noalloc(0, 0, 1024, 1024, 8192, 1.0, A, 8192, B, 1024, 0.0,
                                          C, 1024, 1, 0, 0, 0, 16, check=False)
    assert st == -23 and "scratch" in pg.sgemm_status_string(st)
    torch.cuda.synchronize(dev)
    assert int(torch.count_nonzero(C)) == 0
