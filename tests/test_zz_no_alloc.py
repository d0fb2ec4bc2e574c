"""The entry point that allocates nothing (sgemm_strided_batched_noalloc),
through the C ABI, against the split-K entry point it mirrors
(sgemm_strided_batched_ws_variant with the automatic variant and a caller
workspace of the same size): the same bits on two calls in a row, the second
smaller, so the second reuses the array the first left behind. Also checked
against the oracle's bound, and a forced split too large for the array is
refused before anything runs. Captured into a HIP graph, its calls replay to
the eager bits."""
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


def test_noalloc_in_a_captured_graph(env):
    """The callers this entry point is for include code under HIP graph
    capture: two calls (an automatic split of a deep-K product and a forced
    split) captured into one graph replay to the eager bits, replay after
    replay, with other eager work in between. The partial tiles of both calls
    share the array, one call after the other on the captured stream."""
    torch, pg = env
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(91)
    # (a forced split needs a tile kernel: these shapes get the K-split tile)
    cases = [(0, 1, 256, 256, 16384, 2, 1.0, 2.0, 0), (1, 1, 1024, 768, 4000, 1, -0.5, 0.25, 4)]
    bufs = []
    for tA, tB, M, N, K, batch, alpha, beta, splits in cases:
        lda, ldb = (M if tA else K), (K if tB else N)
        dA = torch.from_numpy(rng.uniform(-1, 1, batch * M * K).astype(np.float32)).to(dev)
        dB = torch.from_numpy(rng.uniform(-1, 1, batch * K * N).astype(np.float32)).to(dev)
        dC0 = torch.from_numpy(rng.uniform(-1, 1, batch * M * N).astype(np.float32)).to(dev)
        bufs.append(((tA, tB, M, N, K, alpha, lda, ldb, beta, batch, splits), dA, dB, dC0,
                     dC0.clone()))

    def call(args, dA, dB, dC):
        tA, tB, M, N, K, alpha, lda, ldb, beta, batch, splits = args
        st = pg.sgemm_strided_batched_noalloc(tA, tB, M, N, K, alpha, dA, lda, dB, ldb, beta,
                                              dC, N, batch, M * K, K * N, M * N, splits,
                                              check=False)
        assert st == 0, (st, pg.sgemm_status_string(st))

    # eager bits (this also looks up the array's address and the CU count)
    for args, dA, dB, dC0, dC in bufs:
        call(args, dA, dB, dC)
    torch.cuda.synchronize(dev)
    want = [dC.cpu().numpy().view(np.uint32).copy() for (_, _, _, _, dC) in bufs]

    log("[noalloc] capture two calls")
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for args, dA, dB, dC0, dC in bufs:
                call(args, dA, dB, dC)
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize(dev)

    for rep in range(4):
        for args, dA, dB, dC0, dC in bufs:
            dC.copy_(dC0)  # beta != 0: every replay starts from the same C
        torch.cuda.synchronize(dev)
        g.replay()
        torch.cuda.synchronize(dev)
        for k, (args, dA, dB, dC0, dC) in enumerate(bufs):
            assert np.array_equal(dC.cpu().numpy().view(np.uint32), want[k]), (rep, args)
        # unrelated eager work between replays, itself through the array
        call((0, 0, 768, 768, 1500, 1.0, 1500, 768, 0.0, 1, 2),
             torch.rand(768 * 1500, device=dev), torch.rand(1500 * 768, device=dev),
             torch.empty(768 * 768, device=dev))
        torch.cuda.synchronize(dev)
