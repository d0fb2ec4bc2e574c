"""GPU parity at the limits of the addressing: leading dimensions of 2^21
and more, one operand larger than 2 GiB, and a matrix-vector product taller
than one launch's grid. Integer inputs in [-3, 3] keep every partial sum
exact, so the GPU must equal the oracle bit for bit.

These buffers are large (up to ~10 GiB of device memory per case), so only
the rows the call uses are filled: padding between rows stays zero, and after
the call everything outside C's window must still be zero.
"""
import sys

import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu

GUARD = 64
CANARY = -7.25


@pytest.fixture(scope="module")
def env():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import precision_gemm_amd as pg
    pg._load()
    return torch, pg


def log(msg):
    sys.stdout.write(msg + "\n")
    sys.stdout.flush()


class Strided:
    """A row-major operand of `rows` x `cols` used elements with row stride
    `ld`, as a flat host buffer (only the used rows written; numpy's zeroed
    pages cost nothing until touched) and a device buffer with guard bands."""

    def __init__(self, torch, rows, cols, ld, values):
        self.rows, self.cols, self.ld = rows, cols, ld
        self.n = 0 if rows == 0 else (rows - 1) * ld + cols
        self.host = np.zeros(max(1, self.n), np.float32)
        if rows:
            np.lib.stride_tricks.as_strided(self.host, (rows, cols), (4 * ld, 4))[:] = values
        dev = torch.device("cuda:0")
        self.dev = torch.zeros(self.n + 2 * GUARD, dtype=torch.float32, device=dev)
        self.dev[:GUARD] = CANARY
        self.dev[GUARD + self.n:] = CANARY
        if rows:
            self.window().copy_(torch.from_numpy(np.ascontiguousarray(values, np.float32)))

    @property
    def ptr(self):
        return self.dev.data_ptr() + 4 * GUARD

    def window(self):
        return self.dev.as_strided((self.rows, self.cols), (self.ld, 1), GUARD)

    def take_and_check_rest(self, torch):
        """The window's values; asserts that nothing outside it moved."""
        got = self.window().cpu().numpy()
        self.window().zero_()
        assert torch.all(self.dev[:GUARD] == CANARY) and \
            torch.all(self.dev[GUARD + self.n:] == CANARY), "a guard band was overwritten"
        assert int(torch.count_nonzero(self.dev[GUARD:GUARD + self.n])) == 0, \
            "C changed outside its window"
        return got


def ints(rng, shape):
    return rng.integers(-3, 4, shape).astype(np.float32)


def run_wide_case(env, tA, tB, M, N, K, ld, alpha, beta, variant, seed):
    torch, pg = env
    rng = np.random.default_rng(seed)
    a_rows, a_cols = (K, M) if tA else (M, K)
    b_rows, b_cols = (N, K) if tB else (K, N)
    A = Strided(torch, a_rows, a_cols, ld, ints(rng, (a_rows, a_cols)))
    B = Strided(torch, b_rows, b_cols, ld, ints(rng, (b_rows, b_cols)))
    Cin = ints(rng, (M, N))
    C = Strided(torch, M, N, ld, Cin)
    log(f"[wide] tA={tA} tB={tB} M={M} N={N} K={K} ld={ld} variant={variant} "
        f"({(A.n + B.n + C.n) * 4 / 2**30:.1f} GiB)")
    dev = torch.device("cuda:0")
    st = pg.sgemm_strided_batched_variant(tA, tB, M, N, K, alpha, A.ptr, ld, B.ptr, ld, beta,
                                          C.ptr, ld, 1, 0, 0, 0, variant,
                                          stream=torch.cuda.current_stream(dev).cuda_stream,
                                          check=False)
    torch.cuda.synchronize(dev)
    assert st == 0, (st, pg.sgemm_status_string(st))
    got = C.take_and_check_rest(torch)
    ref, _ = oracle.sgemm_rows(tA, tB, M, N, K, alpha, A.host, ld, B.host, ld, beta, C.host, ld,
                               want_S=False)
    want = ref[0].astype(np.float32)
    assert np.array_equal(ref[0], want.astype(np.float64))
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} mismatches, first {bad[:3].tolist()}"
    del A, B, C


@pytest.mark.parametrize("tA,tB", [(0, 0), (0, 1), (1, 0), (1, 1)])
@pytest.mark.parametrize("ld", [1 << 21, (1 << 24) + 4])
def test_any_leading_dimension(env, tA, tB, ld):
    """Every leading dimension at once at 2^21 (the first the 32-bit in-tile
    offsets cannot take) and past 2^24, each transpose pair, ragged M, N and
    a K whose first K-step is partial; the automatic choice (the 64-bit-
    addressed tile) and its forced form."""
    _, pg = env
    run_wide_case(env, tA, tB, 36, 68, 40, ld, 2.0, 0.5, -1, seed=ld % 1000 + 2 * tA + tB)
    if ld == 1 << 21:
        run_wide_case(env, tA, tB, 100, 132, 72, ld, -1.0, 0.0, pg.VARIANT_W64x64, seed=7)


@pytest.mark.parametrize("tA,tB", [(0, 0), (1, 1)])
def test_any_leading_dimension_unaligned(env, tA, tB):
    """An odd leading dimension above 2^21: the 1-float form of the
    64-bit-addressed tile."""
    run_wide_case(env, tA, tB, 33, 65, 37, (1 << 22) + 1, 1.0, 2.0, -1, seed=11 + tA)


def test_wide_tile_equals_the_plain_tile(env):
    """At ordinary leading dimensions the 64-bit-addressed tile multiplies in
    the same order as the plain 64 x 64 tile: the same bits on fp32 inputs."""
    torch, pg = env
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(5)
    for tA, tB in ((0, 0), (0, 1), (1, 0), (1, 1)):
        M, N, K = 300, 196, 333 if (tA == 1 and tB == 0) else 332
        A = torch.from_numpy(rng.uniform(-1, 1, M * K).astype(np.float32)).to(dev)
        B = torch.from_numpy(rng.uniform(-1, 1, K * N).astype(np.float32)).to(dev)
        C0 = torch.from_numpy(rng.uniform(-1, 1, M * N).astype(np.float32)).to(dev)
        lda, ldb = (M if tA else K), (K if tB else N)
        outs = []
        for v in (pg.VARIANT_S64x64, pg.VARIANT_W64x64, pg.VARIANT_S64x64_V1,
                  pg.VARIANT_W64x64_V1):
            C = C0.clone()
            st = pg.sgemm_strided_batched_variant(tA, tB, M, N, K, 0.75, A, lda, B, ldb, -1.5,
                                                  C, N, 1, 0, 0, 0, v, check=False)
            torch.cuda.synchronize(dev)
            if st == -18:  # K not a multiple of 4: no 4-float form
                outs.append(None)
                continue
            assert st == 0
            outs.append(C.cpu().numpy())
        if outs[0] is not None:
            assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32)), (tA, tB)
        assert np.array_equal(outs[2].view(np.uint32), outs[3].view(np.uint32)), (tA, tB)


def check_rows(A, lda, B, ldb, Cin, got, tA, tB, M, N, K, alpha, beta, bands):
    for r0, r1 in bands:
        ref, _ = oracle.sgemm_rows(tA, tB, M, N, K, alpha, A, lda, B, ldb, beta, Cin, N,
                                   rows=(r0, r1), want_S=False)
        want = ref[0].astype(np.float32)
        assert np.array_equal(ref[0], want.astype(np.float64))
        g = got[r0 * N:r1 * N].reshape(r1 - r0, N)
        bad = np.argwhere(g != want)
        assert bad.size == 0, f"rows {r0}..{r1}: {len(bad)} mismatches, first {bad[:3].tolist()}"


@pytest.mark.parametrize("tA", [0, 1])
def test_operand_larger_than_2_gib(env, tA):
    """A of 40000 x 16384 floats (2.6 GB): the loaders' buffer windows start
    capped at 2^31 - 1 bytes and count down to the exact bytes left. Every
    loader kind (register-staged tiles, the K-split tile, the direct-to-LDS
    tile and streaming kernel) on bands at both ends and across the 2^31-byte
    mark of A."""
    torch, pg = env
    dev = torch.device("cuda:0")
    M, N, K = 40000, 64, 16384
    rng = np.random.default_rng(40 + tA)
    log(f"[2GiB] drawing A ({M}x{K}, transA={tA})")
    a8 = rng.integers(-3, 4, M * K, dtype=np.int8)
    A = a8.astype(np.float32)
    B = ints(rng, K * N)
    Cin = ints(rng, M * N)
    dA = torch.from_numpy(a8).to(dev).to(torch.float32)
    del a8
    dB = torch.from_numpy(B).to(dev)
    lda, ldb = (M if tA else K), N
    # the row (or k) where A's bytes pass 2^31
    cross = (1 << 31) // (4 * lda)
    bands = [(0, 128), (M - 160, M)]
    if not tA:
        bands.append((cross - 64, cross + 64))
    for v in (-1, pg.VARIANT_M128x128, pg.VARIANT_S64x64_K2, pg.VARIANT_M128x128_DMA,
              pg.VARIANT_T64x64, pg.VARIANT_L256x128):
        dC = torch.from_numpy(Cin).to(dev)
        log(f"[2GiB] transA={tA} variant={v}")
        st = pg.sgemm_strided_batched_variant(tA, 0, M, N, K, 1.0, dA, lda, dB, ldb, 2.0, dC, N,
                                              1, 0, 0, 0, v,
                                              stream=torch.cuda.current_stream(dev).cuda_stream,
                                              check=False)
        torch.cuda.synchronize(dev)
        assert st == 0, (v, st)
        check_rows(A, lda, B, ldb, Cin, dC.cpu().numpy(), tA, 0, M, N, K, 1.0, 2.0, bands)
    del dA


@pytest.mark.parametrize("tA,M,K", [(0, 34_000_000, 8), (1, 270_000_000, 4)])
def test_matrix_vector_taller_than_one_launch(env, tA, M, K):
    """y = op(A) x with more rows than one launch's grid holds (the row-block
    kernels launch several grids, each told its first row): bands at both
    ends and across every launch boundary."""
    torch, pg = env
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(50 + tA)
    log(f"[tall gemv] transA={tA} M={M} K={K}")
    a8 = rng.integers(-3, 4, M * K, dtype=np.int8)
    A = a8.astype(np.float32)
    x = ints(rng, K)
    Cin = ints(rng, M)
    dA = torch.from_numpy(a8).to(dev).to(torch.float32)
    del a8
    dx = torch.from_numpy(x).to(dev)
    dC = torch.full((M + 2 * GUARD,), CANARY, dtype=torch.float32, device=dev)
    dC[GUARD:GUARD + M] = torch.from_numpy(Cin).to(dev)
    lda = M if tA else K
    assert pg.sgemm_select_variant(tA, 1, M, 1, K, 1, 1, 256) == pg.VARIANT_GEMV
    st = pg.sgemm_strided_batched(tA, 1, M, 1, K, 1.0, dA, lda, dx, K, -1.0,
                                  dC.data_ptr() + 4 * GUARD, 1, 1, 0, 0, 0,
                                  stream=torch.cuda.current_stream(dev).cuda_stream, check=False)
    torch.cuda.synchronize(dev)
    assert st == 0, st
    whole = dC.cpu().numpy()
    assert np.all(whole[:GUARD] == CANARY) and np.all(whole[GUARD + M:] == CANARY)
    got = whole[GUARD:GUARD + M]
    # launch boundaries: 2^31 - 1 work-items per grid over 256 threads and 4
    # rows per workgroup, or 512 threads and 64 rows
    per_launch = ((1 << 31) - 1) // 512 * 64 if tA else ((1 << 31) - 1) // 256 * 4
    bands = [(0, 256), (M - 256, M)]
    bands += [(b - 128, b + 128) for b in range(per_launch, M, per_launch)]
    assert len(bands) > 2
    for r0, r1 in bands:
        ref, _ = oracle.sgemm_rows(tA, 1, M, 1, K, 1.0, A, lda, x, K, -1.0, Cin, 1,
                                   rows=(r0, r1), want_S=False)
        want = ref[0, :, 0].astype(np.float32)
        bad = np.flatnonzero(got[r0:r1] != want)
        assert bad.size == 0, f"rows {r0}..{r1}: {bad.size} mismatches, first {bad[:3] + r0}"
    del dA
