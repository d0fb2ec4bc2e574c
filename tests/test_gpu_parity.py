"""GPU parity: the HIP library against the CPU oracle, through the C ABI.

Floating-point cases must meet the acceptance bound
|C_gpu - ref| <= 2e-6 * max(K,1) * (|alpha| * S + |beta| * |C_in|) elementwise.
Integer-valued cases (entries in [-3, 3], alpha/beta in {1, 2, -1, 0.5})
make every partial sum exact in fp32, so there the GPU must equal the oracle
bit for bit whatever the summation order.

Every launch also checks that nothing outside the M x N windows of C moved:
the device buffer carries guard bands before and after it, and ld padding
and gaps between batch items must keep their input bits.
"""
import itertools
import sys

import numpy as np
import pytest

import oracle
import precision_gemm_amd as pg_constants  # module constants only; the library loads in env()
import workloads
from workloads import Workload

pytestmark = pytest.mark.gpu

# every kernel variant that takes any shape (the enum of the C header,
# mirrored by the binding); the GEMV kernel, which only takes N == 1 or M == 1,
# has tests of its own
# (the persistent variants, which only take grids that split evenly over the
# compute units, are tested in test_gpu_persistent.py)
ALL_VARIANTS = [v for v in range(pg_constants.VARIANT_COUNT)
                if v not in (pg_constants.VARIANT_GEMV, pg_constants.VARIANT_P128x128,
                             pg_constants.VARIANT_P64x64)]

GUARD = 64  # floats of canary before and after each device buffer (keeps 256-B alignment)


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


def c_window_mask(w: Workload, n: int) -> np.ndarray:
    """Flat positions of C that the call may write."""
    mask = np.zeros(n, bool)
    if w.M == 0 or w.N == 0:
        return mask
    for b in range(w.batch):
        base = b * w.SC
        rows = base + np.arange(w.M)[:, None] * w.LDC + np.arange(w.N)[None, :]
        mask[rows.reshape(-1)] = True
    return mask


def c_items(flat: np.ndarray, w: Workload) -> np.ndarray:
    """(batch, M, N) view of a flat C buffer."""
    out = np.empty((w.batch, w.M, w.N), flat.dtype)
    for b in range(w.batch):
        out[b] = np.lib.stride_tricks.as_strided(
            flat[b * w.SC:], (w.M, w.N), (w.LDC * flat.itemsize, flat.itemsize))
    return out


def run_gpu(env, w: Workload, A, B, C, variant=-1, c_offset=0):
    """Launch on cuda:0; returns (status, C after the call as a flat array)."""
    torch, pg = env
    dev = torch.device("cuda:0")

    def put(x, extra=0):
        buf = torch.full((x.size + 2 * GUARD + extra,), -7.25, dtype=torch.float32, device=dev)
        buf[GUARD + extra:GUARD + extra + x.size] = torch.from_numpy(x).to(dev)
        return buf, GUARD + extra

    dA, oa = put(A)
    dB, ob = put(B)
    dC, oc = put(C, c_offset)
    pa, pb, pc = (t.data_ptr() + 4 * o for t, o in ((dA, oa), (dB, ob), (dC, oc)))
    st = pg.sgemm_strided_batched_variant(
        w.trans_a, w.trans_b, w.M, w.N, w.K, w.alpha, pa, w.LDA, pb, w.LDB, w.beta, pc, w.LDC,
        w.batch, w.SA, w.SB, w.SC, variant, stream=torch.cuda.current_stream(dev).cuda_stream,
        check=False)
    torch.cuda.synchronize(dev)
    whole = dC.cpu().numpy()
    guard_ok = (np.all(whole[:oc] == np.float32(-7.25)) and
                np.all(whole[oc + C.size:] == np.float32(-7.25)))
    assert guard_ok, "a guard band around C was overwritten"
    return st, whole[oc:oc + C.size]


def check_against_oracle(w, A, B, C, got, exact=False, rows=None, batches=None):
    ref, S = oracle.sgemm_rows(w.trans_a, w.trans_b, w.M, w.N, w.K, w.alpha, A, w.LDA, B,
                               w.LDB, w.beta, C, w.LDC, batch=w.batch, stride_a=w.SA,
                               stride_b=w.SB, stride_c=w.SC, rows=rows, batches=batches)
    r0, r1 = rows or (0, w.M)
    b0, b1 = batches or (0, w.batch)
    g = c_items(got, w)[b0:b1, r0:r1]
    cin = c_items(C, w)[b0:b1, r0:r1]
    if exact:
        want = ref.astype(np.float32)
        assert np.array_equal(ref, want.astype(np.float64)), "integer case not exact in fp32"
        bad = np.argwhere(g != want)
        assert bad.size == 0, f"{w}: {len(bad)} mismatches, first {bad[:3].tolist()} " \
                              f"got {g[tuple(bad[0])]} want {want[tuple(bad[0])]}"
        return None
    rep = oracle.bound_check(g, ref, S, cin, w.alpha, w.beta, w.K)
    assert rep.ok, f"{w.name}: {rep}"
    return rep


def check_untouched(w, C, got):
    mask = c_window_mask(w, C.size)
    assert np.array_equal(got[~mask].view(np.uint32), C[~mask].view(np.uint32)), \
        "C changed outside its M x N windows"


# ------------------------------------------------------------------ the five workloads

@pytest.mark.parametrize("name", [w.name for w in workloads.CONFIGS])
def test_workload_parity(env, name):
    """Full-size workloads in the launch configuration the benchmark times
    (automatic variant). Small ones are checked whole; the 4092^3 product on
    sampled row bands (first, middle, the ragged last band) and the batched
    one on sampled batch items."""
    w = workloads.BY_NAME[name]
    A, B, C = workloads.make_inputs(w)
    log(f"[parity] {name} M={w.M} N={w.N} K={w.K} batch={w.batch}")
    st, got = run_gpu(env, w, A, B, C)
    assert st == 0
    check_untouched(w, C, got)
    if name == "sgemm_4092":
        for rows in ((0, 96), (2000, 2064), (w.M - 100, w.M)):
            rep = check_against_oracle(w, A, B, C, got, rows=rows)
            log(f"  rows {rows}: {rep}")
    elif name.startswith("bmm"):
        for b in (0, 37, w.batch - 1):
            rep = check_against_oracle(w, A, B, C, got, batches=(b, b + 1))
            log(f"  batch {b}: {rep}")
    else:
        rep = check_against_oracle(w, A, B, C, got)
        log(f"  {rep}")


@pytest.mark.parametrize("tA,tB,M,N", [(0, 0, 16384, 64), (1, 1, 64, 16384)])
def test_streaming_kernel_at_full_size(env, tA, tB, M, N):
    """The skinny product in the layouts the automatic dispatch streams through
    the 64 x 64 streaming kernel (the long operand, 268 MB, contiguous in k;
    the short one contiguous along its outputs), fp32 with beta = 1, checked
    on the first and last row bands against the bound."""
    torch, pg = env
    w = Workload("stream_full", tA, tB, M, N, 4096, 1.0, 1.0, seed=61)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert pg.sgemm_select_variant(tA, tB, M, N, 4096, 1, 1, cus) == pg.VARIANT_T64x64
    A, B, C = workloads.make_inputs(w)
    log(f"[parity] streaming kernel tA={tA} tB={tB} {M}x{N}x4096")
    st, got = run_gpu(env, w, A, B, C)
    assert st == 0
    check_untouched(w, C, got)
    for rows in ((0, 48), (M - 48, M)):
        rep = check_against_oracle(w, A, B, C, got, rows=rows)
        log(f"  rows {rows}: {rep}")


def test_workload_4092_sampled_elements(env):
    """Random elements across the whole 4092^3 output, each recomputed alone."""
    w = workloads.HEADLINE
    A, B, C = workloads.make_inputs(w)
    st, got = run_gpu(env, w, A, B, C)
    assert st == 0
    rng = np.random.default_rng(123)
    n = 4000
    is_ = np.concatenate([rng.integers(0, w.M, n), np.full(64, w.M - 1), np.arange(64)])
    js = np.concatenate([rng.integers(0, w.N, n), rng.integers(0, w.N, 64),
                         np.full(64, w.N - 1)])
    bs = np.zeros_like(is_)
    ref, S = oracle.sgemm_elements(0, 0, w.K, w.alpha, A, w.LDA, B, w.LDB, w.beta, C, w.LDC,
                                   bs, is_, js)
    g = got[is_ * w.LDC + js]
    cin = C[is_ * w.LDC + js]
    rep = oracle.bound_check(g, ref, S, cin, w.alpha, w.beta, w.K)
    log(f"  sampled elements: {rep}")
    assert rep.ok


# ------------------------------------------------------------------ variant sweeps

SIZES = [1, 2, 3, 4, 5, 7, 8, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257]
# multiples of 4 (the 4-float variants' domain), ragged against every tile size
SIZES4 = [4, 8, 12, 16, 20, 28, 32, 36, 60, 64, 68, 124, 128, 132, 252, 256, 260]


def sweep_shapes(n, seed):
    rng = np.random.default_rng(seed)
    shapes = {(1, 1, 1), (4, 4, 4), (257, 257, 257), (256, 128, 16), (255, 129, 33),
              (260, 132, 20), (132, 68, 64), (68, 196, 96), (200, 72, 48)}
    while len(shapes) < n:
        pool = SIZES4 if len(shapes) % 2 else SIZES
        shapes.add(tuple(int(x) for x in rng.choice(pool, 3)))
    return sorted(shapes)


def canonical_vectors(tA, tB, M, N, K, lda, ldb):
    """A vector operand whose k elements are adjacent (op(B) with N == 1, B
    untransposed, ldb == 1; op(A) with M == 1, A transposed, lda == 1) is
    described k-contiguous, the same memory, as the library does before it
    picks the load width."""
    if N == 1 and tB == 0 and ldb == 1 and 1 < K:
        tB, ldb = 1, K
    if M == 1 and tA == 1 and lda == 1 and 1 < K:
        tA, lda = 0, K
    return tA, tB, lda, ldb


def vec4_possible(w):
    tA, tB, lda, ldb = canonical_vectors(w.trans_a, w.trans_b, w.M, w.N, w.K, w.LDA, w.LDB)
    a_kc, b_kc = tA == 0, tB == 1
    return ((w.K % 4 == 0) if a_kc else (w.M % 4 == 0)) and \
           ((w.K % 4 == 0) if b_kc else (w.N % 4 == 0)) and \
           lda % 4 == 0 and ldb % 4 == 0 and w.SA % 4 == 0 and w.SB % 4 == 0


@pytest.mark.parametrize("variant", ALL_VARIANTS)
def test_integer_sweep_bitwise(env, variant):
    """Every forced variant x transpose pair over ragged sizes, integer inputs:
    bitwise equality with the oracle."""
    _, pg = env
    ab = [(1.0, 0.0), (2.0, 1.0), (-1.0, 0.5), (0.5, 2.0)]
    n_run = 0
    for idx, (M, N, K) in enumerate(sweep_shapes(40, seed=variant)):
        for tA, tB in itertools.product([0, 1], repeat=2):
            alpha, beta = ab[(idx + 2 * tA + tB) % len(ab)]
            pad = 4 if idx % 3 == 0 else 0
            w = Workload(f"int{M}x{N}x{K}", tA, tB, M, N, K, alpha, beta, seed=idx,
                         dist="int3",
                         lda=(M if tA else K) + pad, ldb=(K if tB else N) + pad, ldc=N + pad)
            A, B, C = workloads.make_inputs(w)
            st, got = run_gpu(env, w, A, B, C, variant=variant)
            if not pg.VARIANT_NAMES[variant].endswith("_V1") and not vec4_possible(w):
                assert st == -18, (w, st)
                continue
            assert st == 0, (w, st)
            check_against_oracle(w, A, B, C, got, exact=True)
            check_untouched(w, C, got)
            n_run += 1
    log(f"  variant {variant}: {n_run} bitwise cases")
    assert n_run > 20


@pytest.mark.parametrize("variant", ALL_VARIANTS)
def test_float_sweep_bound(env, variant):
    """Random fp32 inputs, several tiles plus ragged tails in every dimension,
    all transposes, padded leading dimensions, batches with gaps."""
    shapes = [(300, 200, 100), (513, 257, 77), (96, 160, 520), (640, 384, 36)]
    for (M, N, K), (tA, tB) in itertools.product(shapes, itertools.product([0, 1], repeat=2)):
        w = Workload(f"f{M}x{N}x{K}", tA, tB, M, N, K, 0.75, -1.5, seed=M + N + K,
                     dist="normal", batch=2, lda=(M if tA else K) + 8,
                     ldb=(K if tB else N) + 4, ldc=N + 12)
        w = Workload(**{**w.__dict__, "stride_a": w.SA + 16, "stride_b": w.SB + 4,
                        "stride_c": w.SC + 20})
        A, B, C = workloads.make_inputs(w)
        st, got = run_gpu(env, w, A, B, C, variant=variant)
        if not pg_constants.VARIANT_NAMES[variant].endswith("_V1") and not vec4_possible(w):
            assert st == -18
            continue
        assert st == 0, (w, st)
        check_against_oracle(w, A, B, C, got)
        check_untouched(w, C, got)


# ------------------------------------------------------------------ special cases

def random_shapes(n, seed):
    """Seeded shapes for the automatic dispatch: M, N, K log-uniform (1 to a few
    thousand), every transpose pair, batches, padded or minimal leading
    dimensions (which decide the 4-float path), bounded in size."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        if rng.random() < 0.4:
            M, N = (int(np.exp(rng.uniform(0, np.log(3000)))) for _ in range(2))
        else:
            M, N = (int(rng.integers(200, 3000)) for _ in range(2))
        K = int(np.exp(rng.uniform(0, np.log(6000))))
        gemv = rng.random() < 0.1  # a matrix-vector product, either way round
        if gemv:
            if rng.random() < 0.5:
                N = 1
            else:
                M = 1
        aligned = rng.random() < 0.75  # most real shapes are multiples of 4
        if aligned:
            M, N, K = (x if x == 1 and gemv else max(4, x // 4 * 4) for x in (M, N, K))
        batch = int(rng.choice([1, 1, 1, 2, 3, 8]))
        if M * N * batch > 4_000_000 or (M + N) * K * batch > 16_000_000:
            continue
        tA, tB = int(rng.integers(0, 2)), int(rng.integers(0, 2))
        pad = (lambda: int(rng.choice([0, 0, 4, 8]))) if aligned else \
            (lambda: int(rng.choice([0, 1, 3])))
        a_row, b_row = (M if tA else K), (K if tB else N)
        w = Workload(f"rnd{len(out)}", tA, tB, M, N, K, float(rng.choice([1.0, -0.5, 2.0])),
                     float(rng.choice([0.0, 1.0, 0.25])), seed=1000 + len(out), batch=batch,
                     lda=a_row + pad(), ldb=b_row + pad(), ldc=N + pad())
        out.append(w)
    return out


def test_automatic_dispatch_random_shapes(env):
    """120 seeded shapes through the automatic dispatch (every rule: the GEMV
    kernels, the 32 x 64 and 64 x 32 streaming tiles, the K-split and plain 64 x 64 tiles, the 128 x 128
    tile, the 1-float variant), each checked against the oracle on its first
    and last rows of every batch item, and for writes outside C's windows."""
    torch, pg = env
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    seen = set()
    for w in random_shapes(120, seed=77):
        A, B, C = workloads.make_inputs(w)
        log(f"[random] {w.name} {'NT'[w.trans_a]}{'NT'[w.trans_b]} {w.M}x{w.N}x{w.K} "
            f"b{w.batch} ld {w.LDA},{w.LDB},{w.LDC}")
        st, got = run_gpu(env, w, A, B, C)
        assert st == 0, (w, st)
        for rows in ((0, min(w.M, 6)), (max(0, w.M - 3), w.M)):
            check_against_oracle(w, A, B, C, got, rows=rows)
        check_untouched(w, C, got)
        vec4 = vec4_possible(w)
        tA, tB, _, _ = canonical_vectors(w.trans_a, w.trans_b, w.M, w.N, w.K, w.LDA, w.LDB)
        seen.add(pg.sgemm_select_variant(tA, tB, w.M, w.N, w.K, w.batch, 1 if vec4 else 0, cus))
    for v in (pg.VARIANT_T32x64, pg.VARIANT_T64x32, pg.VARIANT_S64x64, pg.VARIANT_S64x64_K2,
              pg.VARIANT_M128x128, pg.VARIANT_S64x64_V1, pg.VARIANT_GEMV):
        assert v in seen, f"no shape reached {pg.VARIANT_NAMES[v]}"


def test_beta_zero_ignores_nan_in_c(env):
    w = Workload("nanc", 0, 0, 130, 70, 40, 1.0, 0.0, seed=3)
    A, B, C = workloads.make_inputs(w)
    C[:] = np.nan
    st, got = run_gpu(env, w, A, B, C)
    assert st == 0
    assert np.isfinite(c_items(got, w)).all()
    check_against_oracle(w, A, B, C, got)


@pytest.mark.parametrize("alpha,K", [(0.0, 50), (1.0, 0), (0.0, 0)])
@pytest.mark.parametrize("beta", [0.0, 1.0, -2.5])
def test_alpha_zero_or_k_zero_scales_c(env, alpha, K, beta):
    w = Workload("scale", 0, 0, 77, 33, K, alpha, beta, seed=5, batch=3, ldc=40)
    A, B, C = workloads.make_inputs(w)
    if alpha == 0.0 and K:
        A[:] = np.nan  # A and B are not read
    st, got = run_gpu(env, w, A, B, C)
    assert st == 0
    want = c_items(C, w) * np.float32(beta)
    if beta == 0.0:
        want = np.zeros_like(want)
    assert np.array_equal(c_items(got, w), want)
    check_untouched(w, C, got)


@pytest.mark.parametrize("dims", [(0, 5, 5, 1), (5, 0, 5, 1), (5, 5, 5, 0)])
def test_empty_problems_touch_nothing(env, dims):
    M, N, K, batch = dims
    w = Workload("empty", 0, 0, M, N, K, 1.0, 0.0, seed=1, batch=batch, lda=8, ldb=8, ldc=8,
                 stride_a=64, stride_b=64, stride_c=64)
    A = np.ones(64, np.float32)
    B = np.ones(64, np.float32)
    C = np.arange(64, dtype=np.float32)
    st, got = run_gpu(env, w, A, B, C)
    assert st == 0
    assert np.array_equal(got, C)


def test_broadcast_and_strided_batches(env):
    """strideA = 0 (one A shared by all items), B and C items with gaps."""
    w = Workload("bcast", 0, 1, 200, 136, 96, 1.0, 0.5, seed=9, batch=5,
                 stride_a=0, stride_b=136 * 96 + 12, stride_c=200 * 136 + 36)
    A, B, C = workloads.make_inputs(w)
    for variant in (-1, *ALL_VARIANTS):
        st, got = run_gpu(env, w, A, B, C, variant=variant)
        assert st == 0
        check_against_oracle(w, A, B, C, got)
        check_untouched(w, C, got)


def test_unaligned_pointers_use_the_scalar_variant(env):
    """C offset by one float and odd leading dimensions: auto-dispatch must
    still give correct results (the 1-float-load variant)."""
    w = Workload("odd", 1, 1, 101, 67, 45, -1.0, 2.0, seed=11, lda=103, ldb=47, ldc=69)
    A, B, C = workloads.make_inputs(w)
    st, got = run_gpu(env, w, A, B, C, c_offset=1)
    assert st == 0
    check_against_oracle(w, A, B, C, got)
    check_untouched(w, C, got)


def test_deterministic(env):
    w = Workload("det", 0, 0, 1000, 1000, 1000, 1.0, 0.5, seed=13)
    A, B, C = workloads.make_inputs(w)
    _, g1 = run_gpu(env, w, A, B, C)
    _, g2 = run_gpu(env, w, A, B, C)
    assert np.array_equal(g1.view(np.uint32), g2.view(np.uint32))


def test_concurrent_host_threads(env):
    """Calls from several host threads at once, each on a stream of its own
    (the library keeps no per-call state; the CU-count cache is atomic),
    give the bits of the same calls made one at a time: tile kernels, split-K
    with a workspace, a GEMV and a few-row GEMV written transposed."""
    import threading
    torch, pg = env
    dev = torch.device("cuda:0")
    cases = [Workload("thr0", 0, 0, 300, 200, 500, 1.0, 0.5, seed=41),
             Workload("thr1", 1, 1, 257, 129, 1040, -1.5, 0.0, seed=42),
             Workload("thr2", 0, 1, 64, 96, 4096, 1.0, 1.0, seed=43, batch=3),
             Workload("thr3", 1, 0, 640, 320, 96, 0.5, -2.0, seed=44),
             Workload("thr4", 0, 1, 2000, 1, 1028, 1.0, 0.5, seed=45),
             Workload("thr5", 0, 1, 4, 4096, 1028, -1.0, 1.0, seed=46)]

    def call(w, dA, dB, dC, stream, ws):
        # thr2 splits K across workgroups through its own workspace
        if ws is not None:
            return pg.sgemm_strided_batched_ws(
                w.trans_a, w.trans_b, w.M, w.N, w.K, w.alpha, dA, w.LDA, dB, w.LDB, w.beta,
                dC, w.LDC, w.batch, w.SA, w.SB, w.SC, ws, stream=stream, check=False)
        return pg.sgemm_strided_batched(w.trans_a, w.trans_b, w.M, w.N, w.K, w.alpha, dA,
                                        w.LDA, dB, w.LDB, w.beta, dC, w.LDC, w.batch, w.SA,
                                        w.SB, w.SC, stream=stream, check=False)

    def workspace(w):
        n = pg.sgemm_workspace_size(w.trans_a, w.trans_b, w.M, w.N, w.K, w.batch)
        return torch.empty(max(1, n // 4), device=dev) if w.name == "thr2" else None

    inputs = [workloads.make_inputs(w) for w in cases]
    want = []
    for w, (A, B, C) in zip(cases, inputs):
        dA, dB, dC = (torch.from_numpy(x).to(dev) for x in (A, B, C))
        ws = workspace(w)
        assert call(w, dA, dB, dC, torch.cuda.current_stream(dev).cuda_stream, ws) == 0
        torch.cuda.synchronize(dev)
        want.append(dC.cpu().numpy().view(np.uint32).copy())
        check_against_oracle(w, A, B, C, dC.cpu().numpy())

    log(f"[threads] {len(cases)} host threads x 25 calls")
    errors = []

    def worker(k):
        try:
            w, (A, B, C) = cases[k], inputs[k]
            stream = torch.cuda.Stream(dev)
            with torch.cuda.stream(stream):
                dA, dB, dC0 = (torch.from_numpy(x).to(dev) for x in (A, B, C))
                ws = workspace(w)
                for it in range(25):
                    dC = dC0.clone()
                    st = call(w, dA, dB, dC, stream.cuda_stream, ws)
                    if st != 0:
                        errors.append((k, it, "status", st))
                        return
                    got = dC.cpu().numpy().view(np.uint32)  # waits for this stream
                    if not np.array_equal(got, want[k]):
                        errors.append((k, it, "bits differ"))
                        return
                stream.synchronize()
        except Exception as e:  # reported by the main thread
            errors.append((k, repr(e)))

    threads = [threading.Thread(target=worker, args=(k,)) for k in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=100)
    assert not any(t.is_alive() for t in threads), "a calling thread did not finish"
    assert not errors, errors


def test_graph_capture_replays(env):
    """Calls captured into a HIP graph (the library only launches kernels on
    the caller's stream and allocates nothing) replay to the eager bits,
    replay after replay, with other eager work in between: a streaming-tile
    call, a K-split tile call, a split-K call whose reduction kernel is
    captured too (workspace allocated before the capture), and both GEMV
    kernels."""
    torch, pg = env
    dev = torch.device("cuda:0")
    cases = [Workload("g_t32", 0, 1, 256, 192, 700, 1.0, 0.5, seed=51),
             Workload("g_k2", 1, 0, 1000, 1000, 1000, -1.0, 2.0, seed=52),
             Workload("g_split", 0, 0, 128, 192, 8192, 0.5, 1.0, seed=53, batch=2),
             Workload("g_gemv", 0, 1, 3000, 1, 1028, 1.5, 0.5, seed=54),
             Workload("g_gemv_t", 1, 1, 2048, 1, 900, -1.0, 1.0, seed=55, batch=2)]
    bufs, want = [], []
    for w in cases:
        A, B, C = workloads.make_inputs(w)
        dA, dB, dC0 = (torch.from_numpy(x).to(dev) for x in (A, B, C))
        n = pg.sgemm_workspace_size(w.trans_a, w.trans_b, w.M, w.N, w.K, w.batch)
        ws = torch.empty(max(1, n // 4), device=dev) if w.name == "g_split" else None
        if w.name == "g_split":
            assert n > 0, "the split-K case must split"
        dC = dC0.clone()
        bufs.append((w, dA, dB, dC0, dC, ws))

    def call(w, dA, dB, dC, ws):
        if ws is not None:
            return pg.sgemm_strided_batched_ws(
                w.trans_a, w.trans_b, w.M, w.N, w.K, w.alpha, dA, w.LDA, dB, w.LDB, w.beta, dC,
                w.LDC, w.batch, w.SA, w.SB, w.SC, ws)
        return pg.sgemm_strided_batched(w.trans_a, w.trans_b, w.M, w.N, w.K, w.alpha, dA,
                                        w.LDA, dB, w.LDB, w.beta, dC, w.LDC, w.batch, w.SA,
                                        w.SB, w.SC)

    # eager reference bits (this also fills the library's CU-count cache)
    for w, dA, dB, dC0, dC, ws in bufs:
        dC.copy_(dC0)
        call(w, dA, dB, dC, ws)
    torch.cuda.synchronize(dev)
    want = [dC.cpu().numpy().view(np.uint32).copy() for (_, _, _, _, dC, _) in bufs]

    assert pg.sgemm_select_variant(0, 1, 3000, 1, 1028, 1, 1, 256) == pg.VARIANT_GEMV
    log(f"[graph] capture {len(bufs)} calls")
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for w, dA, dB, dC0, dC, ws in bufs:
                call(w, dA, dB, dC, ws)
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize(dev)

    other = torch.rand(300, 300, device=dev)
    for rep in range(4):
        for w, dA, dB, dC0, dC, ws in bufs:
            dC.copy_(dC0)  # beta != 0: every replay starts from the same C
        torch.cuda.synchronize(dev)
        g.replay()
        torch.cuda.synchronize(dev)
        for k, (w, dA, dB, dC0, dC, ws) in enumerate(bufs):
            got = dC.cpu().numpy().view(np.uint32)
            assert np.array_equal(got, want[k]), (rep, w.name)
        # unrelated eager work between replays
        pg.sgemm(0, 0, 300, 300, 300, 1.0, other, 300, other, 300, 0.0, torch.empty_like(other),
                 300)
        torch.cuda.synchronize(dev)


def test_matmul_tensor_wrapper(env):
    torch, pg = env
    dev = torch.device("cuda:0")
    g = torch.Generator(device="cpu").manual_seed(0)
    A = torch.randn(3, 70, 50, generator=g)
    B = torch.randn(3, 60, 50, generator=g)
    C = torch.randn(3, 70, 60, generator=g)
    dC = C.to(dev)
    pg.matmul(A.to(dev), B.to(dev), dC, alpha=2.0, beta=-1.0, transB=True)
    torch.cuda.synchronize(dev)
    want = 2.0 * (A.double() @ B.double().transpose(1, 2)) - C.double()
    S = 2.0 * (A.double().abs() @ B.double().abs().transpose(1, 2)) + C.double().abs()
    err = (dC.cpu().double() - want).abs()
    assert bool((err <= 2e-6 * 50 * S).all())


# ------------------------------------------------------------------ extremes

@pytest.mark.parametrize("tA,tB,M,N", [(0, 1, 4, 8), (0, 1, 12, 1), (1, 1, 8, 1), (0, 0, 1, 8)])
def test_batch_beyond_one_launch(env, tA, tB, M, N):
    """More batch items than one launch's second grid axis holds (65535), for a
    tile kernel and for both GEMV kernels (N == 1, and M == 1 through its
    transpose)."""
    _, pg = env
    w = Workload("manybatch", tA, tB, M, N, 12, 1.0, -1.0, seed=21 + M + N, dist="int3",
                 batch=70000)
    A, B, C = workloads.make_inputs(w)
    gemv = pg.sgemm_select_variant(tA, tB, M, N, 12, 70000, 1, 256) == pg.VARIANT_GEMV
    assert gemv == (M == 1 or N == 1)
    st, got = run_gpu(env, w, A, B, C)
    assert st == 0
    for b0, b1 in ((0, 3), (65534, 65537), (69997, 70000)):
        check_against_oracle(w, A, B, C, got, exact=True, batches=(b0, b1))
    check_untouched(w, C, got)


@pytest.mark.parametrize("which", ["lda", "ldb", "ldc"])
def test_leading_dimension_at_the_limit(env, which):
    """Leading dimensions at 2^21 - 1, the largest the 32-bit-offset kernels take."""
    big = (1 << 21) - 1
    kw = {which: big}
    w = Workload("bigld", 0, 0, 5, 7, 9, 1.5, 0.5, seed=22, **kw)
    A, B, C = workloads.make_inputs(w)
    for variant in (-1, 3):  # the automatic choice (unaligned ld: 1-float loads) and forced
        st, got = run_gpu(env, w, A, B, C, variant=variant)
        assert st == 0
        check_against_oracle(w, A, B, C, got)
        check_untouched(w, C, got)


def test_batch_offsets_beyond_2_pow_31_elements(env):
    """A second batch item more than 2^31 floats (8 GiB) past the first: the
    per-item offsets must be 64-bit. Only the two small windows are copied."""
    torch, pg = env
    dev = torch.device("cuda:0")
    M, N, K = 20, 36, 44
    stride = (1 << 31) + 64
    rng = np.random.default_rng(23)
    big = torch.empty(stride + M * K, dtype=torch.float32, device=dev)  # ~8 GiB
    Bm = rng.integers(-3, 4, (2, K, N)).astype(np.float32)
    Cm = rng.integers(-3, 4, (2, M, N)).astype(np.float32)
    A0 = rng.integers(-3, 4, (M, K)).astype(np.float32)
    A1 = rng.integers(-3, 4, (M, K)).astype(np.float32)
    big[:M * K] = torch.from_numpy(A0.reshape(-1)).to(dev)
    big[stride:stride + M * K] = torch.from_numpy(A1.reshape(-1)).to(dev)
    dB = torch.from_numpy(Bm.reshape(-1)).to(dev)
    dC = torch.from_numpy(Cm.reshape(-1)).to(dev)
    log(f"[extreme] strideA={stride}")
    for variant in (-1, 0, 2, 4, 6):
        dC.copy_(torch.from_numpy(Cm.reshape(-1)))
        st = pg.sgemm_strided_batched_variant(0, 0, M, N, K, 1.0, big, K, dB, N, 2.0, dC, N, 2,
                                              stride, K * N, M * N, variant, check=False)
        torch.cuda.synchronize(dev)
        assert st == 0, variant
        got = dC.cpu().numpy().reshape(2, M, N)
        for b, Ab in ((0, A0), (1, A1)):
            want = Ab.astype(np.float64) @ Bm[b].astype(np.float64) + 2.0 * Cm[b]
            assert np.array_equal(got[b], want.astype(np.float32)), (variant, b)
    del big


@pytest.mark.parametrize("shape", [(1, 1, 100000), (100000, 1, 64), (1, 100000, 64),
                                   (3, 5, 65537), (2047, 3, 1025)])
def test_degenerate_shapes(env, shape):
    """Dot products, single columns and rows, deep ragged K."""
    M, N, K = shape
    for tA, tB in ((0, 0), (1, 1)):
        w = Workload("degen", tA, tB, M, N, K, 1.0, 1.0, seed=M + N + K, dist="int3")
        A, B, C = workloads.make_inputs(w)
        st, got = run_gpu(env, w, A, B, C)
        assert st == 0
        check_against_oracle(w, A, B, C, got, exact=True)


@pytest.mark.parametrize("M,N,K", [(16384, 1, 4096), (1, 16384, 4096), (1, 1, 4096),
                                   (300, 1, 1028), (1, 200, 36), (4096, 1, 2)])
def test_vector_operand_descriptions_agree(env, M, N, K):
    """A vector operand whose k elements are adjacent has two descriptions of
    the same memory: op(B) with N == 1 as B untransposed with ldb == 1 or
    transposed with ldb == K; op(A) with M == 1 as A transposed with lda == 1
    or untransposed with lda == K. Every description gives the same bits,
    within the oracle's bound."""
    base = Workload("vec", 0, 1, M, N, K, 1.0, 0.5, seed=7 * M + N + K, ldb=K)
    A, B, C = workloads.make_inputs(base)
    outs = []
    for tA in ((0, 1) if M == 1 else (0,)):
        for tB in ((0, 1) if N == 1 else (1,)):
            w = Workload("vec", tA, tB, M, N, K, 1.0, 0.5, seed=0, lda=1 if tA else K,
                         ldb=K if tB else 1)
            log(f"[vector] {'NT'[tA]}{'NT'[tB]} {M}x{N}x{K} lda={w.LDA} ldb={w.LDB}")
            st, got = run_gpu(env, w, A, B, C)
            assert st == 0
            check_against_oracle(w, A, B, C, got)
            outs.append(got)
    for got in outs[1:]:
        assert np.array_equal(got.view(np.uint32), outs[0].view(np.uint32))


# ------------------------------------------------------------------ the GEMV kernel

def gemv_cases():
    """(name, tA, tB, M, N, K, lda, ldb, ldc, batch) for the GEMV kernels: N == 1
    and its mirror M == 1; 2 <= N <= 8 with the matrix contiguous in k and its
    mirror 2 <= M <= 8; the matrix contiguous in k (any row count) or along
    the outputs (counts that are multiples of 4); the vector in the
    k-contiguous description and in the stride-1 description the library
    converts; counts on both sides of each kernel's workgroup-size choice; K
    with and without a partial unrolled pass."""
    out = []
    for L in (1, 2, 3, 5, 63, 257, 1000, 4099):
        for K in (4, 12, 1028, 4100):
            if L * K > 6_000_000:
                continue
            pad = 4 if (L + K) % 3 == 0 else 0
            out.append((f"n1_{L}x{K}", 0, 1, L, 1, K, K + pad, K, 1 + (L % 3), 1))
            out.append((f"m1_{L}x{K}", 0, 1, 1, L, K, K, K + pad, L, 1))
    for L in (4, 8, 60, 256, 1000, 4100):
        for K in (4, 36, 1028, 1100):
            if L * K > 6_000_000:
                continue
            pad = 4 if (L + K) % 3 == 0 else 0
            out.append((f"n1t_{L}x{K}", 1, 1, L, 1, K, L + pad, K, 1 + (L % 3), 1))
            out.append((f"m1t_{L}x{K}", 0, 0, 1, L, K, K, L + pad, L, 1))
    # the 64- and 32-wide column blocks (enough of them for a workgroup per CU)
    out.append(("n1t_64", 1, 1, 16384, 1, 68, 16388, 68, 1, 1))
    out.append(("m1t_64", 0, 0, 1, 4096, 132, 132, 4100, 4096, 4))
    out.append(("n1t_32", 1, 1, 8192, 1, 36, 8192, 36, 2, 1))
    # the 8- and 4-wide blocks: few outputs, the latter over K >= 16384
    out.append(("n1t_8", 1, 1, 1000, 1, 1100, 1004, 1100, 1, 1))
    out.append(("n1t_4", 1, 1, 64, 1, 16388, 68, 16388, 1, 1))
    out.append(("m1t_4", 0, 0, 1, 128, 16384, 16384, 132, 128, 2))
    out.append(("m1t_32", 0, 0, 1, 2048, 100, 100, 2052, 2048, 4))
    # a few vectors against a matrix contiguous in k: B's rows (any N up to 8)
    # or B stored K x N (N a multiple of 4)
    for L in (1, 3, 257, 4099):
        for N in (2, 3, 4, 5, 8):
            for K in (4, 1028):
                if L * K > 5_000_000:
                    continue
                out.append((f"nv{N}_{L}x{K}", 0, 1, L, N, K, K + 4 * (L % 2), K, N + L % 3, 1))
                if N % 4 == 0:
                    out.append((f"nv{N}n_{L}x{K}", 0, 0, L, N, K, K, N + 4 * (L % 2), N, 2))
                # the mirror: N rows of A against B stored L x K, C written
                # through the transpose
                out.append((f"mv{N}_{L}x{K}", 0, 1, N, L, K, K + 4 * (L % 2), K + 4, L + L % 3, 1))
                if N % 4 == 0:
                    out.append((f"mv{N}t_{L}x{K}", 1, 1, N, L, K, N + 4 * (L % 2), K, L, 2))
    for L, K in ((300, 1028), (1000, 260)):
        out.append((f"n1_vec_{L}x{K}", 0, 0, L, 1, K, K, 1, 1, 3))
        out.append((f"m1_vec_{L}x{K}", 1, 1, 1, L, K, 1, K + 4, L, 3))
    return out


@pytest.mark.parametrize("variant", [-1, pg_constants.VARIANT_GEMV])
def test_gemv_bitwise(env, variant):
    """The GEMV kernel, auto-dispatched and forced, on integer inputs: bitwise
    equal to the oracle, nothing outside C's windows touched."""
    _, pg = env
    for i, (name, tA, tB, M, N, K, lda, ldb, ldc, batch) in enumerate(gemv_cases()):
        alpha, beta = ((1.0, 0.0), (-2.0, 0.5), (0.5, -1.0))[i % 3]
        w = Workload(name, tA, tB, M, N, K, alpha, beta, seed=500 + i, dist="int3",
                     lda=lda, ldb=ldb, ldc=ldc, batch=batch)
        A, B, C = workloads.make_inputs(w)
        log(f"[gemv] variant {variant} {name} batch={batch}")
        st, got = run_gpu(env, w, A, B, C, variant=variant)
        assert st == 0, (name, st)
        check_against_oracle(w, A, B, C, got, exact=True)
        check_untouched(w, C, got)


@pytest.mark.parametrize("tA,tB,M,N,K", [(0, 1, 16384, 1, 4096), (0, 1, 4096, 1, 4096),
                                         (0, 1, 1, 16384, 4096), (0, 1, 1024, 1, 65536),
                                         (1, 1, 16384, 1, 4096), (1, 1, 4096, 1, 4096),
                                         (0, 0, 1, 16384, 4096), (1, 1, 1024, 1, 65536),
                                         (0, 1, 16384, 3, 4096), (0, 0, 4096, 8, 4096),
                                         (0, 1, 512, 8, 65536), (0, 1, 4, 16384, 4096),
                                         (1, 1, 8, 4096, 4096)])
def test_gemv_float_at_size(env, tA, tB, M, N, K):
    """U(-1, 1) inputs at the sizes the kernels are for, checked against the
    oracle's bound on rows from both ends and the middle (for a few rows, all of
    them)."""
    _, pg = env
    w = Workload("gemv_f", tA, tB, M, N, K, 1.0, 0.5, seed=M + N + K + tA + tB)
    A, B, C = workloads.make_inputs(w)
    assert pg.sgemm_select_variant(tA, tB, M, N, K, 1, 1, 256) == pg.VARIANT_GEMV
    st, got = run_gpu(env, w, A, B, C)
    assert st == 0
    if M <= 192:
        check_against_oracle(w, A, B, C, got)
    else:
        for rows in ((0, 64), (M // 2, M // 2 + 64), (M - 64, M)):
            check_against_oracle(w, A, B, C, got, rows=rows)
    check_untouched(w, C, got)


def test_gemv_random_shapes(env):
    """80 seeded matrix-vector shapes through the automatic dispatch: one of M,
    N from 1 to 8 and the other up to 2000, K up to 2052, every transpose
    pair, padded leading dimensions, batches, integer inputs: bitwise equal to
    the oracle, nothing outside C's windows touched. Most reach a GEMV kernel
    (the one-vector, few-vector, mirror and output-contiguous paths); the
    rest check that the shapes the GEMV kernels leave alone still run."""
    _, pg = env
    rng = np.random.default_rng(2024)
    cus = 256
    reached = 0
    for i in range(80):
        small = int(rng.choice([1, 1, 2, 3, 4, 4, 5, 8]))
        big = int(rng.integers(1, 2000))
        K = int(rng.choice([4, 36, 516, 1028, 2052]))
        if rng.random() < 0.9:
            big = max(4, big // 4 * 4)
        rows_small = rng.random() < 0.5
        M, N = (small, big) if rows_small else (big, small)
        # mostly the layouts the GEMV kernels take, some others
        lean = int(rng.random() < 0.75)
        if rows_small:
            tA, tB = int(rng.integers(0, 2)), lean if rng.random() < 0.9 else 1 - lean
        else:
            tA, tB = 1 - lean if rng.random() < 0.9 else lean, int(rng.integers(0, 2))
        pad = lambda: int(rng.choice([0, 0, 4, 8]))
        batch = int(rng.choice([1, 1, 2, 3]))
        alpha, beta = (1.0, 0.0) if i % 3 == 0 else ((-2.0, 0.5) if i % 3 == 1 else (0.5, -1.0))
        w = Workload(f"grnd{i}", tA, tB, M, N, K, alpha, beta, seed=3000 + i, dist="int3",
                     batch=batch, lda=(M if tA else K) + pad(), ldb=(K if tB else N) + pad(),
                     ldc=N + pad())
        A, B, C = workloads.make_inputs(w)
        cA, cB, _, _ = canonical_vectors(tA, tB, M, N, K, w.LDA, w.LDB)
        v = pg.sgemm_select_variant(cA, cB, M, N, K, batch, 1 if vec4_possible(w) else 0, cus)
        reached += v == pg.VARIANT_GEMV
        log(f"[gemv-random] {w.name} {'NT'[tA]}{'NT'[tB]} {M}x{N}x{K} b{batch} "
            f"ld {w.LDA},{w.LDB},{w.LDC} -> {pg.VARIANT_NAMES[v]}")
        st, got = run_gpu(env, w, A, B, C)
        assert st == 0, (w, st)
        check_against_oracle(w, A, B, C, got, exact=True)
        check_untouched(w, C, got)
    assert reached >= 30, reached


def test_gemv_refuses_other_calls(env):
    """Forced on a call it does not cover, the GEMV variant returns -18, and
    it never splits K (-19)."""
    _, pg = env
    for tA, tB, M, N, K in ((0, 0, 64, 64, 64), (0, 1, 64, 9, 64), (1, 0, 2, 64, 64),
                            (0, 0, 64, 1, 64), (1, 1, 64, 2, 64), (0, 0, 4, 64, 64),
                            (0, 1, 9, 64, 64)):
        w = Workload("gemv_no", tA, tB, M, N, K, 1.0, 0.0, seed=1,
                     ldb=(K if tB else N) + (8 if (tA, tB, N) == (0, 0, 1) else 0))
        A, B, C = workloads.make_inputs(w)
        st, got = run_gpu(env, w, A, B, C, variant=pg.VARIANT_GEMV)
        assert st == -18, (tA, tB, M, N, K, st)
        assert np.array_equal(got.view(np.uint32), C.view(np.uint32))


# ------------------------------------------------------------------ pointer-array batched

def run_pointer_array(env, tA, tB, M, N, K, alpha, beta, lda, ldb, ldc, batch, seed, dist,
                      misalign=(), shared_a=(), variant=-1):
    """Items scattered through three device pools at irregular (16-byte
    aligned) offsets; items listed in `misalign` are shifted one float off
    16-byte alignment; items listed in `shared_a` reuse item 0's A. Returns
    the status and a list of (A, B, C_in, C_out) per item."""
    torch, pg = env
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(seed)
    items = []
    for b in range(batch):
        w = Workload("item", tA, tB, M, N, K, alpha, beta, seed=seed * 1000 + b, dist=dist,
                     lda=lda, ldb=ldb, ldc=ldc)
        items.append(workloads.make_inputs(w))
    shared = set(shared_a)

    def layout(sizes, skip=()):
        offs, pos = [], GUARD
        for b, n in enumerate(sizes):
            if b in skip:
                offs.append(offs[0])
                continue
            pos += 4 * int(rng.integers(0, 9))          # irregular gaps, 16-byte aligned
            offs.append(pos + (1 if b in misalign else 0))
            pos = offs[-1] + n
            pos = (pos + 3) // 4 * 4
        return offs, pos + GUARD

    offA, nA = layout([it[0].size for it in items], skip=shared)
    offB, nB = layout([it[1].size for it in items])
    offC, nC = layout([it[2].size for it in items])
    pools = []
    for offs, n, k in ((offA, nA, 0), (offB, nB, 1), (offC, nC, 2)):
        host = np.full(n, -7.25, np.float32)
        for b, o in enumerate(offs):
            if k == 0 and b in shared:
                continue
            host[o:o + items[b][k].size] = items[b][k]
        pools.append((host, torch.from_numpy(host).to(dev)))
    ptrs = [pg.pointer_array([p[1].data_ptr() + 4 * o for o in offs], dev)
            for p, offs in zip(pools, (offA, offB, offC))]
    st = pg.sgemm_batched_variant(tA, tB, M, N, K, alpha, ptrs[0], lda, ptrs[1], ldb, beta,
                                  ptrs[2], ldc, batch, variant, check=False)
    torch.cuda.synchronize(dev)
    outC = pools[2][1].cpu().numpy()
    # every float of the C pool outside the items' M x N windows keeps its bits
    mask = np.zeros(nC, bool)
    for o in offC:
        if M and N:
            mask[(o + np.arange(M)[:, None] * ldc + np.arange(N)[None, :]).reshape(-1)] = True
    assert np.array_equal(outC[~mask].view(np.uint32), pools[2][0][~mask].view(np.uint32)), \
        "the C pool changed outside the items' windows"
    res = []
    for b in range(batch):
        A = items[0][0] if b in shared else items[b][0]
        res.append((A, items[b][1], items[b][2], outC[offC[b]:offC[b] + items[b][2].size]))
    return st, res


def check_items(tA, tB, M, N, K, alpha, beta, lda, ldb, ldc, res, exact):
    w = Workload("item", tA, tB, M, N, K, alpha, beta, seed=0, lda=lda, ldb=ldb, ldc=ldc)
    for A, B, C, got in res:
        check_against_oracle(w, A, B, C, got, exact=exact)


@pytest.mark.parametrize("variant", [-1, *ALL_VARIANTS])
def test_pointer_array_bitwise(env, variant):
    """Pointer-array batches on every variant and transpose pair, integer
    inputs: bitwise equal to the oracle run item by item, with a shared A
    item and padded leading dimensions."""
    for (M, N, K), (tA, tB) in itertools.product([(68, 132, 40), (260, 36, 20), (12, 8, 100)],
                                                 itertools.product([0, 1], repeat=2)):
        lda, ldb, ldc = (M if tA else K) + 4, (K if tB else N) + 8, N + 4
        log(f"[ptr-array] variant {variant} {M}x{N}x{K} tA={tA} tB={tB}")
        st, res = run_pointer_array(env, tA, tB, M, N, K, 2.0, -1.0, lda, ldb, ldc, batch=5,
                                    seed=M + N + K + 2 * tA + tB, dist="int3", shared_a=(3,),
                                    variant=variant)
        assert st == 0, st
        check_items(tA, tB, M, N, K, 2.0, -1.0, lda, ldb, ldc, res, exact=True)


def test_pointer_array_gemv(env):
    """Pointer-array batches through the GEMV kernels (N == 1, M == 1 and a
    few vectors): items off 16-byte alignment take their plain paths; all
    exact."""
    for tA, tB, M, N, K, lda, ldb, ldc in ((0, 1, 300, 1, 132, 136, 132, 2),
                                           (0, 1, 1, 260, 68, 68, 72, 260),
                                           (1, 1, 300, 1, 132, 304, 132, 2),
                                           (0, 0, 1, 260, 68, 68, 264, 260),
                                           (0, 1, 300, 3, 132, 136, 140, 5),
                                           (0, 0, 300, 8, 132, 132, 12, 8)):
        st, res = run_pointer_array(env, tA, tB, M, N, K, 1.5, -0.5, lda, ldb, ldc, batch=5,
                                    seed=41 + M, dist="int3", misalign=(1, 3), shared_a=(4,),
                                    variant=pg_constants.VARIANT_GEMV)
        assert st == 0, st
        check_items(tA, tB, M, N, K, 1.5, -0.5, lda, ldb, ldc, res, exact=True)


@pytest.mark.parametrize("variant", [-1, 0, 2, 4, 5, 6, 7])
def test_pointer_array_misaligned_items(env, variant):
    """Items whose A or B is not 16-byte aligned, in a launch of a 4-float
    kernel: those items take the kernel's plain per-element path and must
    still be exact; their aligned neighbours take the MFMA path."""
    M, N, K = 72, 100, 48
    st, res = run_pointer_array(env, 0, 0, M, N, K, 1.0, 0.5, K, N, N, batch=6, seed=31,
                                dist="int3", misalign=(1, 4), variant=variant)
    assert st == 0
    check_items(0, 0, M, N, K, 1.0, 0.5, K, N, N, res, exact=True)
    st, res = run_pointer_array(env, 1, 1, M, N, K, -0.5, 0.0, M, K, N, batch=4, seed=32,
                                dist="normal", misalign=(0, 3), variant=variant)
    assert st == 0
    check_items(1, 1, M, N, K, -0.5, 0.0, M, K, N, res, exact=False)


def test_pointer_array_float_and_special_cases(env):
    """fp32 inputs within the bound; alpha = 0 and K = 0 scale each C item
    through the array without reading A or B (NULL arrays allowed)."""
    torch, pg = env
    st, res = run_pointer_array(env, 0, 1, 300, 200, 150, 0.75, -1.5, 152, 152, 204, batch=3,
                                seed=33, dist="normal")
    assert st == 0
    check_items(0, 1, 300, 200, 150, 0.75, -1.5, 152, 152, 204, res, exact=False)
    for alpha, K in ((0.0, 30), (1.0, 0)):
        dev = torch.device("cuda:0")
        C = [torch.randn(40, 24, device=dev) for _ in range(3)]
        before = [c.clone() for c in C]
        st = pg.sgemm_batched(0, 0, 40, 24, K, alpha, None, max(K, 1), None, 24, -2.0,
                              pg.pointer_array(C), 24, 3, check=False)
        torch.cuda.synchronize(dev)
        assert st == 0
        for c, c0 in zip(C, before):
            assert torch.equal(c, c0 * -2.0)


# ------------------------------------------------------------------ column-major

def colmajor_store(X, ld, cols):
    """Column-major storage of the 2-D array X (rows x cols) with leading
    dimension ld: element (r, c) at r + c*ld. The buffer ends at the last
    stored element."""
    rows = X.shape[0]
    buf = np.full((cols - 1) * ld + rows if rows and cols else 0, -7.25, np.float32)
    for c in range(cols):
        buf[c * ld:c * ld + rows] = X[:, c]
    return buf


@pytest.mark.parametrize("tA,tB", list(itertools.product([0, 1], repeat=2)))
def test_colmajor_against_definition(env, tA, tB):
    """The column-major entry points: operands stored by columns as the
    header's index formulas say, results compared with the oracle on the
    same logical matrices (row-major, untransposed). Integer inputs are
    bitwise, fp32 inputs within the bound; the strided form checks two
    items with gaps."""
    torch, pg = env
    dev = torch.device("cuda:0")
    for (M, N, K), dist in (((68, 132, 36), "int3"), ((257, 129, 65), "normal"),
                            ((4, 300, 8), "int3")):
        # integer cases keep every ld and stride a multiple of 4 (4-float
        # kernels); the fp32 case has odd ones (1-float kernels)
        aligned = dist == "int3"
        r4 = (lambda n: (n + 3) // 4 * 4 + 4) if aligned else (lambda n: n + 3)
        rng = np.random.default_rng(M * N + K + tA + 2 * tB)
        draw = (lambda *s: rng.integers(-3, 4, s).astype(np.float32)) if dist == "int3" else \
            (lambda *s: rng.standard_normal(s).astype(np.float32))
        batch = 2
        Aop = [draw(M, K) for _ in range(batch)]     # op(A) as a logical M x K matrix
        Bop = [draw(K, N) for _ in range(batch)]     # op(B) as a logical K x N matrix
        Cm = [draw(M, N) for _ in range(batch)]
        alpha, beta = (2.0, -1.0) if dist == "int3" else (0.75, 1.5)
        # stored matrices: transA = 0 keeps op(A) (M x K by columns), 1 stores its
        # transpose; likewise for B
        As = [a.T.copy() if tA else a for a in Aop]
        Bs = [b.T.copy() if tB else b for b in Bop]
        lda, ldb, ldc = r4(As[0].shape[0]), r4(Bs[0].shape[0]), r4(M)
        bufA = [colmajor_store(a, lda, a.shape[1]) for a in As]
        bufB = [colmajor_store(b, ldb, b.shape[1]) for b in Bs]
        bufC = [colmajor_store(c, ldc, N) for c in Cm]
        sA, sB, sC = (r4(len(x[0])) for x in (bufA, bufB, bufC))

        def pack(bufs, stride):
            out = np.full(stride * (batch - 1) + len(bufs[-1]), -7.25, np.float32)
            for b, x in enumerate(bufs):
                out[b * stride:b * stride + len(x)] = x
            return out
        hA, hB, hC = pack(bufA, sA), pack(bufB, sB), pack(bufC, sC)
        dA, dB = (torch.from_numpy(x).to(dev) for x in (hA, hB))
        for form in ("single", "strided"):
            dC = torch.from_numpy(hC).to(dev)
            log(f"[colmajor] {form} {M}x{N}x{K} tA={tA} tB={tB} {dist}")
            if form == "single":
                st = pg.sgemm_colmajor(tA, tB, M, N, K, alpha, dA, lda, dB, ldb, beta, dC, ldc,
                                       check=False)
                items = 1
            else:
                st = pg.sgemm_colmajor_strided_batched(tA, tB, M, N, K, alpha, dA, lda, dB,
                                                       ldb, beta, dC, ldc, batch, sA, sB, sC,
                                                       check=False)
                items = batch
            torch.cuda.synchronize(dev)
            assert st == 0
            out = dC.cpu().numpy()
            written = np.zeros(out.size, bool)
            for b in range(items):
                idx = b * sC + np.arange(M)[:, None] + np.arange(N)[None, :] * ldc
                written[idx.reshape(-1)] = True
                got = out[idx]
                ref, S = oracle.sgemm_rows(0, 0, M, N, K, alpha, Aop[b].reshape(-1), K,
                                           Bop[b].reshape(-1), N, beta, Cm[b].reshape(-1), N)
                ref, S = ref.reshape(M, N), S.reshape(M, N)
                if dist == "int3":
                    assert np.array_equal(got, ref.astype(np.float32)), (form, b)
                else:
                    rep = oracle.bound_check(got, ref, S, Cm[b], alpha, beta, K)
                    assert rep.ok, (form, b, rep)
            assert np.array_equal(out[~written].view(np.uint32), hC[~written].view(np.uint32))


# ------------------------------------------------------------------ split-K

def run_gpu_ws(env, w: Workload, A, B, C, variant=-1, splits=0, ws_floats=None):
    """As run_gpu, through sgemm_strided_batched_ws_variant with a workspace of
    ws_floats floats (None: what sgemm_workspace_size asks for, at least one
    float). The workspace carries guard bands too."""
    torch, pg = env
    dev = torch.device("cuda:0")
    if ws_floats is None:
        ws_floats = max(1, pg.sgemm_workspace_size(w.trans_a, w.trans_b, w.M, w.N, w.K,
                                                   w.batch) // 4)

    def put(x):
        buf = torch.full((x.size + 2 * GUARD,), -7.25, dtype=torch.float32, device=dev)
        buf[GUARD:GUARD + x.size] = torch.from_numpy(x).to(dev)
        return buf

    dA, dB, dC = put(A), put(B), put(C)
    ws = torch.full((ws_floats + 2 * GUARD,), 3.5, dtype=torch.float32, device=dev)
    st = pg.sgemm_strided_batched_ws_variant(
        w.trans_a, w.trans_b, w.M, w.N, w.K, w.alpha, dA.data_ptr() + 4 * GUARD, w.LDA,
        dB.data_ptr() + 4 * GUARD, w.LDB, w.beta, dC.data_ptr() + 4 * GUARD, w.LDC, w.batch,
        w.SA, w.SB, w.SC, variant, splits, (ws.data_ptr() + 4 * GUARD, 4 * ws_floats),
        stream=torch.cuda.current_stream(dev).cuda_stream, check=False)
    torch.cuda.synchronize(dev)
    whole, wsh = dC.cpu().numpy(), ws.cpu().numpy()
    assert np.all(whole[:GUARD] == np.float32(-7.25)) and \
        np.all(whole[GUARD + C.size:] == np.float32(-7.25)), "a guard band around C was overwritten"
    assert np.all(wsh[:GUARD] == np.float32(3.5)) and \
        np.all(wsh[GUARD + ws_floats:] == np.float32(3.5)), "a write past the workspace"
    return st, whole[GUARD:GUARD + C.size]


# every tile kernel (not the streaming ones, which split K across their own waves)
SPLIT_VARIANTS = [v for v in ALL_VARIANTS
                  if v not in (pg_constants.VARIANT_T64x64, pg_constants.VARIANT_T32x64,
                               pg_constants.VARIANT_T64x32)]


@pytest.mark.parametrize("variant", SPLIT_VARIANTS)
def test_splitk_bitwise(env, variant):
    """Forced split counts on every tile variant and transpose pair, ragged
    M/N, K not a multiple of the slice, batches with gaps, integer inputs:
    bitwise equal to the oracle, nothing written outside C's windows or the
    workspace."""
    _, pg = env
    n_run = 0
    for (M, N, K, batch), (tA, tB) in itertools.product(
            [(68, 132, 1000, 1), (36, 20, 2048, 3), (260, 64, 776, 2)],
            itertools.product([0, 1], repeat=2)):
        for splits in (2, 3, 7):
            alpha, beta = (2.0, -1.0) if splits != 3 else (0.5, 0.0)
            w = Workload(f"sk{M}x{N}x{K}", tA, tB, M, N, K, alpha, beta, seed=M + K + splits,
                         dist="int3", batch=batch, lda=(M if tA else K) + 4,
                         ldb=(K if tB else N) + 8, ldc=N + 4)
            w = Workload(**{**w.__dict__, "stride_a": w.SA + 8, "stride_b": w.SB + 4,
                            "stride_c": w.SC + 12})
            A, B, C = workloads.make_inputs(w)
            log(f"[split-K] variant {variant} {M}x{N}x{K} b{batch} tA={tA} tB={tB} S={splits}")
            st, got = run_gpu_ws(env, w, A, B, C, variant=variant, splits=splits,
                                 ws_floats=splits * M * N * batch)
            assert st == 0, (w, st)
            check_against_oracle(w, A, B, C, got, exact=True)
            check_untouched(w, C, got)
            n_run += 1
    assert n_run == 36


def test_splitk_automatic(env):
    """The automatic split: deep-K shapes with few tiles split (fp32 within
    the bound; the workspace size query is large enough); a workspace of a
    third of that still gives correct results with fewer slices; no
    workspace, or a grid that fills the GPU, gives the unsplit call's bits."""
    torch, pg = env
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for tA, tB, M, N, K, batch in ((0, 0, 256, 256, 16384, 1), (1, 1, 100, 72, 9000, 2),
                                   (0, 1, 64, 64, 4096, 1), (1, 0, 128, 200, 3000, 1)):
        w = Workload(f"auto{M}x{N}x{K}", tA, tB, M, N, K, 0.75, 1.5, seed=K, dist="normal",
                     batch=batch)
        A, B, C = workloads.make_inputs(w)
        need = pg.sgemm_workspace_size(tA, tB, M, N, K, batch)
        assert need >= 2 * 4 * M * N * batch, (w, need, cus)
        log(f"[split-K auto] {M}x{N}x{K} b{batch} tA={tA} tB={tB} workspace {need} B")
        for ws_floats in (need // 4, need // 12):
            st, got = run_gpu_ws(env, w, A, B, C, ws_floats=ws_floats)
            assert st == 0
            check_against_oracle(w, A, B, C, got)
            check_untouched(w, C, got)
        # no workspace: exactly the unsplit call
        st, got = run_gpu_ws(env, w, A, B, C, ws_floats=0)
        st2, ref = run_gpu(env, w, A, B, C)
        assert st == st2 == 0
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    # a full grid does not split: the same bits as the plain call
    w = Workload("full", 0, 0, 1024, 1024, 1024, 1.0, 0.5, seed=3)
    A, B, C = workloads.make_inputs(w)
    assert pg.sgemm_workspace_size(0, 0, 1024, 1024, 1024, 1) == 0
    st, got = run_gpu_ws(env, w, A, B, C, ws_floats=1 << 20)
    st2, ref = run_gpu(env, w, A, B, C)
    assert st == st2 == 0
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_splitk_deterministic(env):
    """Two launches of the same split call give the same bits, and the
    single-matrix entry point sgemm_ws matches the strided form."""
    torch, pg = env
    dev = torch.device("cuda:0")
    M, N, K = 192, 160, 12000
    g = torch.Generator(device=dev).manual_seed(5)
    A = torch.randn(M, K, device=dev, generator=g)
    B = torch.randn(K, N, device=dev, generator=g)
    ws = torch.empty(pg.sgemm_workspace_size(0, 0, M, N, K) // 4 + 1, device=dev)
    outs = []
    for form in ("ws", "ws", "strided"):
        C = torch.zeros(M, N, device=dev)
        if form == "ws":
            pg.sgemm_ws(0, 0, M, N, K, 1.0, A, K, B, N, 0.0, C, N, ws)
        else:
            pg.sgemm_strided_batched_ws(0, 0, M, N, K, 1.0, A, K, B, N, 0.0, C, N, 1, 0, 0, 0,
                                        ws)
        torch.cuda.synchronize(dev)
        outs.append(C.cpu().numpy())
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))
    assert np.array_equal(outs[0].view(np.uint32), outs[2].view(np.uint32))
    ref, S = oracle.sgemm_rows(0, 0, M, N, K, 1.0, A.cpu().numpy().reshape(-1), K,
                               B.cpu().numpy().reshape(-1), N, 0.0,
                               np.zeros(M * N, np.float32), N)
    rep = oracle.bound_check(outs[0], ref[0], S[0], np.zeros((M, N), np.float32), 1.0, 0.0, K)
    assert rep.ok, rep


def test_splitk_batch_beyond_one_launch(env):
    """33000 items x 2 slices are more workgroup rows than one launch takes
    (65535): the split launches are chunked in whole items and the reduction
    still sees every item."""
    M, N, K, batch = 8, 12, 600, 33000
    w = Workload("skbig", 0, 1, M, N, K, 1.0, 2.0, seed=77, dist="int3", batch=batch)
    A, B, C = workloads.make_inputs(w)
    log(f"[split-K chunked] {M}x{N}x{K} batch {batch}")
    st, got = run_gpu_ws(env, w, A, B, C, variant=2, splits=2, ws_floats=2 * M * N * batch)
    assert st == 0
    check_against_oracle(w, A, B, C, got, exact=True, batches=(0, 40))
    check_against_oracle(w, A, B, C, got, exact=True, batches=(32760, 32800))
    check_against_oracle(w, A, B, C, got, exact=True, batches=(batch - 40, batch))
