"""Pins for the CPU oracle against facts that do not come from the oracle itself.

Every test here runs on the CPU. Together they are chosen so that a plausible
slip in the oracle (a dropped alpha or beta term, a wrong sign, a transposed
operand, a wrong leading dimension or batch stride, a wrong k range) fails at
least one of them; ``test_pins_reject_mutants`` demonstrates this on mutated
copies of the definition.
"""
from fractions import Fraction
import itertools

import numpy as np
import pytest

import oracle
import workloads
from conftest import read_golden


def stored(op: np.ndarray, trans: int, ld: int | None = None) -> tuple[np.ndarray, int]:
    """Row-major storage of a logical operand op (rows x cols), transposed if asked,
    with row stride ld (padding filled with a loud sentinel)."""
    mat = op.T if trans else op
    rows, cols = mat.shape
    ld = cols if ld is None else ld
    buf = np.full(max(1, rows * ld), 1e30, np.float32)
    for r in range(rows):
        buf[r * ld:r * ld + cols] = mat[r]
    return buf, max(1, ld)


def call(opA, opB, C, alpha, beta, tA=0, tB=0, lda=None, ldb=None, ldc=None, **kw):
    M, K = opA.shape
    N = opB.shape[1]
    A, lda = stored(np.asarray(opA, np.float32), tA, lda)
    B, ldb = stored(np.asarray(opB, np.float32), tB, ldb)
    Cb, ldc = stored(np.asarray(C, np.float32), 0, ldc)
    ref, S = oracle.sgemm_rows(tA, tB, M, N, K, alpha, A, lda, B, ldb, beta, Cb, ldc, **kw)
    return ref[0], S[0]


# ---------------------------------------------------------------- hand cases

def test_hand_2x2_golden():
    g = read_golden("hand_2x2.txt")
    A = np.array(g["A"], np.float32).reshape(2, 2)
    B = np.array(g["B"], np.float32).reshape(2, 2)
    C = np.array(g["C"], np.float32).reshape(2, 2)
    ref, _ = call(A, B, C, g["alpha"], g["beta"])
    assert ref.reshape(-1).tolist() == g["expected"]


@pytest.mark.parametrize("tA,tB", list(itertools.product([0, 1], repeat=2)))
def test_hand_2x3x2_all_transposes(tA, tB):
    g = read_golden("hand_2x3x2.txt")
    M, N, K = (int(x) for x in g["M N K"])
    # Build the stored buffers straight from the fixture (not via transpose code).
    A = np.array(g["A_T"] if tA else g["A"], np.float32)
    B = np.array(g["B_T"] if tB else g["B"], np.float32)
    lda = M if tA else K
    ldb = K if tB else N
    C = np.full(M * N, np.nan, np.float32)  # beta = 0: C must not be read
    ref, _ = oracle.sgemm_rows(tA, tB, M, N, K, g["alpha"], A, lda, B, ldb, g["beta"], C, N)
    assert ref.reshape(-1).tolist() == g["expected"]


def test_symbolic_expansion_tiny():
    """Brute force on every shape with M, N, K <= 3: the product written out with
    exact rational arithmetic on dyadic inputs (every fp64 step is exact)."""
    rng = np.random.default_rng(11)
    for M, N, K in itertools.product(range(1, 4), repeat=3):
        for tA, tB in itertools.product([0, 1], repeat=2):
            opA = rng.integers(-16, 17, (M, K)) / 8.0
            opB = rng.integers(-16, 17, (K, N)) / 8.0
            C = rng.integers(-16, 17, (M, N)) / 8.0
            alpha, beta = 1.5, -0.25
            ref, S = call(opA, opB, C, alpha, beta, tA, tB)
            for i in range(M):
                for j in range(N):
                    dot = sum(Fraction(opA[i, k]) * Fraction(opB[k, j]) for k in range(K))
                    exact = Fraction(alpha) * dot + Fraction(beta) * Fraction(C[i, j])
                    sabs = sum(abs(Fraction(opA[i, k]) * Fraction(opB[k, j])) for k in range(K))
                    assert Fraction(ref[i, j]) == exact, (M, N, K, tA, tB, i, j)
                    assert Fraction(S[i, j]) == sabs


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("tA,tB", list(itertools.product([0, 1], repeat=2)))
def test_identity_left(tA, tB):
    rng = np.random.default_rng(1)
    M, N = 7, 5
    B = rng.uniform(-1, 1, (M, N)).astype(np.float32)
    C = rng.uniform(-1, 1, (M, N)).astype(np.float32)
    ref, _ = call(np.eye(M), B, C, 2.0, -0.5, tA, tB)
    np.testing.assert_array_equal(ref, 2.0 * B.astype(np.float64) - 0.5 * C.astype(np.float64))


@pytest.mark.parametrize("tA,tB", list(itertools.product([0, 1], repeat=2)))
def test_permutation(tA, tB):
    rng = np.random.default_rng(2)
    M, N = 6, 9
    perm = rng.permutation(M)
    P = np.eye(M)[perm]                      # (P @ B)[i] = B[perm[i]]
    B = rng.uniform(-1, 1, (M, N)).astype(np.float32)
    ref, _ = call(P, B, np.zeros((M, N)), 1.0, 0.0, tA, tB)
    np.testing.assert_array_equal(ref, B[perm].astype(np.float64))
    # right multiplication by a permutation permutes columns
    A = rng.uniform(-1, 1, (N, M)).astype(np.float32)
    ref2, _ = call(A, P, np.zeros((N, M)), 1.0, 0.0, tA, tB)
    inv = np.argsort(perm)                   # (A @ P)[:, j] = A[:, inv[j]]
    np.testing.assert_array_equal(ref2, A[:, inv].astype(np.float64))


def test_alpha_zero_scales_c_only():
    rng = np.random.default_rng(3)
    A = np.full((4, 3), np.nan)              # alpha = 0: A and B are not read
    B = np.full((3, 5), np.inf)
    C = rng.uniform(-1, 1, (4, 5)).astype(np.float32)
    ref, S = call(A, B, C, 0.0, 3.0)
    np.testing.assert_array_equal(ref, 3.0 * C.astype(np.float64))
    ref0, _ = call(A, B, C, 0.0, 0.0)
    np.testing.assert_array_equal(ref0, np.zeros((4, 5)))


def test_beta_zero_does_not_read_c():
    A = np.array([[1.0, 2.0]])
    B = np.array([[3.0], [4.0]])
    ref, _ = call(A, B, np.array([[np.nan]]), 1.0, 0.0)
    assert ref[0, 0] == 11.0


def test_k_zero_is_beta_c():
    C = np.array([[1.5, -2.0]], np.float32)
    A = np.zeros((1, 0))
    B = np.zeros((0, 2))
    ref, S = call(A, B, C, 5.0, 2.0)
    np.testing.assert_array_equal(ref, [[3.0, -4.0]])
    np.testing.assert_array_equal(S, [[0.0, 0.0]])


def test_k_one_outer_product():
    x = np.array([1.0, -2.0, 0.5], np.float32)
    y = np.array([3.0, 0.25, -1.0, 4.0], np.float32)
    C = np.ones((3, 4), np.float32)
    for tA, tB in itertools.product([0, 1], repeat=2):
        ref, _ = call(x[:, None], y[None, :], C, -1.0, 2.0, tA, tB)
        np.testing.assert_array_equal(ref, -np.outer(x, y).astype(np.float64) + 2.0)


def test_rank1_closed_form():
    """A[i,k] = x_i and B[k,j] = y_j give (AB)[i,j] = K * x_i * y_j exactly."""
    M, N, K = 5, 6, 37
    x = np.array([1, -2, 0.5, 4, -0.25], np.float32)
    y = np.array([2, 1, -1, 0.125, 8, -3], np.float32)
    for tA, tB in itertools.product([0, 1], repeat=2):
        ref, S = call(np.repeat(x[:, None], K, 1), np.repeat(y[None, :], K, 0),
                      np.zeros((M, N)), 1.0, 0.0, tA, tB)
        np.testing.assert_array_equal(ref, K * np.outer(x, y).astype(np.float64))
        np.testing.assert_array_equal(S, K * np.abs(np.outer(x, y)).astype(np.float64))


# ---------------------------------------------------------------- library special case

@pytest.mark.parametrize("tA,tB", list(itertools.product([0, 1], repeat=2)))
def test_matches_numpy_float64_matmul(tA, tB):
    rng = np.random.default_rng(4)
    M, N, K = 37, 29, 53
    opA = rng.uniform(-1, 1, (M, K)).astype(np.float32)
    opB = rng.standard_normal((K, N)).astype(np.float32)
    C = rng.uniform(-1, 1, (M, N)).astype(np.float32)
    ref, S = call(opA, opB, C, 0.75, -1.25, tA, tB, lda=(M if tA else K) + 3,
                  ldb=(K if tB else N) + 5, ldc=N + 2)
    A64, B64, C64 = (m.astype(np.float64) for m in (opA, opB, C))
    want = 0.75 * (A64 @ B64) - 1.25 * C64
    np.testing.assert_allclose(ref, want, rtol=0, atol=1e-12 * (np.abs(A64) @ np.abs(B64)).max())
    np.testing.assert_allclose(S, np.abs(A64) @ np.abs(B64), rtol=1e-13)


# ---------------------------------------------------------------- consistency

def _rand_problem(rng, tA, tB, M, N, K, batch, pad=0):
    lda = (M if tA else K) + pad
    ldb = (K if tB else N) + pad
    ldc = N + pad
    ra, ca = (K, M) if tA else (M, K)
    rb, cb = (N, K) if tB else (K, N)
    sa = (ra - 1) * lda + ca + 7
    sb = (rb - 1) * ldb + cb + 3
    sc = (M - 1) * ldc + N + 5
    A = rng.uniform(-1, 1, sa * batch).astype(np.float32)
    B = rng.uniform(-1, 1, sb * batch).astype(np.float32)
    C = rng.uniform(-1, 1, sc * batch).astype(np.float32)
    return A, B, C, lda, ldb, ldc, sa, sb, sc


def test_batched_equals_loop_of_single_calls():
    rng = np.random.default_rng(5)
    M, N, K, batch = 9, 11, 13, 3
    for tA, tB in itertools.product([0, 1], repeat=2):
        A, B, C, lda, ldb, ldc, sa, sb, sc = _rand_problem(rng, tA, tB, M, N, K, batch, pad=2)
        ref, S = oracle.sgemm_rows(tA, tB, M, N, K, 1.5, A, lda, B, ldb, 0.5, C, ldc,
                                   batch=batch, stride_a=sa, stride_b=sb, stride_c=sc)
        for b in range(batch):
            r1, s1 = oracle.sgemm_rows(tA, tB, M, N, K, 1.5, A[b * sa:], lda, B[b * sb:], ldb,
                                       0.5, C[b * sc:], ldc)
            np.testing.assert_array_equal(ref[b], r1[0])
            np.testing.assert_array_equal(S[b], s1[0])
            # and against numpy on the extracted operands
            opA = _extract(A[b * sa:], tA, M, K, lda)
            opB = _extract(B[b * sb:], tB, K, N, ldb)
            Cm = _extract(C[b * sc:], 0, M, N, ldc)
            np.testing.assert_allclose(ref[b], 1.5 * opA @ opB + 0.5 * Cm, atol=1e-12)


def _extract(buf, trans, rows, cols, ld):
    """Logical rows x cols operand read from a row-major buffer via numpy strides."""
    srows, scols = (cols, rows) if trans else (rows, cols)
    m = np.lib.stride_tricks.as_strided(buf, (srows, scols), (ld * 4, 4)).astype(np.float64)
    return m.T if trans else m


def test_broadcast_stride_zero():
    rng = np.random.default_rng(6)
    M, N, K, batch = 4, 5, 6, 3
    A = rng.uniform(-1, 1, M * K).astype(np.float32)           # shared by every item
    B = rng.uniform(-1, 1, K * N * batch).astype(np.float32)
    C = np.zeros(M * N * batch, np.float32)
    ref, _ = oracle.sgemm_rows(0, 0, M, N, K, 1.0, A, K, B, N, 0.0, C, N,
                               batch=batch, stride_a=0, stride_b=K * N, stride_c=M * N)
    for b in range(batch):
        want = A.reshape(M, K).astype(np.float64) @ B[b * K * N:(b + 1) * K * N].reshape(K, N)
        np.testing.assert_allclose(ref[b], want, atol=1e-12)


def test_padded_ld_equals_minimal_and_transpose_copy():
    rng = np.random.default_rng(7)
    M, N, K = 10, 7, 12
    opA = rng.uniform(-1, 1, (M, K)).astype(np.float32)
    opB = rng.uniform(-1, 1, (K, N)).astype(np.float32)
    C = rng.uniform(-1, 1, (M, N)).astype(np.float32)
    base, baseS = call(opA, opB, C, 1.25, 0.5)
    for tA, tB in itertools.product([0, 1], repeat=2):
        for pad in (0, 3):
            r, s = call(opA, opB, C, 1.25, 0.5, tA, tB, lda=(M if tA else K) + pad,
                        ldb=(K if tB else N) + pad, ldc=N + pad)
            np.testing.assert_array_equal(r, base)
            np.testing.assert_array_equal(s, baseS)


def test_rows_subset_threads_and_elements_agree():
    rng = np.random.default_rng(8)
    M, N, K, batch = 23, 17, 31, 2
    for tA, tB in itertools.product([0, 1], repeat=2):
        A, B, C, lda, ldb, ldc, sa, sb, sc = _rand_problem(rng, tA, tB, M, N, K, batch, pad=1)
        args = (tA, tB, M, N, K, -0.5, A, lda, B, ldb, 2.0, C, ldc)
        kw = dict(batch=batch, stride_a=sa, stride_b=sb, stride_c=sc)
        full, fullS = oracle.sgemm_rows(*args, **kw, threads=1)
        multi, multiS = oracle.sgemm_rows(*args, **kw, threads=5)
        np.testing.assert_array_equal(full, multi)
        part, _ = oracle.sgemm_rows(*args, **kw, rows=(5, 19), batches=(1, 2))
        np.testing.assert_array_equal(part[0], full[1, 5:19])
        bs = rng.integers(0, batch, 40)
        is_ = rng.integers(0, M, 40)
        js = rng.integers(0, N, 40)
        e, eS = oracle.sgemm_elements(tA, tB, K, -0.5, A, lda, B, ldb, 2.0, C, ldc,
                                      bs, is_, js, stride_a=sa, stride_b=sb, stride_c=sc)
        np.testing.assert_array_equal(e, full[bs, is_, js])
        np.testing.assert_array_equal(eS, fullS[bs, is_, js])


def test_integer_inputs_are_exact():
    """Small-integer operands: every partial sum is an integer below 2**24, so
    the double result equals numpy's integer matmul exactly."""
    rng = np.random.default_rng(9)
    M, N, K = 33, 65, 130
    opA = rng.integers(-3, 4, (M, K))
    opB = rng.integers(-3, 4, (K, N))
    C = rng.integers(-3, 4, (M, N))
    ref, _ = call(opA, opB, C, 2.0, -1.0, 1, 0)
    np.testing.assert_array_equal(ref, 2 * (opA @ opB) - C)


# ---------------------------------------------------------------- acceptance bound

def test_bound_check_accepts_rounding_and_rejects_errors():
    rng = np.random.default_rng(10)
    M, N, K = 16, 16, 64
    opA = rng.uniform(-1, 1, (M, K)).astype(np.float32)
    opB = rng.uniform(-1, 1, (K, N)).astype(np.float32)
    C = rng.uniform(-1, 1, (M, N)).astype(np.float32)
    ref, S = call(opA, opB, C, 1.0, 0.5)
    # a sequential float32 evaluation is within the bound
    f32 = np.zeros((M, N), np.float32)
    for k in range(K):
        f32 = f32 + np.outer(opA[:, k], opB[k, :]).astype(np.float32)
    f32 = f32 + np.float32(0.5) * C
    assert oracle.bound_check(f32, ref, S, C, 1.0, 0.5, K).ok
    # a single dropped product term is not
    bad = f32.copy()
    bad[3, 4] -= opA[3, 7] * opB[7, 4]
    rep = oracle.bound_check(bad, ref, S, C, 1.0, 0.5, K)
    assert not rep.ok and rep.n_bad == 1
    nan = f32.copy()
    nan[0, 0] = np.nan
    assert not oracle.bound_check(nan, ref, S, C, 1.0, 0.5, K).ok


# The acceptance bound at its edge. Each case states the limit worked out by
# hand from the bound 2e-6 * max(K,1) * (|alpha| S + |beta| |c|) and places the
# GPU value just inside it (must pass) and just outside it (must fail). A bound
# that lost its factor K, squared it, dropped max(K, 1), took alpha or beta
# with its sign, or dropped the |beta||c| term fails at least one of them.
EDGE = 0.05  # relative distance from the limit on either side


def _edge_case(ref, S, c_in, alpha, beta, K, limit):
    inside = np.array([ref + limit * (1 - EDGE), ref - limit * (1 - EDGE)])
    outside = np.array([ref + limit * (1 + EDGE), ref - limit * (1 + EDGE)])
    r, s, c = (np.full(2, v, np.float64) for v in (ref, S, c_in))
    ok = oracle.bound_check(inside, r, s, c, alpha, beta, K)
    bad = oracle.bound_check(outside, r, s, c, alpha, beta, K)
    assert ok.ok, ok
    assert not bad.ok and bad.n_bad == 2, bad


def test_bound_edge_negative_alpha_with_beta():
    # op(A) = [1, -2, 0.5], op(B) = [2, 1, -4]^T: the product is 2 - 2 - 2 = -2,
    # S = 2 + 2 + 2 = 6; alpha = -2, beta = 0.5, c = 4 give 4 + 2 = 6 and the
    # limit 2e-6 * 3 * (2 * 6 + 0.5 * 4) = 8.4e-5.
    ref, S = call(np.array([[1, -2, 0.5]]), np.array([[2], [1], [-4]]), np.array([[4.0]]),
                  -2.0, 0.5)
    assert (ref[0, 0], S[0, 0]) == (6.0, 6.0)
    _edge_case(6.0, 6.0, 4.0, -2.0, 0.5, 3, 8.4e-5)


def test_bound_edge_k_zero_uses_max_k_1():
    # K = 0: C = beta * c = 2 * 3 = 6, S = 0, limit 2e-6 * 1 * (2 * 3) = 1.2e-5
    # (a bound scaled by K itself would be 0 and reject even the inside case).
    _edge_case(6.0, 0.0, 3.0, 1.0, 2.0, 0, 1.2e-5)


def test_bound_edge_beta_term_dominates():
    # alpha = 1, S = 1e-3, beta = -4, c = 100, K = 2:
    # limit 2e-6 * 2 * (1e-3 + 400) = 1.600004e-3, the |beta||c| term nearly all of it.
    _edge_case(-399.5, 1e-3, 100.0, 1.0, -4.0, 2, 1.600004e-3)


def test_bound_edge_scales_with_k():
    # The same element at K = 1 and K = 1000: S = 2, alpha = 1, beta = 0
    # (c is not part of the bound): limits 4e-6 and 4e-3.
    _edge_case(1.0, 2.0, 7.0, 1.0, 0.0, 1, 4e-6)
    _edge_case(1.0, 2.0, 7.0, 1.0, 0.0, 1000, 4e-3)


# ---------------------------------------------------------------- pins vs mutants

def _mutants():
    def good(A, B, C, a, b):
        return a * A @ B + b * C
    return {
        "drop_beta": lambda A, B, C, a, b: a * A @ B,
        "drop_alpha": lambda A, B, C, a, b: A @ B + b * C,
        "sign": lambda A, B, C, a, b: a * A @ B - b * C,
        "transpose_a": lambda A, B, C, a, b: a * A.T @ B + b * C if A.shape[0] == A.shape[1] else None,
        "transpose_b": lambda A, B, C, a, b: a * A @ B.T + b * C if B.shape[0] == B.shape[1] else None,
        "swap_operands": lambda A, B, C, a, b: a * B @ A + b * C if A.shape == B.shape else None,
        "drop_last_k": lambda A, B, C, a, b: a * A[:, :-1] @ B[:-1, :] + b * C,
    }, good


def test_pins_reject_mutants():
    g = read_golden("hand_2x2.txt")
    A = np.array(g["A"]).reshape(2, 2)
    B = np.array(g["B"]).reshape(2, 2)
    C = np.array(g["C"]).reshape(2, 2)
    mutants, good = _mutants()
    assert good(A, B, C, g["alpha"], g["beta"]).reshape(-1).tolist() == g["expected"]
    for name, f in mutants.items():
        out = f(A, B, C, g["alpha"], g["beta"])
        assert out is None or out.reshape(-1).tolist() != g["expected"], name


# ---------------------------------------------------------------- workloads

def test_workload_shapes_and_counts():
    w = workloads.BY_NAME["bmm_64x512x512x520_tn"]
    assert (w.LDA, w.LDB, w.LDC) == (512, 512, 512)
    assert (w.SA, w.SB, w.SC) == (266240, 266240, 262144)
    s = workloads.BY_NAME["skinny_16384x64x4096_nt"]
    assert (s.LDA, s.LDB, s.LDC) == (4096, 4096, 64)
    h = workloads.HEADLINE
    assert h.flops() == 137_036_693_376
    assert h.algorithmic_bytes() == 267_911_424
    A, B, C = workloads.make_inputs(workloads.BY_NAME["sgemm_128"])
    assert A.dtype == np.float32 and A.size == 128 * 128
    assert A.min() >= -1 and A.max() <= 1
    A2, _, _ = workloads.make_inputs(workloads.BY_NAME["sgemm_128"])
    np.testing.assert_array_equal(A, A2)
