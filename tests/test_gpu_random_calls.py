"""Seeded random calls through the C ABI, compared with the oracle: bit for bit
on integer inputs, within its error bound on U(-1, 1) inputs.

Each call draws its shape from ragged and tile-sized dimensions (1 to 1000), a
transpose pair, padded leading dimensions, batch strides with gaps (some of
them breaking 16-byte alignment), an alpha/beta pair and an entry point:
- the plain call with the automatic choice or a forced tile variant;
- split-K with a caller workspace, the split automatic or forced;
- the entry point that allocates nothing.

Inputs are small integers and alpha/beta powers of two or zero, so every
result is exact in fp32 and must equal the oracle's. A call may be refused
only with the status its contract documents (a variant the layout does not
admit, a split the variant does not take, a split too large for the
workspace or the fixed array); every other status fails. The guard bands
around C and the elements of C outside its M x N windows must not change."""
import sys

import numpy as np
import pytest

import test_gpu_parity as T
import workloads
from workloads import Workload

pytestmark = pytest.mark.gpu

CALLS = 3000
ALPHA_BETA = [(1.0, 0.0), (2.0, 1.0), (-1.0, 0.5), (0.5, 2.0), (0.0, 1.0), (1.0, -1.0),
              (-2.0, 0.0)]
SIZES = T.SIZES + T.SIZES4 + [300, 384, 511, 513, 640, 768, 1000]


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


def run_split(env, w, A, B, C, variant, splits, ws, noalloc):
    """A split-K call (workspace form, or the form that allocates nothing) on
    guarded copies of the operands; returns (status, C after the call)."""
    torch, pg = env
    dev = torch.device("cuda:0")

    def put(x):
        buf = torch.full((x.size + 2 * T.GUARD,), -7.25, dtype=torch.float32, device=dev)
        buf[T.GUARD:T.GUARD + x.size] = torch.from_numpy(x).to(dev)
        return buf

    dA, dB, dC = put(A), put(B), put(C)
    pa, pb, pc = (t.data_ptr() + 4 * T.GUARD for t in (dA, dB, dC))
    stream = torch.cuda.current_stream(dev).cuda_stream
    args = (w.trans_a, w.trans_b, w.M, w.N, w.K, w.alpha, pa, w.LDA, pb, w.LDB, w.beta, pc,
            w.LDC, w.batch, w.SA, w.SB, w.SC)
    if noalloc:
        st = pg.sgemm_strided_batched_noalloc(*args, splits, stream=stream, check=False)
    else:
        st = pg.sgemm_strided_batched_ws_variant(*args, variant, splits, ws, stream=stream,
                                                 check=False)
    torch.cuda.synchronize(dev)
    whole = dC.cpu().numpy()
    assert np.all(whole[:T.GUARD] == np.float32(-7.25)), "guard band before C overwritten"
    assert np.all(whole[T.GUARD + C.size:] == np.float32(-7.25)), "guard band after C overwritten"
    return st, whole[T.GUARD:T.GUARD + C.size]


def test_random_calls_bitwise(env):
    torch, pg = env
    ws = torch.empty(64 << 20, dtype=torch.uint8, device=torch.device("cuda:0"))
    rng = np.random.default_rng(4321)
    variants = [-1] + list(T.ALL_VARIANTS)
    checked, refused = {}, {}
    for i in range(CALLS):
        while True:
            M, N, K = (int(rng.choice(SIZES)) for _ in range(3))
            batch = int(rng.choice([1, 1, 1, 2, 3, 5]))
            if M * N * K * batch <= 6e7:
                break
        tA, tB = int(rng.integers(2)), int(rng.integers(2))
        pad = int(rng.choice([0, 0, 0, 4, 1, 12]))
        alpha, beta = ALPHA_BETA[int(rng.integers(len(ALPHA_BETA)))]
        lda, ldb, ldc = (M if tA else K) + pad, (K if tB else N) + pad, N + pad
        gap = int(rng.choice([0, 0, 8, 3]))
        w = Workload(f"call{i}", tA, tB, M, N, K, alpha, beta, seed=i, dist="int3", batch=batch,
                     lda=lda, ldb=ldb, ldc=ldc, stride_a=(K if tA else M) * lda + gap,
                     stride_b=(N if tB else K) * ldb + gap, stride_c=M * ldc + gap)
        A, B, C = workloads.make_inputs(w)
        pick, variant = rng.random(), int(rng.choice(variants))
        if pick < 0.2:
            splits = int(rng.choice([0, 2, 3, 4, 7]))
            key, allowed = f"ws v{variant}", (0, -18, -19, -21)
            st, got = run_split(env, w, A, B, C, variant, splits, ws, noalloc=False)
        elif pick < 0.27:
            splits = int(rng.choice([0, 1, 2, 5]))
            key, allowed = "noalloc", (0, -19, -23)
            st, got = run_split(env, w, A, B, C, -1, splits, None, noalloc=True)
        else:
            key, allowed = f"plain v{variant}", (0, -18)
            st, got = T.run_gpu(env, w, A, B, C, variant=variant)
        assert st in allowed, (w, key, st, pg.sgemm_status_string(st))
        if (i + 1) % 500 == 0:
            log(f"  {i + 1} calls")
        if st != 0:
            refused[key] = refused.get(key, 0) + 1
            continue
        T.check_against_oracle(w, A, B, C, got, exact=True)
        T.check_untouched(w, C, got)
        checked[key] = checked.get(key, 0) + 1
    log(f"  {sum(checked.values())} checked bitwise, {sum(refused.values())} refused as "
        f"documented")
    # every entry point and every forced variant was exercised
    assert checked.get("noalloc", 0) >= 50
    for v in variants:
        assert checked.get(f"plain v{v}", 0) >= 30, v
    assert sum(n for k, n in checked.items() if k.startswith("ws ")) >= 200


def test_random_calls_float_bound(env):
    """The same entry points on U(-1, 1) inputs with deeper K (up to 4096, so
    that split-K takes many slices and the reduction changes the summation
    order): every element within the oracle's error bound."""
    torch, pg = env
    ws = torch.empty(64 << 20, dtype=torch.uint8, device=torch.device("cuda:0"))
    rng = np.random.default_rng(8765)
    variants = [-1] + list(T.ALL_VARIANTS)
    sizes = [1, 7, 33, 64, 100, 129, 256, 300, 513]
    ks = [1, 17, 64, 520, 1000, 2048, 4096]
    n_checked = 0
    for i in range(300):
        while True:
            M, N = (int(rng.choice(sizes)) for _ in range(2))
            K, batch = int(rng.choice(ks)), int(rng.choice([1, 1, 2, 3]))
            if M * N * K * batch <= 1.2e8:
                break
        tA, tB = int(rng.integers(2)), int(rng.integers(2))
        pad = int(rng.choice([0, 4, 1]))
        alpha, beta = float(rng.uniform(-2, 2)), float(rng.choice([0.0, 1.0, -0.75]))
        lda, ldb, ldc = (M if tA else K) + pad, (K if tB else N) + pad, N + pad
        w = Workload(f"fcall{i}", tA, tB, M, N, K, alpha, beta, seed=50000 + i, batch=batch,
                     lda=lda, ldb=ldb, ldc=ldc)
        A, B, C = workloads.make_inputs(w)
        pick, variant = rng.random(), int(rng.choice(variants))
        if pick < 0.3:
            splits = int(rng.choice([0, 2, 5, 16]))
            allowed = (0, -18, -19, -21)
            st, got = run_split(env, w, A, B, C, variant, splits, ws, noalloc=False)
        elif pick < 0.4:
            allowed = (0, -19, -23)
            st, got = run_split(env, w, A, B, C, -1, int(rng.choice([0, 3])), None, noalloc=True)
        else:
            allowed = (0, -18)
            st, got = T.run_gpu(env, w, A, B, C, variant=variant)
        assert st in allowed, (w, st, pg.sgemm_status_string(st))
        if (i + 1) % 50 == 0:
            log(f"  {i + 1} calls")
        if st != 0:
            continue
        T.check_against_oracle(w, A, B, C, got)
        T.check_untouched(w, C, got)
        n_checked += 1
    log(f"  {n_checked} calls within the bound")
    assert n_checked >= 100
