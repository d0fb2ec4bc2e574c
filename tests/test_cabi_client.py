"""The C ABI from a plain C program (tests/cabi/sgemm_client.c).

The client links libsgemm.so and the HIP runtime only: it allocates device
memory with hipMalloc, calls one entry point on a stream it creates and
writes C back. Its results are checked against the CPU oracle (the acceptance
bound of the header) and against the same call made through the Python
binding, which must give the same bits: the library is deterministic and the
dispatch depends only on the arguments and the device.

The argument-rejection check needs no GPU: the library validates arguments
before its first HIP call.
"""
import os
import struct
import subprocess
import sys

import numpy as np
import pytest

import oracle
import workloads
from conftest import ROOT
from workloads import Workload

CLIENT = os.path.join(ROOT, "tests", "cabi", "sgemm_client")

ENTRY_SGEMM, ENTRY_STRIDED, ENTRY_WS, ENTRY_POINTERS, ENTRY_COLMAJOR = range(5)


@pytest.fixture(scope="module")
def client():
    if not os.path.exists(CLIENT):
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "sgemm_cabi_build", os.path.join(ROOT, "tests", "cabi", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
    return CLIENT


def log(msg):
    sys.stdout.write(msg + "\n")
    sys.stdout.flush()


def test_c_client_sees_argument_errors(client):
    """Statuses reach a C caller as the header documents them (no GPU work)."""
    out = subprocess.run([client, "--errors"], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stdout + out.stderr
    assert "status -3" in out.stdout and "status -14" in out.stdout


def write_case(path, w: Workload, entry, A, B, C):
    head = [w.trans_a, w.trans_b, w.M, w.N, w.K, w.LDA, w.LDB, w.LDC, w.batch,
            w.SA, w.SB, w.SC, entry]
    with open(path, "wb") as f:
        f.write(struct.pack("=13q", *head))
        f.write(struct.pack("=2d", w.alpha, w.beta))
        f.write(struct.pack("=3q", A.size, B.size, C.size))
        for x in (A, B, C):
            f.write(np.ascontiguousarray(x, np.float32).tobytes())


def run_client(client, tmp_path, w, entry, A, B, C):
    case, out = tmp_path / "case.bin", tmp_path / "out.bin"
    write_case(case, w, entry, A, B, C)
    res = subprocess.run([client, str(case), str(out)], capture_output=True, text=True,
                         timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    raw = out.read_bytes()
    status = struct.unpack("=q", raw[:8])[0]
    return status, np.frombuffer(raw[8:], np.float32).copy()


def run_binding(w, entry, A, B, C):
    import torch
    import precision_gemm_amd as pg
    dev = torch.device("cuda:0")
    dA, dB, dC = (torch.from_numpy(x.copy()).to(dev) for x in (A, B, C))
    args = (w.trans_a, w.trans_b, w.M, w.N, w.K, w.alpha)
    if entry == ENTRY_SGEMM:
        st = pg.sgemm(*args, dA, w.LDA, dB, w.LDB, w.beta, dC, w.LDC, check=False)
    elif entry == ENTRY_STRIDED:
        st = pg.sgemm_strided_batched(*args, dA, w.LDA, dB, w.LDB, w.beta, dC, w.LDC, w.batch,
                                      w.SA, w.SB, w.SC, check=False)
    elif entry == ENTRY_WS:
        nbytes = pg.sgemm_workspace_size(w.trans_a, w.trans_b, w.M, w.N, w.K, w.batch)
        ws = torch.empty(max(1, nbytes // 4), dtype=torch.float32, device=dev)
        st = pg.sgemm_strided_batched_ws(*args, dA, w.LDA, dB, w.LDB, w.beta, dC, w.LDC,
                                         w.batch, w.SA, w.SB, w.SC, (ws.data_ptr(), nbytes),
                                         check=False)
    elif entry == ENTRY_POINTERS:
        base = lambda t, s: [t.data_ptr() + 4 * b * s for b in range(w.batch)]
        arr = lambda p: torch.tensor(p, dtype=torch.int64, device=dev)
        st = pg.sgemm_batched(*args, arr(base(dA, w.SA)), w.LDA, arr(base(dB, w.SB)), w.LDB,
                              w.beta, arr(base(dC, w.SC)), w.LDC, w.batch, check=False)
    else:
        st = pg.sgemm_colmajor(*args, dA, w.LDA, dB, w.LDB, w.beta, dC, w.LDC, check=False)
    torch.cuda.synchronize(dev)
    return st, dC.cpu().numpy()


def rowmajor_twin(w: Workload) -> Workload:
    """The row-major product of the transposes, C^T = op(B)^T op(A)^T, whose
    buffers are those of the column-major call w (its A is w's B)."""
    return Workload(w.name, w.trans_b, w.trans_a, w.N, w.M, w.K, w.alpha, w.beta, w.seed,
                    lda=w.LDB, ldb=w.LDA, ldc=w.LDC)


def check_oracle(w, entry, A, B, C, got):
    """Bound check of every item, the column-major call through its row-major
    twin."""
    if entry == ENTRY_COLMAJOR:
        rw, Ar, Br = rowmajor_twin(w), B, A
    else:
        rw, Ar, Br = w, A, B
    ref, S = oracle.sgemm_rows(rw.trans_a, rw.trans_b, rw.M, rw.N, rw.K, rw.alpha, Ar, rw.LDA,
                               Br, rw.LDB, rw.beta, C, rw.LDC, batch=rw.batch,
                               stride_a=rw.SA, stride_b=rw.SB, stride_c=rw.SC)
    for b in range(rw.batch):
        idx = b * rw.SC + np.arange(rw.M)[:, None] * rw.LDC + np.arange(rw.N)[None, :]
        rep = oracle.bound_check(got[idx], ref[b], S[b], C[idx], rw.alpha, rw.beta, rw.K)
        assert rep.ok, (b, str(rep))
    # nothing outside the output windows moved
    mask = np.zeros(C.size, bool)
    for b in range(rw.batch):
        mask[(b * rw.SC + np.arange(rw.M)[:, None] * rw.LDC + np.arange(rw.N)[None, :])
             .reshape(-1)] = True
    assert np.array_equal(got[~mask].view(np.uint32), C[~mask].view(np.uint32))


CASES = [
    # (entry, workload)
    (ENTRY_SGEMM, Workload("c_sgemm", 1, 0, 300, 200, 136, 1.25, 0.5, seed=31)),
    (ENTRY_SGEMM, Workload("c_sgemm_odd", 0, 1, 97, 61, 45, -0.75, 0.0, seed=32,
                           lda=47, ldb=46, ldc=63)),
    (ENTRY_STRIDED, Workload("c_strided_shared_b", 0, 1, 130, 68, 200, 1.0, -1.0, seed=33,
                             batch=3, stride_b=0)),
    (ENTRY_WS, Workload("c_splitk", 0, 0, 64, 96, 8192, 1.0, 0.25, seed=34, batch=2)),
    (ENTRY_POINTERS, Workload("c_pointers", 1, 1, 100, 72, 52, 1.5, -0.5, seed=35, batch=2)),
    (ENTRY_COLMAJOR, Workload("c_colmajor", 1, 0, 68, 132, 36, 0.5, 2.0, seed=36,
                              lda=68, ldb=132, ldc=72)),
    # matrix-vector products: the GEMV kernels, row-major N == 1 and a
    # column-major N == 1 call (its row-major twin has M == 1)
    (ENTRY_SGEMM, Workload("c_gemv", 0, 1, 300, 1, 136, -1.5, 0.5, seed=37, lda=140, ldc=2)),
    (ENTRY_STRIDED, Workload("c_gemv_t", 1, 1, 260, 1, 68, 1.0, 0.0, seed=38, batch=3)),
    (ENTRY_COLMAJOR, Workload("c_colmajor_gemv", 0, 0, 260, 1, 68, 1.0, 0.5, seed=39,
                              lda=264, ldb=68, ldc=260)),
]


@pytest.mark.gpu
@pytest.mark.parametrize("entry,w", CASES, ids=[c[1].name for c in CASES])
def test_c_client_matches_oracle_and_binding(client, tmp_path, entry, w):
    if entry == ENTRY_COLMAJOR:
        twin_a, twin_b, C = workloads.make_inputs(rowmajor_twin(w))
        A, B = twin_b, twin_a
    else:
        A, B, C = workloads.make_inputs(w)
    log(f"[cabi] {w.name} entry={entry} {w.M}x{w.N}x{w.K} batch={w.batch}")
    st, got = run_client(client, tmp_path, w, entry, A, B, C)
    assert st == 0, st
    check_oracle(w, entry, A, B, C, got)
    st2, got2 = run_binding(w, entry, A, B, C)
    assert st2 == 0, st2
    assert np.array_equal(got.view(np.uint32), got2.view(np.uint32)), \
        "the C caller and the Python binding got different bits"
