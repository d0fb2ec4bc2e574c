"""The C-ABI library loads, exports every symbol the header declares, and its
host-side logic (argument checks, quick returns, variant choice) behaves as
documented. Nothing here launches a kernel, so it runs without a GPU."""
import os
import re
import subprocess

import pytest

from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "sgemm.h")


@pytest.fixture(scope="module")
def pg():
    import precision_gemm_amd as pg
    if not os.path.exists(pg.library_path()):
        from precision_gemm_amd import _build
        _build.build()
    pg._load()
    return pg


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(sgemm\w*)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("sgemm", "sgemm_strided_batched", "sgemm_status_string",
              "sgemm_select_variant", "sgemm_strided_batched_variant"):
        assert n in names


def test_binding_mirrors_the_variant_enum(pg):
    """The binding's variant constants match the header's enum."""
    text = open(HEADER).read()
    enum = dict((n, int(v)) for n, v in re.findall(r"SGEMM_VARIANT_(\w+)\s*=\s*(-?\d+)", text))
    assert enum["COUNT"] == pg.VARIANT_COUNT == len(pg.VARIANT_NAMES)
    for name, value in enum.items():
        if name != "COUNT":
            assert getattr(pg, "VARIANT_" + name) == value, name
            if value >= 0:
                assert pg.VARIANT_NAMES[value] == name


def test_library_exports_every_declared_symbol(pg):
    out = subprocess.run(["nm", "-D", "--defined-only", pg.library_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(pg._load(), name)


def test_header_compiles_as_c():
    src = '#include "sgemm.h"\nint main(void){return (int)sizeof(&sgemm);}\n'
    subprocess.run(["gcc", "-x", "c", "-std=c99", "-Wall", "-Werror", "-I",
                    os.path.join(ROOT, "include"), "-fsyntax-only", "-"],
                   input=src, text=True, check=True)


WINDOW_CAP = (1 << 31) - 1


def expected_ranges(left, step, n):
    """Window i starts i * step bytes further in: the bytes left from there to
    the operand's end, within [0, 2^31 - 1]."""
    return [min(max(left - i * step, 0), WINDOW_CAP) for i in range(n)]


@pytest.mark.parametrize("step", [64, 4096, 64 * 4092, 64 * ((1 << 21) - 1), 512 * 4096])
def test_window_ranges_match_the_bytes_left(pg, step):
    """The buffer-range countdown the kernels keep per operand window, for
    operands from a few bytes to 300 GiB past the window start, including every
    crossing of the 2^31 cap, against the exact bytes left."""
    GiB = 1 << 30
    lefts = [0, 4, 1000, WINDOW_CAP - 1, WINDOW_CAP, WINDOW_CAP + 1, 2 * GiB + 3 * step + 4,
             3 * GiB - 7, 8 * GiB, 128 * GiB - 64, 128 * GiB + 64, 200 * GiB, 300 * GiB]
    for left in lefts:
        # enough windows to cross the cap and walk past the end where that is
        # within reach, else a few thousand capped ones
        cross = max(0, (left - WINDOW_CAP) // step + 1)
        n = int(min(cross + 4 + (WINDOW_CAP // step + 2 if cross < 4000 else 0), 6000))
        assert pg.sgemm_window_ranges(left, step, n) == expected_ranges(left, step, n), left


def test_window_ranges_rejects_bad_arguments(pg):
    with pytest.raises(pg.SgemmError):
        pg.sgemm_window_ranges(100, 0, 3)
    with pytest.raises(pg.SgemmError):
        pg.sgemm_window_ranges(100, 64, -1)


FAKE = 1 << 20  # never dereferenced: every call below returns before any device work


def base_args(**over):
    a = dict(transA=0, transB=0, M=4, N=4, K=4, alpha=1.0, A=FAKE, lda=4, B=FAKE, ldb=4,
             beta=0.0, C=FAKE, ldc=4, batch=1, strideA=0, strideB=0, strideC=0)
    a.update(over)
    return a


def call(pg, **over):
    a = base_args(**over)
    return pg.sgemm_strided_batched(a["transA"], a["transB"], a["M"], a["N"], a["K"],
                                    a["alpha"], a["A"], a["lda"], a["B"], a["ldb"],
                                    a["beta"], a["C"], a["ldc"], a["batch"], a["strideA"],
                                    a["strideB"], a["strideC"], check=False)


@pytest.mark.parametrize("over,status", [
    (dict(transA=2), -1), (dict(transB=-1), -2), (dict(M=-1), -3), (dict(N=-1), -4),
    (dict(K=-1), -5), (dict(A=None), -7), (dict(lda=3), -8), (dict(B=None), -9),
    (dict(ldb=3), -10), (dict(C=None), -12), (dict(ldc=3), -13), (dict(batch=-1), -14),
    (dict(strideA=-4), -15), (dict(strideB=-4), -16), (dict(strideC=-4), -17),
    # stored row length depends on the transpose flags
    (dict(transA=1, M=8, lda=4), -8), (dict(transB=1, K=8, ldb=4, lda=8), -10),
])
def test_argument_errors(pg, over, status):
    assert call(pg, **over) == status
    assert pg.sgemm_status_string(status).startswith(f"invalid argument {-status}")


@pytest.mark.parametrize("over", [
    dict(M=0), dict(N=0), dict(batch=0),
    dict(K=0, beta=1.0), dict(alpha=0.0, beta=1.0),
    # NULL operands are fine where they are never read
    dict(M=0, A=None, B=None, C=None), dict(K=0, beta=1.0, A=None, B=None),
    dict(alpha=0.0, beta=1.0, A=None, B=None, C=None),
])
def test_quick_returns_launch_nothing(pg, over):
    assert call(pg, **over) == 0


def test_variant_argument_checked(pg):
    a = base_args()
    st = pg.sgemm_strided_batched_variant(0, 0, 4, 4, 4, 1.0, FAKE, 4, FAKE, 4, 0.0, FAKE, 4,
                                          1, 0, 0, 0, pg.VARIANT_COUNT, check=False)
    assert st == -18
    st = pg.sgemm_strided_batched_variant(0, 0, 4, 4, 4, 1.0, FAKE + 4, 4, FAKE, 4, 0.0, FAKE,
                                          4, 1, 0, 0, 0, pg.VARIANT_S64x64, check=False)
    assert st == -18  # 4-float variant forced on an unaligned A
    assert a  # keep the helper in use


def test_any_leading_dimension_is_accepted(pg):
    """Every ld at or above the stored row length is valid; a variant with
    32-bit in-tile offsets cannot be forced for one of 2^21 or more (the
    64-bit-addressed W64x64 builds run those calls). Nothing here launches."""
    top = (1 << 31) - 1
    assert call(pg, M=0, lda=top, ldb=top, ldc=top) == 0
    assert call(pg, K=0, beta=1.0, lda=top) == 0
    for which in ("lda", "ldb", "ldc"):
        ld = dict(lda=4, ldb=4, ldc=4)
        ld[which] = 1 << 21
        for v in (pg.VARIANT_M128x128, pg.VARIANT_S64x64, pg.VARIANT_S64x64_V1,
                  pg.VARIANT_T64x64, pg.VARIANT_T32x64, pg.VARIANT_S64x64_K2):
            st = pg.sgemm_strided_batched_variant(0, 0, 4, 4, 4, 1.0, FAKE, ld["lda"], FAKE,
                                                  ld["ldb"], 0.0, FAKE, ld["ldc"], 1, 0, 0, 0,
                                                  v, check=False)
            assert st == -18, (which, v)
    assert "2^21" in pg.sgemm_status_string(-18)


def test_status_strings(pg):
    assert pg.sgemm_status_string(0) == "success"
    assert pg.sgemm_status_string(-99) == "invalid argument"
    assert len(pg.sgemm_status_string(1)) > 0  # a hipError_t message


def test_select_variant(pg):
    sel = pg.sgemm_select_variant
    # whole waves of 128 x 128 tiles: 4092^3 (1024 tiles, four per CU), 2048^3,
    # 6144^3, 8192^3 and the batched 64 x 512^2 workload
    for shape, batch, tA in (((4092, 4092, 4092), 1, 0), ((2048, 2048, 2048), 1, 0),
                             ((6144, 6144, 6144), 1, 0), ((8192, 8192, 8192), 1, 0),
                             ((512, 512, 520), 64, 1)):
        assert sel(tA, 0, *shape, batch, True, 256) == pg.VARIANT_M128x128, shape
    # few 64 x 64 tiles per CU over K >= 768: the K-split eight-wave tile
    for shape in ((1024, 1024, 1024), (3072, 3072, 3072), (1536, 1536, 1536),
                  (1024, 1024, 4096), (1000, 1000, 1000)):
        assert sel(0, 0, *shape, 1, True, 256) == pg.VARIANT_S64x64_K2, shape
    # at most one tile per CU: the eight-wave streaming kernel, skinny or not,
    # on its 64 x 32 tile over K >= 512 (512 x 512: 128 tiles; 1024 x 512:
    # 256), on the 32 x 64 one below
    for shape in ((512, 512, 512), (512, 512, 8192), (1024, 512, 1024), (128, 128, 2048),
                  (8192, 64, 4096), (64, 8192, 4096), (4096, 128, 4096), (64, 8192, 8192)):
        assert sel(0, 0, *shape, 1, True, 256) == pg.VARIANT_T64x32, shape
    for shape in ((512, 512, 256), (96, 96, 384), (128, 128, 128), (256, 256, 16)):
        assert sel(0, 0, *shape, 1, True, 256) == pg.VARIANT_T32x64, shape
    # a matrix-vector product whose vector is contiguous in k (N == 1 with B
    # transposed, M == 1 with A not): the GEMV kernels, the matrix either way
    for shape in ((16384, 1, 4096), (1, 16384, 4096), (1, 1, 4), (7, 1, 100000), (1, 3, 8)):
        assert sel(0, 1, *shape, 1, True, 256) == pg.VARIANT_GEMV, shape
        assert sel(0, 1, *shape, 1, False, 256) == pg.VARIANT_S64x64_V1, shape
    assert sel(1, 1, 16384, 1, 4096, 1, True, 256) == pg.VARIANT_GEMV
    assert sel(0, 0, 1, 16384, 4096, 1, True, 256) == pg.VARIANT_GEMV
    for tA, tB in ((0, 0), (1, 0)):
        assert sel(tA, tB, 16384, 1, 4096, 1, True, 256) != pg.VARIANT_GEMV
    for tA, tB in ((1, 0), (1, 1)):
        assert sel(tA, tB, 1, 16384, 4096, 1, True, 256) != pg.VARIANT_GEMV
    # a few vectors (2 <= N <= 8) against a matrix contiguous in k, K >= 512:
    # up to four contiguous ones on any grid, otherwise only where the 64 x 32
    # tiles would not fill the CUs (4096 rows: 64 tiles)
    for tB in (0, 1):
        for n in (2, 3, 5, 8):
            assert sel(0, tB, 4096, n, 4096, 1, True, 256) == pg.VARIANT_GEMV, (tB, n)
            want = tB == 1 and n <= 4
            assert (sel(0, tB, 16384, n, 4096, 1, True, 256) == pg.VARIANT_GEMV) == want
        assert sel(0, tB, 4096, 8, 256, 1, True, 256) != pg.VARIANT_GEMV
    assert sel(1, 1, 16384, 2, 4096, 1, True, 256) != pg.VARIANT_GEMV
    assert sel(0, 1, 16384, 9, 4096, 1, True, 256) != pg.VARIANT_GEMV
    # the mirror: a few rows against B stored N x K
    for tA in (0, 1):
        for m in (2, 3, 5, 8):
            assert sel(tA, 1, m, 4096, 4096, 1, True, 256) == pg.VARIANT_GEMV, (tA, m)
            want = tA == 0 and m <= 4
            assert (sel(tA, 1, m, 16384, 4096, 1, True, 256) == pg.VARIANT_GEMV) == want
    assert sel(0, 0, 4, 4096, 4096, 1, True, 256) != pg.VARIANT_GEMV
    assert sel(0, 1, 4, 4096, 256, 1, True, 256) != pg.VARIANT_GEMV
    # N <= 32 < M: the 64 x 32 tile for small grids or any grid over K >= 512;
    # M <= 32 with K >= 512: the 32 x 64 tile on any grid
    for shape in ((16384, 1, 4096), (65536, 32, 4096), (4096, 8, 256), (100, 32, 64)):
        assert sel(0, 0, *shape, 1, True, 256) == pg.VARIANT_T64x32, shape
    # a last round of tiles that the 64 x 32 tile fills better (cost model)
    for shape in ((1152, 1152, 4096), (1536, 1536, 4096), (1536, 1536, 8192)):
        assert sel(0, 0, *shape, 1, True, 256) == pg.VARIANT_T64x32, shape
    assert sel(0, 0, 1536, 1536, 1536, 1, True, 256) == pg.VARIANT_S64x64_K2
    for shape in ((2, 16384, 4096), (32, 65536, 4096), (16, 16, 4096), (32, 32, 32)):
        assert sel(0, 0, *shape, 1, True, 256) == pg.VARIANT_T32x64, shape
    assert sel(0, 0, 32768, 16, 256, 1, True, 256) != pg.VARIANT_T64x32    # 512 tiles, short K
    assert sel(0, 0, 1024, 512, 1024, 1, True, 128) != pg.VARIANT_T32x64   # two per CU
    assert sel(0, 0, 512, 512, 128, 3, True, 256) != pg.VARIANT_T32x64     # 384 tiles
    assert sel(0, 0, 512, 512, 2048, 8, True, 256) == pg.VARIANT_S64x64_K2
    # ... and the plain 64 x 64 tile below K = 768; for K <= 128 it also beats
    # the 128 x 128 tile on full grids (per-tile fixed costs dominate), while
    # for 128 < K <= 512 the 128 x 128 tile takes an equal share of work per
    # CU and the plain tile only the grids it fills better
    assert sel(0, 0, 1024, 1024, 512, 1, True, 256) == pg.VARIANT_S64x64
    assert sel(0, 0, 128, 128, 128, 1, True, 2) == pg.VARIANT_S64x64
    for shape in ((8192, 8192, 128), (2048, 2048, 64)):
        assert sel(0, 0, *shape, 1, True, 256) == pg.VARIANT_S64x64, shape
    for shape, batch in (((2048, 2048, 512), 1), ((4096, 4096, 256), 1), ((256, 256, 256), 128),
                         ((4096, 4096, 520), 1)):
        assert sel(0, 0, *shape, batch, True, 256) == pg.VARIANT_M128x128, shape
    # beyond one 32 x 64 tile per CU, a skinny dimension with a long operand
    # over 128 MiB, contiguous in k, against a short operand contiguous along
    # its outputs, with one 64 x 64 tile per CU at most, streams through the
    # 64 x 64 kernel; the other layouts, two tiles per CU and a long operand
    # of at most 128 MiB go to the K-split tile
    assert sel(0, 0, 16384, 64, 4096, 1, True, 256) == pg.VARIANT_T64x64
    assert sel(1, 1, 64, 16384, 8192, 1, True, 256) == pg.VARIANT_T64x64
    for tA, tB in ((0, 1), (1, 1), (1, 0)):
        assert sel(tA, tB, 16384, 64, 4096, 1, True, 256) == pg.VARIANT_S64x64_K2
    for tA, tB in ((0, 1), (0, 0), (1, 0)):
        assert sel(tA, tB, 64, 16384, 4096, 1, True, 256) == pg.VARIANT_S64x64_K2
    assert sel(0, 0, 32768, 64, 4096, 1, True, 256) == pg.VARIANT_S64x64_K2
    assert sel(0, 0, 16384, 64, 4096, 1, True, 128) == pg.VARIANT_S64x64_K2
    assert sel(0, 1, 16384, 64, 2048, 1, True, 256) == pg.VARIANT_S64x64_K2
    assert sel(0, 1, 64, 16384, 2048, 1, True, 256) == pg.VARIANT_S64x64_K2
    assert sel(0, 1, 16384, 64, 128, 1, True, 256) != pg.VARIANT_T64x64
    # the CU count enters the model: on 64 CUs 2048^3 has four 128 x 128 tiles per CU
    assert sel(0, 0, 2048, 2048, 2048, 1, True, 64) == pg.VARIANT_M128x128
    # a tile whose grid would exceed one launch is passed over: 2^24 tiles of
    # 64 x 64 (2^32 work-items), while 2^22 tiles of 128 x 128 still fit
    assert sel(0, 0, 1 << 29, 128, 128, 1, True, 256) == pg.VARIANT_M128x128
    assert sel(0, 0, 1 << 20, 128, 128, 1, True, 256) == pg.VARIANT_S64x64
    # no 4-float loads: the 1-float variant
    assert sel(0, 0, 4092, 4092, 4092, 1, False, 256) == pg.VARIANT_S64x64_V1
    assert sel(3, 0, 4, 4, 4, 1, True, 256) == -1


# ------------------------------------------------------------------ split-K (host side)

def test_select_splits(pg):
    sel = pg.sgemm_select_splits
    K2, S64, M128, T = (pg.VARIANT_S64x64_K2, pg.VARIANT_S64x64, pg.VARIANT_M128x128,
                        pg.VARIANT_T64x64)
    # 16 tiles of 64 x 64 on 256 CUs: 16 slices of 1024, one workgroup per CU
    assert sel(0, 0, 256, 256, 16384, 1, K2, 256) == 16
    assert sel(0, 0, 256, 256, 16384, 1, K2, 64) == 4
    # a full grid does not split
    assert sel(0, 0, 1024, 1024, 1024, 1, K2, 256) == 1
    assert sel(0, 0, 1024, 1024, 4096, 1, K2, 256) == 1
    assert sel(0, 0, 1024, 1024, 8192, 1, M128, 256) == 4       # 64 tiles of 128 x 128
    # 144 tiles: two slices would leave some CUs two workgroups of half the
    # work (no gain); seven put at most four short ones on a CU
    assert sel(0, 0, 768, 768, 16384, 1, K2, 256) == 7
    # at most 128 slices
    assert sel(0, 1, 64, 64, 1 << 18, 1, K2, 256) == 128
    # slices are at least 256 deep
    assert sel(0, 0, 128, 128, 128, 1, S64, 256) == 1
    assert sel(0, 0, 128, 128, 4096, 1, S64, 256) == 16
    # the slice length is rounded up to the K-step, so the count can drop:
    # 1000 / 3 -> 336 (BK 16) -> 3 slices; 1000 / 3 -> 352 (BK 32) -> 3 slices
    assert sel(0, 0, 64, 64, 1000, 1, S64, 256) == 3
    assert sel(0, 0, 64, 64, 1000, 1, K2, 256) == 3
    assert sel(0, 0, 64, 64, 600, 1, K2, 256) == 2
    # batch items count as tiles
    assert sel(0, 0, 64, 64, 8192, 64, K2, 256) == 4
    # the streaming kernel splits K across its own waves
    assert sel(0, 1, 64, 64, 1 << 20, 1, T, 256) == 1
    assert sel(0, 0, 64, 64, 4096, 1, pg.VARIANT_COUNT, 256) == -18
    assert sel(0, 0, -1, 64, 4096, 1, K2, 256) == -3


def ws_call(pg, variant=-1, splits=0, ws=None, **over):
    a = base_args(**over)
    return pg.sgemm_strided_batched_ws_variant(
        a["transA"], a["transB"], a["M"], a["N"], a["K"], a["alpha"], a["A"], a["lda"],
        a["B"], a["ldb"], a["beta"], a["C"], a["ldc"], a["batch"], a["strideA"], a["strideB"],
        a["strideC"], variant, splits, ws, check=False)


def test_split_arguments_checked(pg):
    # the ordinary argument checks come first
    assert ws_call(pg, M=-1) == -3
    assert ws_call(pg, splits=-1) == -19
    assert ws_call(pg, splits=1 << 16) == -19
    assert ws_call(pg, ws=(0, 64)) == -20                 # NULL with a size
    assert ws_call(pg, ws=(FAKE + 2, 64)) == -20          # not 4-byte aligned
    assert ws_call(pg, variant=pg.VARIANT_COUNT) == -18
    # a forced split needs its whole workspace: 4 slices of 64 x 64 = 64 KiB
    # (checked before any device work, as the variant is forced too)
    kw = dict(M=64, N=64, K=4096, lda=4096, ldb=64, ldc=64)
    assert ws_call(pg, variant=pg.VARIANT_S64x64, splits=4, ws=(FAKE, 4 * 64 * 64 * 4 - 4),
                   **kw) == -21
    assert ws_call(pg, variant=pg.VARIANT_T64x64, splits=4, ws=(FAKE, 1 << 20), **kw) == -19
    assert ws_call(pg, variant=pg.VARIANT_T32x64, splits=4, ws=(FAKE, 1 << 20), **kw) == -19
    assert ws_call(pg, variant=pg.VARIANT_T64x32, splits=4, ws=(FAKE, 1 << 20), **kw) == -19
    # the GEMV kernel: -18 off its calls, -19 for a forced split on them
    assert ws_call(pg, variant=pg.VARIANT_GEMV, splits=4, ws=(FAKE, 1 << 20), **kw) == -18
    kv = dict(M=64, N=1, K=4096, lda=4096, transB=1, ldb=4096, ldc=1)
    assert ws_call(pg, variant=pg.VARIANT_GEMV, splits=4, ws=(FAKE, 1 << 20), **kv) == -19
    for st in (-19, -20, -21):
        assert "invalid" in pg.sgemm_status_string(st) or "too small" in \
            pg.sgemm_status_string(st)


def test_oversize_grid_is_rejected(pg):
    """More output tiles in one item than one launch's tile axis holds (in
    work-items, a signed 32-bit range) is an error before any device work.
    Only rejected calls are made here: the pointers are fake."""
    # 2^22 tiles of 64 x 64 for the 512-thread K-split tile: 2^31 work-items
    assert ws_call(pg, variant=pg.VARIANT_S64x64_K2, splits=1, M=1 << 28, N=64, K=4, lda=4,
                   ldb=64, ldc=64) == -22
    # 2^23 + 1 tiles for the 256-thread streaming tile
    assert ws_call(pg, variant=pg.VARIANT_T64x64, splits=1, M=((1 << 23) + 1) * 64, N=64, K=4,
                   lda=4, ldb=64, ldc=64) == -22
    assert "too large" in pg.sgemm_status_string(-22)


def test_workspace_size_without_a_device(pg):
    # no device to query here: the size is 0 (and invalid shapes are always 0)
    assert pg.sgemm_workspace_size(0, 0, 256, 256, 16384, 1) >= 0
    assert pg.sgemm_workspace_size(0, 0, -1, 256, 16384, 1) == 0


# ------------------------------------------------------------------ properties of the host decisions

from hypothesis import given, settings, strategies as st  # noqa: E402

_dim = st.integers(min_value=1, max_value=1 << 16)


@settings(max_examples=300, deadline=None)
@given(tA=st.integers(0, 1), tB=st.integers(0, 1), M=_dim, N=_dim, K=_dim,
       batch=st.integers(1, 512), vec4=st.booleans(), cus=st.integers(1, 512))
def test_select_variant_is_always_a_kernel(pg, tA, tB, M, N, K, batch, vec4, cus):
    """Any valid shape gets a variant in range; without 4-float loads it is the
    1-float variant; with them, the GEMV kernels exactly for N == 1 with B
    transposed or M == 1 with A not (the vector contiguous in k); the 64 x 64 streaming kernel only for
    a dimension of at most 64, one 64 x 64 tile per CU at most and the long
    operand contiguous in k against a short one that is not; the 64 x 32 one for M > 32 with at most one tile per CU and
    K >= 512, or N <= 32 with one tile per CU or K >= 512; otherwise the
    32 x 64 one exactly for grids of at most one tile per CU or M <= 32 with
    K >= 512."""
    v = pg.sgemm_select_variant(tA, tB, M, N, K, batch, vec4, cus)
    assert 0 <= v < pg.VARIANT_COUNT
    if not vec4:
        assert v == pg.VARIANT_S64x64_V1
    if v == pg.VARIANT_T64x64:
        assert min(M, N) <= 64 and K >= 512 and -(-M // 64) * -(-N // 64) * batch <= cus
        assert (tA, tB) == ((0, 0) if M > N else (1, 1))
    few6432 = -(-M // 64) * -(-N // 32) * batch <= cus
    t6432 = M > 32 and (few6432 or K >= 512 if N <= 32 else few6432 and K >= 512)
    t3264 = -(-M // 32) * -(-N // 64) * batch <= cus or (M <= 32 and K >= 512)
    gemv = (N == 1 and tB == 1) or (M == 1 and tA == 0) or \
        (2 <= N <= 8 and tA == 0 and K >= 512 and
         ((tB == 1 and N <= 4) or -(-M // 64) * batch < cus)) or \
        (2 <= M <= 8 and tB == 1 and K >= 512 and
         ((tA == 0 and M <= 4) or -(-N // 64) * batch < cus))
    if vec4 and gemv:
        assert v == pg.VARIANT_GEMV
    elif vec4 and t6432:
        assert v == pg.VARIANT_T64x32
    elif vec4 and t3264:
        assert v == pg.VARIANT_T32x64
    else:
        # beyond those rules the 64 x 32 tile only from the cost model, K >= 2048
        assert v != pg.VARIANT_T32x64 and (v != pg.VARIANT_T64x32 or K >= 2048)
    assert v not in (pg.VARIANT_L256x128, pg.VARIANT_L256x256, pg.VARIANT_M128x128_DMA)


@settings(max_examples=300, deadline=None)
@given(M=_dim, N=_dim, K=st.integers(1, 1 << 22), batch=st.integers(1, 64),
       variant=st.sampled_from([0, 1, 2, 3, 5, 6, 7]), cus=st.integers(1, 512))
def test_select_splits_covers_k_exactly(pg, M, N, K, batch, variant, cus):
    """The split count S is in [1, 128]; the slices of round_up(ceil(K/S), BK)
    k cover K with no empty slice; a split only happens with slices at least
    256 deep."""
    S = pg.sgemm_select_splits(0, 0, M, N, K, batch, variant, cus)
    assert 1 <= S <= 128
    if S == 1:
        return
    bk = 32 if variant == pg.VARIANT_S64x64_K2 else 16
    # the slice length the library uses for this S (the count it returns is
    # already that of the non-empty slices)
    ks = None
    for s0 in range(S, 129):
        cand = -(-(-(-K // s0)) // bk) * bk
        if -(-K // cand) == S:
            ks = cand
            break
    assert ks is not None
    assert ks % bk == 0 and (S - 1) * ks < K <= S * ks
    assert K // S >= 128   # slices are never thin (at least ~256 deep before rounding)
