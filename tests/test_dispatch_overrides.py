"""Per-shape dispatch overrides (sgemm_set_dispatch_overrides): host-side
checks through the C ABI, no GPU needed. The automatic choice takes an
installed record for exactly its shape, where the call's alignment allows the
record's variant; other shapes keep the cost model's choice; invalid tables
are refused whole; replacement is safe against concurrent lookups."""
import json
import threading

import pytest

import precision_gemm_amd as pg


@pytest.fixture
def lib():
    pg._load()
    pg.sgemm_set_dispatch_overrides([])
    yield pg
    pg.sgemm_set_dispatch_overrides([])  # the table is process-wide


def sel(lib, tA, tB, M, N, K, batch=1, vec4=True, cus=256):
    return lib.sgemm_select_variant(tA, tB, M, N, K, batch, vec4, cus)


def test_no_table_by_default(lib):
    assert lib.sgemm_dispatch_override_count() == 0
    assert sel(lib, 0, 0, 1024, 1024, 1024) == lib.VARIANT_S64x64_K2


def test_record_replaces_the_model_for_its_shape_only(lib):
    model = {s: sel(lib, *s) for s in [(0, 0, 1024, 1024, 1024), (1, 0, 1024, 1024, 1024),
                                        (0, 0, 1024, 1024, 1023), (0, 0, 2048, 2048, 2048)]}
    assert lib.sgemm_set_dispatch_overrides([(0, 0, 1024, 1024, 1024, 1, "M128x128"),
                                             (0, 0, 2048, 2048, 2048, 1, lib.VARIANT_T64x32)]) == 0
    assert lib.sgemm_dispatch_override_count() == 2
    assert sel(lib, 0, 0, 1024, 1024, 1024) == lib.VARIANT_M128x128
    assert sel(lib, 0, 0, 2048, 2048, 2048) == lib.VARIANT_T64x32
    # another transpose, another K or another batch is another shape
    assert sel(lib, 1, 0, 1024, 1024, 1024) == model[(1, 0, 1024, 1024, 1024)]
    assert sel(lib, 0, 0, 1024, 1024, 1023) == model[(0, 0, 1024, 1024, 1023)]
    assert sel(lib, 0, 0, 1024, 1024, 1024, batch=2) != lib.VARIANT_M128x128
    # the CU count does not enter an override
    assert sel(lib, 0, 0, 1024, 1024, 1024, cus=64) == lib.VARIANT_M128x128


def test_load_width_decides_whether_a_record_applies(lib):
    lib.sgemm_set_dispatch_overrides([(0, 0, 512, 512, 512, 1, "M128x128"),
                                      (0, 0, 640, 640, 640, 1, "W64x64_V1")])
    # a 4-float variant cannot serve a call without 16-byte loads: the model's
    # 1-float variant runs instead; a 1-float record applies either way
    assert sel(lib, 0, 0, 512, 512, 512, vec4=False) == lib.VARIANT_S64x64_V1
    assert sel(lib, 0, 0, 512, 512, 512, vec4=True) == lib.VARIANT_M128x128
    assert sel(lib, 0, 0, 640, 640, 640, vec4=False) == lib.VARIANT_W64x64_V1
    assert sel(lib, 0, 0, 640, 640, 640, vec4=True) == lib.VARIANT_W64x64_V1


def test_later_record_wins_and_replacement_is_whole(lib):
    lib.sgemm_set_dispatch_overrides([(0, 1, 300, 300, 300, 1, "S64x64"),
                                      (0, 1, 300, 300, 300, 1, "L256x128")])
    assert lib.sgemm_dispatch_override_count() == 1
    assert sel(lib, 0, 1, 300, 300, 300) == lib.VARIANT_L256x128
    lib.sgemm_set_dispatch_overrides([(1, 1, 77, 77, 77, 3, "T32x64")])
    assert lib.sgemm_dispatch_override_count() == 1
    assert sel(lib, 0, 1, 300, 300, 300) != lib.VARIANT_L256x128
    assert sel(lib, 1, 1, 77, 77, 77, batch=3) == lib.VARIANT_T32x64
    assert lib.sgemm_set_dispatch_overrides([]) == 0
    assert lib.sgemm_dispatch_override_count() == 0


@pytest.mark.parametrize("bad", [
    (2, 0, 8, 8, 8, 1, 1),            # transpose flag
    (0, -1, 8, 8, 8, 1, 1),
    (0, 0, -8, 8, 8, 1, 1),           # negative sizes
    (0, 0, 8, 8, -1, 1, 1),
    (0, 0, 8, 8, 8, -1, 1),
    (0, 0, 8, 8, 8, 1, -1),           # no variant
    (0, 0, 8, 8, 8, 1, 15),
    (0, 0, 8, 1, 8, 1, 10),           # GEMV: only some shapes
    (0, 0, 8, 8, 8, 1, 13),           # persistent: only some grids
    (0, 0, 8, 8, 8, 1, 14),
])
def test_invalid_tables_are_refused_whole(lib, bad):
    lib.sgemm_set_dispatch_overrides([(0, 0, 100, 100, 100, 1, "S64x64")])
    st = lib.sgemm_set_dispatch_overrides([(0, 0, 200, 200, 200, 1, "S64x64"), bad], check=False)
    assert st == -24 and "dispatch override" in lib.sgemm_status_string(st)
    assert lib.sgemm_dispatch_override_count() == 1
    assert sel(lib, 0, 0, 100, 100, 100) == lib.VARIANT_S64x64
    with pytest.raises(lib.SgemmError):
        lib.sgemm_set_dispatch_overrides([bad])


def test_count_and_null_entries_refused(lib):
    f = lib._load().sgemm_set_dispatch_overrides
    assert f(None, 1) == -24
    assert f(None, -1) == -25
    assert f(None, lib.MAX_DISPATCH_OVERRIDES + 1) == -25
    assert "count" in lib.sgemm_status_string(-25)
    assert f(None, 0) == 0


def test_load_from_a_tuning_file(lib, tmp_path):
    path = tmp_path / "overrides.json"
    path.write_text(json.dumps([[0, 0, 1536, 1536, 2048, 1, "S64x64"],
                                [1, 0, 512, 512, 520, 64, 0]]))
    assert lib.load_dispatch_overrides(str(path)) == 0
    assert sel(lib, 0, 0, 1536, 1536, 2048) == lib.VARIANT_S64x64
    assert sel(lib, 1, 0, 512, 512, 520, batch=64) == lib.VARIANT_L256x128


def test_replacement_while_other_threads_choose(lib):
    """Lookups from several threads while the table is replaced and cleared
    over and over: every answer is the model's or the record's."""
    model = sel(lib, 0, 0, 1024, 1024, 1024)
    stop = threading.Event()
    seen, errors = set(), []

    def chooser():
        while not stop.is_set():
            v = sel(lib, 0, 0, 1024, 1024, 1024)
            seen.add(v)
            if v not in (model, lib.VARIANT_M128x128):
                errors.append(v)

    threads = [threading.Thread(target=chooser) for _ in range(4)]
    for t in threads:
        t.start()
    records = [(0, 0, 1024, 1024, 1024, 1, "M128x128")] + \
              [(0, 0, 64 + i, 64, 64, 1, "S64x64") for i in range(500)]
    for i in range(300):
        lib.sgemm_set_dispatch_overrides(records if i % 2 == 0 else [])
    stop.set()
    for t in threads:
        t.join()
    assert not errors
    assert model in seen or lib.VARIANT_M128x128 in seen


def test_sweep_rows_become_override_records(lib):
    """tune.overrides_from keeps the shapes the automatic choice missed by at
    least the threshold, names the fastest variant, skips variants that run
    only some shapes, and describes a vector operand as the chooser sees it."""
    from precision_gemm_amd import tune

    def row(tA, tB, M, N, K, batch, best, auto, regret):
        return {"shape": {"transA": tA, "transB": tB, "M": M, "N": N, "K": K, "batch": batch,
                          "beta": 0.0}, "best": best, "auto": auto, "regret": regret}

    rows = [row(0, 0, 4096, 4096, 256, 1, "L256x128", "M128x128", 0.074),
            row(0, 0, 2048, 2048, 2048, 1, "M128x128", "M128x128", 0.0),
            row(0, 0, 1000, 1000, 1000, 1, "S64x64", "S64x64_K2", 0.01),
            row(0, 0, 16384, 1, 4096, 1, "T64x32", "GEMV", 0.05),
            row(1, 0, 1, 16384, 4096, 1, "T32x64", "GEMV", 0.03),
            row(0, 0, 512, 512, 520, 64, "P128x128", "M128x128", 0.2)]
    recs = tune.overrides_from(rows, min_regret=0.02)
    assert recs == [[0, 0, 4096, 4096, 256, 1, "L256x128"],
                    [0, 1, 16384, 1, 4096, 1, "T64x32"],
                    [0, 0, 1, 16384, 4096, 1, "T32x64"]]
    assert lib.sgemm_set_dispatch_overrides(recs) == 0
    assert sel(lib, 0, 0, 4096, 4096, 256) == lib.VARIANT_L256x128
    # the vector shapes as the chooser receives them (B described k-contiguous)
    assert sel(lib, 0, 1, 16384, 1, 4096) == lib.VARIANT_T64x32
    assert sel(lib, 0, 0, 1, 16384, 4096) == lib.VARIANT_T32x64
    assert tune.overrides_from(rows, min_regret=0.1) == []


def test_override_records_judged_over_both_modes(lib):
    """With the same shapes timed HBM-resident as well, a variant is judged by
    the sum of its two times: a win back to back that is a loss from HBM
    earns no record, a win in both does."""
    from precision_gemm_amd import tune

    def row(M, us, auto):
        best = min(us, key=us.get)
        return {"shape": {"transA": 0, "transB": 0, "M": M, "N": M, "K": M, "batch": 1,
                          "beta": 0.0}, "us": us, "best": best, "auto": auto,
                "regret": us[auto] / us[best] - 1.0}

    b2b = [row(1024, {"S64x64": 19.2, "S64x64_K2": 19.7}, "S64x64_K2"),
           row(1536, {"S64x64": 68.4, "S64x64_K2": 70.8}, "S64x64_K2")]
    hbm = [row(1024, {"S64x64": 26.8, "S64x64_K2": 21.1}, "S64x64_K2"),
           row(1536, {"S64x64": 69.0, "S64x64_K2": 71.0}, "S64x64_K2")]
    assert [r[2] for r in tune.overrides_from(b2b, 0.02)] == [1024, 1536]
    assert tune.overrides_from(b2b, 0.02, other=hbm) == [[0, 0, 1536, 1536, 1536, 1, "S64x64"]]
