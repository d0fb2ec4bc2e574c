"""The dispatch sweep tool (precision_gemm_amd.tune) on the GPU: one small
shape in each timing mode, with short timing windows. Every applicable
variant gets a time, the fastest and the automatic choice are among them, and
the regret is consistent with the times. Then the loop from a sweep to an
installed per-shape override table."""
import sys

import pytest

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("hbm", [False, True])
def test_sweep_reports_every_variant(hbm):
    import io

    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import precision_gemm_amd as pg
    from precision_gemm_amd import tune
    sys.stdout.write(f"[tune] sweep of one shape, hbm={hbm}\n")
    sys.stdout.flush()
    out = io.StringIO()
    rows = tune.sweep([(0, 1, 640, 384, 1000, 1, 1.0)], rounds=1, target_ms=2.0, hbm=hbm,
                      out=out)
    assert len(rows) == 1
    r = rows[0]
    assert r["mode"] == ("hbm_resident" if hbm else "back_to_back")
    assert r["copies"] >= (4 if hbm else 1)
    names = set(r["us"])
    assert pg.VARIANT_NAMES[pg.VARIANT_M128x128] in names and "GEMV" not in names
    assert r["best"] in names and r["auto"] in names
    assert all(t > 0 for t in r["us"].values())
    best, auto = r["us"][r["best"]], r["us"][r["auto"]]
    assert best == min(r["us"].values())
    assert r["regret"] == pytest.approx(auto / best - 1.0, abs=1e-3)
    assert "regret" in out.getvalue()


def test_sweep_to_override_table():
    """The tuning loop end to end on two small shapes: a sweep in each timing
    mode, override records judged over both (threshold 0, so any shape whose
    fastest variant is not the automatic one gets a record), installed; the
    automatic choice then names each record's variant."""
    import io

    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import precision_gemm_amd as pg
    from precision_gemm_amd import tune
    shapes = [(0, 0, 1536, 1536, 1536, 1, 0.0), (1, 0, 512, 512, 520, 8, 0.0)]
    out = io.StringIO()
    runs = [tune.sweep(shapes, rounds=1, target_ms=2.0, hbm=h, out=out) for h in (False, True)]
    records = tune.overrides_from(runs[0], 0.0, other=runs[1])
    sys.stdout.write(f"[tune] records: {records}\n")
    sys.stdout.flush()
    assert all(len(r) == 7 and r[6] not in tune.NOT_OVERRIDABLE for r in records)
    try:
        assert pg.sgemm_set_dispatch_overrides(records) == 0
        for tA, tB, M, N, K, batch, name in records:
            assert pg.VARIANT_NAMES[pg.sgemm_select_variant(tA, tB, M, N, K, batch, 1, 256)] == name
    finally:
        pg.sgemm_set_dispatch_overrides([])
