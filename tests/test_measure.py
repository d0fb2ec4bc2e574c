"""Pins for the report's counting and roofline arithmetic against numbers the
pages print (fixtures under tests/golden, each with its citation)."""
import pytest

from conftest import read_golden
from precision_gemm_amd import measure
import workloads


def test_page_counts_for_4092():
    g = read_golden("page_counts.txt")
    flops = measure.gemm_flops(4092, 4092, 4092)
    assert round(flops / 1e9) == g["gemm_4092_gflop"]
    assert flops == workloads.HEADLINE.flops()
    assert round(measure.naive_kernel_read_bytes(4092, 4092, 4092) / 1e9) == g["naive_read_gb"]
    assert measure.block_tile_intensity(128, 128) == g["block_ai_128"]
    assert measure.block_tile_intensity(32, 32) == g["block_ai_32"]
    tm = 8
    assert (1 + tm) / tm == g["loads_per_fma_tm8"]


def test_roofline_reproduces_printed_lab_output():
    g = read_golden("roofline_p3.txt")
    peak, bw = g["peak_tflops"] * 1e12, g["bw_tbs"] * 1e12
    soft = measure.place_on_roofline(g["softmax_ai"] * 1000.0, 1000.0, peak, bw)
    assert f"{soft.ridge:.1f}" == f"{g['ridge']:.1f}"
    assert soft.bound == "memory-bound"
    assert f"{soft.attainable / 1e12:.1f}" == f"{g['softmax_attainable_tflops']:.1f}"
    assert f"{soft.frac_of_peak * 100:.1f}" == f"{g['softmax_pct']:.1f}"
    gemm = measure.place_on_roofline(g["gemm_ai"] * 1000.0, 1000.0, peak, bw)
    assert gemm.bound == "compute-bound"
    assert f"{gemm.attainable / 1e12:.1f}" == f"{g['gemm_attainable_tflops']:.1f}"
    assert f"{gemm.frac_of_peak * 100:.1f}" == f"{g['gemm_pct']:.1f}"
    # the printed GEMM intensity is 2N^3 flops over three N x N matrices of 2-byte elements
    n = 4096
    assert f"{2 * n**3 / (3 * n * n * 2):.1f}" == f"{g['gemm_ai']:.1f}"


def test_mi355x_workload_rooflines():
    """The five workloads against MI355X FP32-MFMA peak and HBM bandwidth."""
    by = workloads.BY_NAME
    roofs = {n: measure.place_on_roofline(w.flops(), w.algorithmic_bytes(),
                                 measure.MI355X_FP32_MFMA_PEAK, measure.MI355X_HBM_BW)
             for n, w in by.items()}
    assert roofs["sgemm_4092"].bound == "compute-bound"
    assert roofs["sgemm_4092"].intensity == pytest.approx(511.5, abs=0.05)
    assert roofs["skinny_16384x64x4096_nt"].intensity == pytest.approx(30.9, abs=0.05)
    assert roofs["sgemm_4092"].ridge == pytest.approx(19.66, abs=0.01)
    # 70 % of FP32-MFMA peak at 4092^3 is 110.1 TFLOP/s, i.e. at most 1.2445 ms
    t = by["sgemm_4092"].flops() / (0.7 * measure.MI355X_FP32_MFMA_PEAK)
    assert t == pytest.approx(1.2445e-3, rel=1e-4)


def test_bench_roofline_bound_follows_the_ridge():
    """bench.py reports a call above the ridge against the FP32-MFMA peak and a
    matrix-vector product (below it) against the HBM peak, in GB/s of
    algorithmic bytes."""
    import bench
    peak, bw = measure.MI355X_FP32_MFMA_PEAK, measure.MI355X_HBM_BW
    gemv = workloads.BY_NAME["gemv_16384x1x4096_nt"]
    roof = measure.place_on_roofline(gemv.flops(), gemv.algorithmic_bytes(), peak, bw)
    assert roof.bound == "memory-bound" and roof.intensity == pytest.approx(0.5, abs=0.01)
    ms = 0.04
    tflops = gemv.flops() / (ms * 1e-3) / 1e12
    e = bench.roofline_entry(gemv, roof, tflops, peak / 1e12, ms, None)
    assert (e["bound"], e["unit"], e["peak"]) == ("hbm", "GB/s", 8000.0)
    assert e["achieved"] == pytest.approx(gemv.algorithmic_bytes() / (ms * 1e-3) / 1e9, rel=1e-3)
    assert e["frac"] == pytest.approx(e["achieved"] / 8000.0, abs=1e-4)
    big = workloads.BY_NAME["sgemm_4092"]
    roof = measure.place_on_roofline(big.flops(), big.algorithmic_bytes(), peak, bw)
    ms = 0.91
    tflops = big.flops() / (ms * 1e-3) / 1e12
    e = bench.roofline_entry(big, roof, tflops, peak / 1e12, ms, 123)
    assert (e["bound"], e["unit"], e["traffic"]) == ("mfma", "TFLOP/s", 123)
    assert e["achieved"] == pytest.approx(tflops, abs=1e-3)
    assert e["hbm_frac_at_achieved"] == pytest.approx(e["hbm_gbs_at_achieved"] / 8000.0, abs=1e-4)
    # the skinny product is reported against HBM from its HBM-resident time,
    # with its MFMA fraction beside it
    sk = workloads.BY_NAME["skinny_16384x64x4096_nt"]
    roof = measure.place_on_roofline(sk.flops(), sk.algorithmic_bytes(), peak, bw)
    assert roof.bound == "compute-bound"
    ms = 0.1
    tflops = sk.flops() / (ms * 1e-3) / 1e12
    e = bench.roofline_entry(sk, roof, tflops, peak / 1e12, ms, None, hbm_figure=True)
    assert (e["bound"], e["unit"], e["timing"]) == ("hbm", "GB/s", "hbm_resident")
    assert e["achieved"] == pytest.approx(277_872_640 / 1e-4 / 1e9, rel=1e-4)
    assert e["mfma_frac_at_achieved"] == pytest.approx(tflops / 157.3, abs=1e-4)
    assert "skinny_16384x64x4096_nt" in bench.HBM_FIGURE


def test_bench_counter_summary_is_tied_to_kernel_code_and_variant(tmp_path, monkeypatch):
    """bench.py takes traffic and clock figures from the committed counter
    summary only while it describes the current kernel code and the variant
    the run launches, per timing mode."""
    import json
    import bench
    sha = bench.kernel_source_hash()
    data = {"sgemm_4092": {"kernel_sha": sha, "variant": "M128x128", "bytes_per_launch": 11,
                           "gui_cycles": 2_208_000, "counter_dur_ns": 920_000},
            "sgemm_4092@hbm": {"kernel_sha": sha, "variant": "M128x128", "bytes_per_launch": 22,
                               "gui_cycles": 2_198_100, "counter_dur_ns": 919_700},
            "sgemm_1024": {"kernel_sha": "stale", "variant": "S64x64_K2", "bytes_per_launch": 33},
            "skinny_16384x64x4096_nt": {"kernel_sha": sha, "variant": "T64x64",
                                        "bytes_per_launch": 44, "gui_cycles": 178_300,
                                        "counter_dur_ns": 68_950}}
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps(data))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    assert bench.load_traffic("sgemm_4092", "M128x128") == 11
    assert bench.load_traffic("sgemm_4092", "M128x128", "hbm_resident") == 22
    assert bench.load_traffic("sgemm_4092", "L256x128") is None
    assert bench.load_traffic("sgemm_1024", "S64x64_K2") is None
    clk = bench.clock_report("sgemm_4092", "M128x128")
    assert clk["back_to_back"]["sclk_mhz"] == 2400 and clk["hbm_resident"]["sclk_mhz"] == 2390
    assert bench.clock_report("sgemm_1024", "S64x64_K2")["back_to_back"] is None
    # a 69 us kernel: the raw quotient (2586 MHz, above the part's 2.4 GHz) is
    # reported, but not as the clock
    short = bench.clock_report("skinny_16384x64x4096_nt", "T64x64")["back_to_back"]
    assert short["sclk_mhz"] is None and short["gui_active_mhz"] == 2586


def test_bench_host_and_rocm_records(tmp_path, monkeypatch):
    """The bench line names the host CPU (model, family and model numbers,
    cores usable) and the installed ROCm release from its version file, or
    None where there is no such file."""
    import bench
    h = bench.host_info()
    assert set(h) >= {"cpu_model", "cpu_family", "cpu_model_number", "cores_available"}
    assert h["cores_available"] >= 1
    (tmp_path / ".info").mkdir()
    (tmp_path / ".info" / "version").write_text("9.8.7-123\n")
    monkeypatch.setenv("ROCM_PATH", str(tmp_path))
    assert bench.rocm_version() == "9.8.7-123"
    monkeypatch.setenv("ROCM_PATH", str(tmp_path / "absent"))
    assert bench.rocm_version() is None
