"""Host-side checks of bench.py (no GPU): the single-GPU guard, the algorithmic byte
counts its roofline fields use, and the percentile helper."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_algorithmic_bytes_at_the_canonical_shape():
    # two-pass: gate and up read twice, QDATA and the 128-row-padded scales written once
    assert bench.producer_bytes(37810, 14336, True) == 4641423360
    # single read: inputs once
    assert bench.producer_single_read_bytes(37810, 14336, True) == 2473246720
    # GEMM distinct data: A and W with scales, the padded bf16 output
    a = 37824 * 7168 + 37888 * 896
    w = 5376 * 7168 + 5376 * 896
    assert bench.gemm_bytes(37810, 5376, 14336) == a + w + 37824 * 5376 * 2


def test_percentiles_nearest_rank():
    p = bench.percentiles([float(i) for i in range(1, 11)])
    assert p == {"p10": 1.0, "p50": 5.0, "p90": 9.0}  # ranks ceil(q n): 1, 5, 9
    assert bench.percentiles([3.0]) == {"p10": 3.0, "p50": 3.0, "p90": 3.0}


def test_traffic_summaries_match_the_sources():
    """The committed counter summaries were taken on the kernel sources in the tree,
    so the bench line reports their traffic rather than null."""
    assert bench.measured_gemm_traffic() is not None
    assert bench.measured_traffic(bench.PRODUCER_TRAFFIC_SUMMARY, bench.PRODUCER_SOURCES) is not None
    assert bench.measured_traffic(bench.SINGLE_READ_TRAFFIC_SUMMARY, bench.PRODUCER_SOURCES) is not None


def test_traffic_run_names_its_own_profiled_run():
    """The traffic figure is labelled as coming from the separate profiled runs, with
    that command's own kernel-trace time and the fraction of peak at that time."""
    r = bench.traffic_run(bench.GEMM_TRAFFIC_SUMMARY, bench.GEMM_SOURCES, 2.0 * 37810 * 5376 * 14336,
                          bench.PEAK_MFMA_TFLOPS, 1e12)
    assert r is not None and "separate" in r["source"] and r["summary"] == bench.GEMM_TRAFFIC_SUMMARY
    assert 1.0 < r["trace_ms_per_launch"] < 10.0
    assert abs(r["frac_at_trace_ms"] - 2.0 * 37810 * 5376 * 14336 / (r["trace_ms_per_launch"] * 1e-3) / 1e12 /
               bench.PEAK_MFMA_TFLOPS) < 1e-3
    p = bench.traffic_run(bench.PRODUCER_TRAFFIC_SUMMARY, bench.PRODUCER_SOURCES, 4641423360, bench.PEAK_HBM_GBS, 1e9)
    assert p is not None and 0.3 < p["trace_ms_per_launch"] < 3.0


def test_source_digest_ignores_comments_only(tmp_path):
    """A summary stays valid across comment edits and is retired by any code edit."""
    a = tmp_path / "a.hip"
    a.write_text("int x = 1; // one\n/* block\n   comment */ int y;\n")
    b = tmp_path / "b.hip"
    b.write_text("int x = 1;   // other words\n\nint y;\n")
    c = tmp_path / "c.hip"
    c.write_text("int x = 2;\nint y;\n")
    assert bench.source_digest([str(a)]) == bench.source_digest([str(b)])
    assert bench.source_digest([str(a)]) != bench.source_digest([str(c)])


def test_host_cpu_names_the_host():
    h = bench.host_cpu()
    assert h["nproc"] >= 1 and h["os_cpu_count"] >= h["nproc"] and h["cpu_model"]
    assert 1 <= bench.baseline_threads() <= h["nproc"]
