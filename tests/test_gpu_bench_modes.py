"""The bench's single-kernel modes (the ones the profiler commands run) on the tiny
workload: each prints one JSON line with its timing fields."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args):
    print(f"[bench] {' '.join(args)}", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "tiny", "--steps", "2",
                        "--warmup", "1", *args], capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout
    return json.loads(lines[0])


def test_only_gemm_with_copy_calibration(gpu):
    d = run_bench("--only-gemm", "--copy-bytes", str(1 << 24))
    assert d["gemm_ms"] > 0 and d["copy_bytes"] == 1 << 24 and d["copy_gbs"] > 0


def test_only_producer_two_pass_and_single_read(gpu):
    d2 = run_bench("--only-producer")
    d1 = run_bench("--only-producer", "--single-read")
    assert d2["producer_ms"] > 0 and d1["producer_ms"] > 0
    assert d1["algorithmic_bytes"] < d2["algorithmic_bytes"]


def test_profile_step_with_copy_calibration(gpu):
    """The timed step alone (the profiler's command): producer and GEMM timings."""
    d = run_bench("--profile-step", "--copy-bytes", str(1 << 24))
    assert d["mode"] == "profile-step" and d["producer_ms"] > 0 and d["gemm_ms"] > 0
    assert d["dispatches_per_kernel"] == 3 and d["copy_gbs"] > 0


def test_chain_times_every_step_of_both_paths(gpu):
    """The FC1 -> FC2 block, fused against unfused (full size, one timed step): every
    step of each path is timed, the unfused path's elementwise kernels included."""
    d = run_bench("--chain")
    assert d["mode"] == "chain"
    assert set(d["fused"]) == {"modulate_quantize", "fc1_gemm", "fc2_producer", "fc2_gemm", "total_ms"}
    assert set(d["unfused"]) == {"modulate", "quantize", "fc1_gemm", "fc2_producer", "fc2_gemm", "bias_add",
                                 "gated_residual", "total_ms"}
    for path in ("fused", "unfused"):
        parts = {k: v for k, v in d[path].items() if k != "total_ms"}
        assert all(v > 0 for v in parts.values())
        assert abs(sum(parts.values()) - d[path]["total_ms"]) < 1e-3
