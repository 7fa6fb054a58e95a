"""bench.py's GPU paths, run as the command line runs them (small workloads).

The bench line of a forward and of a split-KV workload must carry the
roofline, per-launch and clock fields; --launch-trace must time every launch
and give each a plausible clock.
"""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args):
    r = subprocess.run([sys.executable, "bench.py", *args], cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    return json.loads(r.stdout.strip().splitlines()[-1])


def test_bench_line_of_a_forward_workload():
    d = run_bench("--workload", "c2", "--steps", "5", "--warmup", "2", "--no-cpu-baseline")
    assert d["unit"] == "TFLOPS" and d["value"] > 0 and d["steps"] == 5 and d["warmup"] == 2
    rf = d["roofline"]
    assert rf["bound"] == "mfma" and rf["kernel"] == "fa_fwd_serial_kernel"
    assert abs(rf["frac"] - d["value"] / rf["peak"]) < 1e-3
    assert 0 < d["per_launch_ms"]["min"] <= d["per_launch_ms"]["median"]
    c = d["clock"]
    assert 0.3 < c["shader_ghz"] < 3.5 and 0.3 < c["timed_region_ghz_est"] < 3.5
    # the estimate is the clock after the region scaled by the duration ratio
    ratio = d["per_launch_ms"]["median"] / d["ms_per_step"]
    assert abs(c["timed_region_ghz_est"] - c["shader_ghz"] * ratio) < 2e-3


def test_bench_line_of_the_decode_workload():
    d = run_bench("--workload", "c6", "--steps", "3", "--warmup", "1", "--no-cpu-baseline")
    assert d["unit"] == "GB/s" and d["value"] > 0 and d["roofline"]["bound"] == "hbm"
    assert "clock" not in d


def test_launch_trace():
    d = run_bench("--workload", "c2", "--launch-trace", "12")
    assert d["launches"] == 12 and len(d["us"]) == 12 and len(d["shader_ghz"]) == 12
    assert all(u > 0 for u in d["us"])
    assert all(g is not None and 0.3 < g < 3.5 for g in d["shader_ghz"])
    assert d["mean_us"]["6-25"] is not None and d["mean_us"]["46-"] is None
