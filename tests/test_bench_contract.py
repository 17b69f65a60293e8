"""The bench's command-line contract: one JSON line with the required fields
(GPU), and a clear refusal of more than one GPU (CPU, before any GPU use)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True,
                         timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout.strip() == ""


@pytest.mark.gpu
def test_bench_prints_one_complete_json_line():
    # A child process (never an exec of this one): the small workload, few steps.
    res = subprocess.run([sys.executable, BENCH, "--workload", "tiny", "--steps", "20",
                          "--warmup", "20", "--cpu-budget", "1", "--kernel-reps", "20"],
                         capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stderr[-3000:]
    lines = [l for l in res.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, res.stdout
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline", "path_counters", "device_us_trials"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 20 and d["warmup"] >= 20
    assert d["higher_is_better"] is False and d["unit"] == "us" and d["value"] > 0
    assert abs(d["ms_per_step"] * 1e3 - d["value"]) < 1e-2
    assert d["config"]["workload"] == "tiny"
    r = d["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in r, key
    assert r["bound"] == "hbm" and r["peak"] == 8000.0 and r["unit"] == "GB/s"
    assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["cores"] >= 1 and c["value"] > 0 and c["sample"]
    # The timed steps are split launches (two partitions) with their reduces.
    pc = d["path_counters"]
    assert pc["split_launches"] == 20 and pc["reduce_launches"] == 20
