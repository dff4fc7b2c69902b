"""The bench.py contract: one JSON line with the fields the measurement needs, and a refusal of
more than one GPU (this path runs on one)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def test_more_than_one_gpu_is_refused():
    """--gpus 2 exits with status 2 and says why, before touching a GPU."""
    r = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


@pytest.mark.gpu
def test_bench_line_fields_small_workload():
    """A short run on the small fp32 workload prints exactly one JSON line carrying the metric,
    the per-step statistics, the per-kernel times and a roofline block for the binding kernel."""
    r = subprocess.run([sys.executable, "-u", BENCH, "--workload", "flare_encode_fp32_B1_H1_N1024_M16_D32_R4",
                        "--steps", "5", "--warmup", "2", "--no-cpu-baseline"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
              "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "step_ms", "phases_ms"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 5 and d["warmup"] == 2
    assert d["value"] > 0 and d["ms_per_step"] > 0
    assert d["step_ms"]["min"] <= d["step_ms"]["median"] <= max(d["step_ms"]["mean"], d["step_ms"]["median"])
    ro = d["roofline"]
    for k in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert k in ro, k
    assert ro["peak"] == 8000.0 and 0 < ro["frac"] < 1
    assert all(v > 0 for v in d["phases_ms"].values())
