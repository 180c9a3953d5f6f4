"""bench.py keeps its output contract on the MI355X: one JSON line with the metric, the whole-job
value, the step's timing, the workload, a roofline block for the dominant kernel and the oracle's
CPU baseline (a short run: one warm-up and one timed step, the smallest configuration block)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args, timeout=600):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT, capture_output=True,
                          text=True, timeout=timeout)


@pytest.mark.gpu
def test_bench_json_line():
    r = _run("--steps", "1", "--warmup", "1", "--configs", "c1", "--power-sample", "0", "--cpu-rows", "8",
             "--reps-scale", "0.1")
    assert r.returncode == 0, r.stderr[-3000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
                "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 1 and d["warmup"] == 1
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert d["unit"] == "TFLOP/s" and d["dtype"] == "bf16" and d["vs_baseline"] is None
    assert isinstance(d["config"].get("workload"), str) and "model" not in d["config"]
    rf = d["roofline"]
    assert rf["bound"] in ("hbm", "mfma", "alu") and rf["unit"] in ("GB/s", "TFLOP/s")
    assert rf["peak"] > 0 and 0 < rf["achieved"] <= rf["peak"]
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    assert rf["traffic"] is None or rf["traffic"] > 0
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1 and cb["sample"]
    assert "c1" in d["configs"] and "roofline" in d["configs"]["c1"]


def test_bench_refuses_several_gpus():  # before any GPU work: runs on the host too
    r = _run("--gpus", "2", timeout=120)
    assert r.returncode == 2 and "one GPU" in (r.stdout + r.stderr)
