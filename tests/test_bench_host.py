"""Host-side pieces of bench.py: the amd-smi sample parser (socket power and XCD clocks)."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _smi_json(power, clocks):
    clock = {f"gfx_{i}": {"clk": {"value": c, "unit": "MHz"}, "min_clk": {"value": 500, "unit": "MHz"},
                          "max_clk": {"value": 2400, "unit": "MHz"}, "clk_locked": "DISABLED",
                          "deep_sleep": "DISABLED"} for i, c in enumerate(clocks)}
    clock["mem_0"] = {"clk": {"value": 1900, "unit": "MHz"}}
    clock["vclk_0"] = {"clk": "N/A"}
    return json.dumps({"gpu_data": [{"gpu": 0, "power": {"socket_power": {"value": power, "unit": "W"},
                                                          "gfx_voltage": "N/A"}, "clock": clock}]})


def test_smi_sample_reads_socket_power_and_xcd_clocks(monkeypatch):
    out = _smi_json(1308, [1941, 1885, 1947, 1863, 1895, 1878, 1915, 1900])
    monkeypatch.setattr(subprocess, "run", lambda *a, **k: subprocess.CompletedProcess(a, 0, out, ""))
    w, clk = bench._smi_sample()
    assert w == 1308.0
    assert clk == [1941.0, 1885.0, 1947.0, 1863.0, 1895.0, 1878.0, 1915.0, 1900.0]  # gfx_* only


def test_smi_sample_missing_or_garbled_gives_none(monkeypatch):
    monkeypatch.setattr(subprocess, "run", lambda *a, **k: subprocess.CompletedProcess(a, 0, "not json", ""))
    assert bench._smi_sample() is None

    def boom(*a, **k):
        raise FileNotFoundError("amd-smi")

    monkeypatch.setattr(subprocess, "run", boom)
    assert bench._smi_sample() is None
    na = json.dumps({"gpu_data": [{"power": {"socket_power": "N/A"}, "clock": {}}]})
    monkeypatch.setattr(subprocess, "run", lambda *a, **k: subprocess.CompletedProcess(a, 0, na, ""))
    assert bench._smi_sample() is None

