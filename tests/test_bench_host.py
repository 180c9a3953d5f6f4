"""Host-side pieces of bench.py: the amd-smi sample parser (socket power and XCD clocks) and the
HBM-traffic summaries made from rocprofv3 counter runs."""
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



def _pmc_csv(path, rows):
    """A rocprofv3 counter-collection CSV with the columns the summaries read."""
    with open(path, "w") as f:
        f.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
        for did, name, value in rows:
            f.write(f'{did},"{name}",C,{value}\n')


def test_backward_traffic_summary_scales_by_the_copy_and_averages_calls(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.md"))
    copy = "__amd_rocclr_copyBuffer"
    pre, dq, dkv = ("void ma::(anonymous namespace)::bwd_pre_kernel<128>(ma::BwdPreParams)",
                    "void ma::(anonymous namespace)::bwd_dq_kernel<128, false>(ma::BwdParams)",
                    "void ma::(anonymous namespace)::bwd_dkv_kernel<128, false>(ma::BwdParams)")
    other = "void ma::(anonymous namespace)::merge_kernel<128, true, 8, 2>(ma::MergeParams)"
    # a 1 MiB copy reads 512 KiB and writes 1024 KiB by the counters: factors 2 (fetch) and 1 (write)
    fetch = [(1, copy, 512), (2, pre, 10), (3, dq, 100), (4, dkv, 200), (5, other, 7), (6, pre, 20), (7, dq, 300),
             (8, dkv, 400)]
    write = [(1, copy, 1024), (2, pre, 1), (3, dq, 2), (4, dkv, 3), (5, other, 7), (6, pre, 4), (7, dq, 5), (8, dkv, 6)]
    _pmc_csv(tmp_path / "f.csv", fetch)
    _pmc_csv(tmp_path / "w.csv", write)
    bench.summarize_pmc(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), 1, "rocprofv3 --pmc PMC -- cmd")
    calls = [2 * (10 + 100 + 200) + (1 + 2 + 3), 2 * (20 + 300 + 400) + (4 + 5 + 6)]  # KiB
    expect = round(sum(calls) / 2 * 1024)
    assert bench.stored_traffic() == expect
    text = (tmp_path / "traffic.md").read_text()
    assert "rocprofv3 --pmc FETCH_SIZE -- cmd" in text and "rocprofv3 --pmc WRITE_SIZE -- cmd" in text
    # a summary taken on other kernel sources is not reported
    (tmp_path / "traffic.md").write_text(text.replace(bench.kernel_source_hash(), "0" * 64))
    assert bench.stored_traffic() is None


def test_small_tile_traffic_summary_counts_the_table_launches_per_call(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "SMALL_TRAFFIC_FILE", str(tmp_path / "small.md"))
    copy = "__amd_rocclr_copyBuffer"
    res = "void ma::(anonymous namespace)::fwd_bf16_resident_kernel<128, true>(ma::FwdParams)"
    res_ka = "void ma::(anonymous namespace)::fwd_bf16_resident_kernel<128, false>(ma::FwdParams)"
    ring = "void ma::(anonymous namespace)::fwd_bf16_kernel<128, false, 4>(ma::FwdParams)"
    # dispatch 0 is a small tile-table upload the runtime blits: not the calibration copy
    fetch = [(0, copy, 3), (1, ring, 999), (2, res, 30), (3, res, 50), (4, res, 70), (5, res, 90), (6, copy, 512),
             (7, res_ka, 999)]
    write = [(0, copy, 0.03), (1, ring, 999), (2, res, 100), (3, res, 100), (4, res, 100), (5, res, 100),
             (6, copy, 1024), (7, res_ka, 999)]
    _pmc_csv(tmp_path / "f.csv", fetch)
    _pmc_csv(tmp_path / "w.csv", write)
    bench.summarize_pmc_small(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), 1, 2, "rocprofv3 --pmc PMC -- cmd")
    expect = round((2 * (30 + 50 + 70 + 90) + 400) * 1024 / 2)
    assert bench.stored_traffic(bench.SMALL_TRAFFIC_FILE, "fwd_p210_bytes_per_call") == expect
    assert bench.stored_traffic(bench.SMALL_TRAFFIC_FILE, "no_such_key") is None


def test_kernel_source_hash_ignores_comments_only():
    src = ('int f(int a) {  // the sum\n  /* block\n comment */ return a + 1;\n}\n'
           'const char* s = "not // a comment /* either */";\n')
    assert bench.strip_comments(src) == ('int f(int a) {\n   return a + 1;\n}\n'
                                         'const char* s = "not // a comment /* either */";')
    assert bench.strip_comments(src.replace("the sum", "one more")) == bench.strip_comments(src)
    assert bench.strip_comments(src.replace("a + 1", "a + 2")) != bench.strip_comments(src)
