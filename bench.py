"""Bench of one GPU's share of distributed long-context attention on MI355X.

Headline step (printed as ONE JSON line): one pass of the whole hot path over the Mesh-Attention
share of GPU 9 of n = 64 at S = 1,048,576 tokens ([Mesh] section 3.3, KV partition rotation):
8 Q partitions x 8 KV partitions of 16384 tokens, 32 query / 8 KV heads, head_dim 128, bf16,
non-causal:

  1. host mapping: the GPU's Q and KV partitions, its groups and the pair work list (C++ mapper);
  2. mesh_attn_tile_fwd  -> 64 partial (O, LSE), one call;
  3. mesh_attn_merge     -> seven 8-way merges and the owned partition's 15-way merge (its 8
                            partials plus 7 incoming seeded partials, as the reduce-scatter with
                            online softmax brings them);
  4. mesh_attn_tile_bwd  -> dQ of the 8 Q partitions (summed over the 8 KV partitions) and dK/dV of
                            the 8 KV partitions (summed over the 8 Q partitions), one call, from the
                            merged O and LSE and a seeded dO.

`value` is the step's algorithmic tile FLOPs (forward 4*d*Hq and backward 10*d*Hq per allowed pair)
per second of wall time, inputs resident in HBM.  Per-part times come from HIP events recorded on
the stream the kernels are launched on (torch's current stream, which the binding passes).

After the headline, `configs` reports each configuration of the hot path on its own (rates and
fractions of peak, a roofline block for its dominant kernel, and the fp64 oracle timed on a
bounded sample of it): fp32 S=256 in 4 partitions; the 8k GQA tile; the zigzag causal share of
S=131072; the Mesh 8x8 share (fused, GOO replay, gradient add-reduce); the 4 x 8k backward; the
striped causal variant of the Mesh share; and the small-tile sweep.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "tile fwd/bwd TFLOP/s + % bf16 MFMA peak; merge GB/s + % HBM peak (1 GPU)"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 vector
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E

HQ, HKV, D = 32, 8, 128
# the Mesh share: GPU g of n = a * b, partitions of P tokens
MESH_N, MESH_A, MESH_B, MESH_G, MESH_P = 64, 8, 8, 9, 16384
CONFIG_NAMES = ["c1", "c2", "c3", "c4", "c5", "striped", "small"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10, help="timed headline steps")
    ap.add_argument("--warmup", type=int, default=2, help="untimed headline steps before them")
    ap.add_argument("--no-step", action="store_true", help="skip the headline step (per-config runs only)")
    ap.add_argument("--configs", default=",".join(CONFIG_NAMES),
                    help="per-config blocks after the step (comma list; 'none' for none): " + ", ".join(CONFIG_NAMES))
    ap.add_argument("--reps-scale", type=float, default=1.0, help="scales every per-config repetition count")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=128, help="query rows of the headline's oracle sample")
    ap.add_argument("--power-sample", type=float, default=3.0,
                    help="after the timed steps (outside the timed region), run the headline forward and then "
                         "backward back to back for this many seconds each while sampling socket power and "
                         "shader clocks with amd-smi (0: off)")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="after the timed steps, one plain device copy of this many MiB (outside the timed "
                         "region): the reference launch for scaling HBM byte counters")
    return ap.parse_args()


# ------------------------------------------------------------------ helpers --

def cpu_info():
    model = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model, len(os.sched_getaffinity(0))


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return 1


def _median(xs):
    return statistics.median(xs) if xs else float("nan")


def timed(fn, reps, warmup):
    """Median and mean milliseconds of fn() over `reps` runs after `warmup` runs, from events
    recorded on the current stream around each run.  The runs are enqueued back to back and the
    host synchronises once at the end, so host pauses between launches stay behind queued work."""
    import torch
    for _ in range(warmup):
        fn()
    stream = torch.cuda.current_stream()
    evs = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        evs.append((e0, e1))
    torch.cuda.synchronize()
    ts = [a.elapsed_time(b) for a, b in evs]
    return _median(ts), sum(ts) / len(ts)


def reps_of(n, args):
    return max(1, int(round(n * args.reps_scale)))


def tf(flop, ms, mean_ms=None, reps=None):
    t = flop / (ms * 1e-3) / 1e12
    r = {"ms": round(ms, 4), "TFLOP/s": round(t, 1), "frac_bf16_peak": round(t / PEAK_BF16_TFLOPS, 4), "flop": flop}
    if mean_ms is not None:
        r["ms_mean"] = round(mean_ms, 4)
    if reps is not None:
        r["reps"] = reps
    return r


def gb(nbytes, ms, mean_ms=None, reps=None):
    g = nbytes / (ms * 1e-3) / 1e9
    r = {"ms": round(ms, 4), "GB/s": round(g, 1), "frac_hbm_peak": round(g / PEAK_HBM_GBPS, 4), "bytes": nbytes}
    if mean_ms is not None:
        r["ms_mean"] = round(mean_ms, 4)
    if reps is not None:
        r["reps"] = reps
    return r


def timed_tf(flop, fn, reps, warmup):
    med, mean = timed(fn, reps, warmup)
    return tf(flop, med, mean, reps)


def timed_gb(nbytes, fn, reps, warmup):
    med, mean = timed(fn, reps, warmup)
    return gb(nbytes, med, mean, reps)


def roofline_mfma(part, kernel, traffic=None):
    return {"bound": "mfma", "achieved": part["TFLOP/s"], "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": part["frac_bf16_peak"], "traffic": traffic, "kernel": kernel}


def mall_flush(scratch, it):
    """A 512 MiB read, so that the next kernel's inputs come from HBM, not the 256 MB MALL (a read
    leaves clean lines: no write-back drains while the next kernel runs)."""
    return scratch.max()


# ----------------------------------------------------------- power and clock --

def _smi_sample():
    """(socket power W, [shader clock MHz of each XCD]) from one amd-smi call, or None."""
    import subprocess
    try:
        r = subprocess.run(["amd-smi", "metric", "-g", "0", "-p", "-c", "--json"], capture_output=True, text=True,
                           timeout=10)
        d = json.loads(r.stdout)
        g = (d["gpu_data"] if isinstance(d, dict) else d)[0]
        w = g["power"]["socket_power"]["value"]
        clk = [v["clk"]["value"] for n, v in g["clock"].items()
               if n.startswith("gfx_") and isinstance(v, dict) and isinstance(v.get("clk", {}).get("value"), (int, float))]
        return (float(w), [float(c) for c in clk]) if isinstance(w, (int, float)) and clk else None
    except Exception:
        return None


def power_clock(runs, seconds):
    """Socket power and shader clock while each entry of `runs` (name, fn) is enqueued back to back
    for `seconds`; amd-smi refreshes about once a second, so the first second of a phase is dropped."""
    import threading
    import torch
    samples, label, stop = [], ["idle"], threading.Event()

    def sampler():
        while not stop.is_set():
            t = time.time()
            x = _smi_sample()
            if x:
                samples.append((t, label[0], x[0], statistics.mean(x[1])))
            time.sleep(0.25)

    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    time.sleep(1.5)
    res, starts = {}, {}
    for name, fn in runs:
        label[0] = name
        starts[name] = time.time()
        n, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            fn()
            n += 1
            torch.cuda.synchronize()
        res[name] = {"ms_per_call": round((time.perf_counter() - t0) * 1e3 / n, 4), "calls": n}
        label[0] = "idle"
        time.sleep(1.5)
    stop.set()
    th.join()
    for name in list(res) + ["idle"]:
        sel = [(w, c) for t, lab, w, c in samples if lab == name and (name == "idle" or t >= starts[name] + 1.0)]
        entry = res.setdefault(name, {})
        if sel:
            entry.update({"socket_w_median": statistics.median(w for w, _ in sel),
                          "gfx_mhz_median": round(statistics.median(c for _, c in sel)),
                          "gfx_mhz_range": [round(min(c for _, c in sel)), round(max(c for _, c in sel))],
                          "samples": len(sel)})
    return res


# ------------------------------------------------------------ HBM counters --

TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_tile_bwd_mesh_8x8_1m.md")
KERNEL_SOURCES = ["bwd.hip", "fwd_bf16.hip", "merge.hip", "api.hip", "ma_device.h", "ma_internal.h"]
BWD_KERNELS = ("bwd_pre_kernel", "bwd_dq_kernel", "bwd_dkv_kernel")


def strip_comments(src):
    """C++ source without its comments (// to the end of the line, /* ... */), blank lines and trailing
    blanks; string and character literals are kept as they are."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    lines = (line.rstrip() for line in "".join(out).splitlines())
    return "\n".join(line for line in lines if line)


def kernel_source_hash():
    """sha256 over the HIP sources the measured kernels are built from, comments left out (a change of
    the code invalidates stored counters; a change of a comment does not)."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "distributed_long_context_amd", "csrc")
    for name in KERNEL_SOURCES:
        with open(os.path.join(csrc, name)) as f:
            h.update(name.encode() + b"\0" + strip_comments(f.read()).encode())
    return h.hexdigest()


def stored_traffic(path=None, key="tile_bwd_bytes_per_launch"):
    """HBM bytes per call from a committed counter summary (default: the headline's tile backward),
    or None when the summary is missing or was taken on other kernel sources."""
    try:
        with open(path or TRAFFIC_FILE) as f:
            text = f.read()
    except OSError:
        return None
    vals = {}
    for line in text.splitlines():
        if line.startswith("    ") and ":" in line:
            k, v = line.strip().split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("source_sha256") != kernel_source_hash():
        return None
    try:
        return int(vals[key])
    except (KeyError, ValueError):
        return None


SMALL_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_fwd_small_tiles_210.md")


def _pmc_per_dispatch(path):
    import csv
    import collections
    by = collections.OrderedDict()
    for r in csv.DictReader(open(path)):
        key = (int(r["Dispatch_Id"]), r["Kernel_Name"])
        by[key] = by.get(key, 0.0) + float(r["Counter_Value"])
    return by


def _calib_copy(per_dispatch):
    """The counter value of the calibration copy: the largest runtime blit (__amd_rocclr_copyBuffer)
    in the run.  The runtime also blits small host-to-device copies, such as the tile tables."""
    return max(v for (_, n), v in per_dispatch.items() if "copyBuffer" in n)


def summarize_pmc_small(fetch_csv, write_csv, copy_mib, calls, command):
    """Write the HBM-traffic summary of the 210-token small-tile forward (every dispatch of the
    tile-table instance of the resident-KV kernel in the run belongs to its `calls` calls) from two
    rocprofv3 --pmc runs, scaled like summarize_pmc by the plain device copy of copy_mib MiB."""
    fetch, write = _pmc_per_dispatch(fetch_csv), _pmc_per_dispatch(write_csv)
    copy_kib = copy_mib * 1024.0
    f_scale, w_scale = copy_kib / _calib_copy(fetch), copy_kib / _calib_copy(write)
    sel = [k for k in fetch if "fwd_bf16_resident_kernel<128, true>" in k[1]]  # the tile-table launches
    read = sum(fetch[k] for k in sel) * f_scale * 1024 / calls
    written = sum(write.get(k, 0.0) for k in sel) * w_scale * 1024 / calls
    tile_bytes = 210 * HQ * D * 2 * 2 + 2 * 210 * HKV * D * 2 + HQ * 210 * 4
    lines = ["# HBM traffic of the small-tile forward: the 13440 x 13440 share in 210 x 210 tiles (counters)", "",
             "Workload: 4096 non-causal tiles of 210 x 210 tokens (32/8 heads, d = 128, bf16), one",
             "mesh_attn_tile_fwd_tabled call: every tile runs the resident-KV kernel in one launch from the",
             "tile table (the bench also times the call through mesh_attn_tile_fwd; those launches are not counted).",
             "Two rocprofv3 runs of the same command, one counter each (KiB per dispatch):", "",
             "    " + command.replace("PMC", "FETCH_SIZE"), "    " + command.replace("PMC", "WRITE_SIZE"), "",
             f"Calibration: the plain device copy of {copy_mib} MiB gives the factors {f_scale:.4f} (fetch) and "
             f"{w_scale:.4f} (write).", "",
             f"Resident-kernel dispatches: {len(sel)} over {calls} calls. Per call: {read / 1e9:.3f} GB read, "
             f"{written / 1e9:.3f} GB written ({(read + written) / 1e9:.3f} GB), against "
             f"{4096 * tile_bytes / 1e9:.3f} GB of compulsory bytes (each tile's Q, K, V read once, O and LSE written "
             "once): tiles that share a Q or KV partition are served from the caches.", "",
             "Traffic that bench.py reports for this workload while the kernel sources are unchanged:", "",
             f"    fwd_p210_bytes_per_call: {int(round(read + written))}",
             f"    source_sha256: {kernel_source_hash()}", ""]
    with open(SMALL_TRAFFIC_FILE, "w") as f:
        f.write("\n".join(lines))
    print(f"wrote {SMALL_TRAFFIC_FILE}: {(read + written) / 1e9:.3f} GB per call")


def summarize_pmc(fetch_csv, write_csv, copy_mib, command):
    """Write the HBM-traffic summary of the headline's tile backward from two rocprofv3 --pmc runs
    (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), each scaled by what the same counter reads for
    the plain device copy of copy_mib MiB made by --calib-copy-mb."""
    import collections

    fetch, write = _pmc_per_dispatch(fetch_csv), _pmc_per_dispatch(write_csv)

    def by_kernel(d):
        agg = collections.OrderedDict()
        for (_, name), v in d.items():
            agg.setdefault(name, []).append(v)
        return agg

    fk, wk = by_kernel(fetch), by_kernel(write)
    mean = lambda xs: sum(xs) / len(xs)
    copy_kib = copy_mib * 1024.0
    # the reference copy is the runtime's device-to-device blit of --calib-copy-mb (torch's elementwise
    # copy kernels of the input set-up are not it)
    copy_name = next(k for k in fk if "copyBuffer" in k)
    f_copy, w_copy = _calib_copy(fetch), _calib_copy(write)
    f_scale, w_scale = copy_kib / f_copy, copy_kib / w_copy
    short = lambda n: n.replace("ma::(anonymous namespace)::", "").replace("void ", "").split("(")[0]
    # one backward call = the consecutive dispatches of the three backward kernels
    calls, cur = [], None
    for (did, name), v in fetch.items():
        if any(t in name for t in BWD_KERNELS):
            if cur is None:
                cur = [0.0, 0.0]
            cur[0] += v * f_scale
            cur[1] += write.get((did, name), 0.0) * w_scale
        elif cur is not None:
            calls.append(cur)
            cur = None
    if cur is not None:
        calls.append(cur)
    per_call = mean([c[0] + c[1] for c in calls]) * 1024
    lines = ["# HBM traffic of the tile backward, Mesh 8x8 share at 1M tokens (counters)", "",
             "Workload: GPU 9 of n = 64 at S = 1,048,576: 8 Q partitions x 8 KV partitions of 16384 tokens,",
             "32/8 heads, head_dim 128, bf16, non-causal; one mesh_attn_tile_bwd call over the 64 pairs",
             "(8 bwd_pre launches, one bwd_dq launch, one bwd_dkv launch).",
             "Two rocprofv3 runs of the same command, one counter each (KiB per dispatch):", "",
             "    " + command.replace("PMC", "FETCH_SIZE"), "    " + command.replace("PMC", "WRITE_SIZE"), "",
             f"Calibration: the plain device copy of {copy_mib} MiB ({short(copy_name)}) reads FETCH_SIZE "
             f"{f_copy:.0f} KiB and WRITE_SIZE {w_copy:.0f} KiB, so the factors are "
             f"{f_scale:.4f} (fetch) and {w_scale:.4f} (write).", "",
             "| Kernel | dispatches | FETCH_SIZE KiB (mean) | WRITE_SIZE KiB (mean) | scaled MiB read | scaled MiB written |",
             "|---|---|---|---|---|---|"]
    for k in fk:
        if k == copy_name or k not in wk:
            continue
        f_, w_ = mean(fk[k]), mean(wk[k])
        lines.append(f"| {short(k)} | {len(fk[k])} | {f_:.0f} | {w_:.0f} | {f_ * f_scale / 1024:.1f} | "
                     f"{w_ * w_scale / 1024:.1f} |")
    lines += ["", f"Backward calls found: {len(calls)}; their mean scaled bytes (read + written) per call is the "
              "traffic that bench.py reports while the kernel sources are unchanged:", "",
              f"    tile_bwd_bytes_per_launch: {int(round(per_call))}",
              f"    source_sha256: {kernel_source_hash()}", ""]
    with open(TRAFFIC_FILE, "w") as f:
        f.write("\n".join(lines))
    print(f"wrote {TRAFFIC_FILE}: {per_call / 2**30:.2f} GiB per call")


# ---------------------------------------------------------- oracle baselines --

def oracle_sample(kind, rows, scale):
    """The fp64 oracle, as it stands, on a bounded sample of one configuration; returns
    (seconds, algorithmic FLOP of the sample, description).  Inputs are the tests' seeded draws."""
    import numpy as np
    import synthetic
    from oracle import attn_tile, attn_tile_bwd, merge

    def bf(wid, t, part, shape):
        return synthetic.normal_bf16(wid, t, part, shape)[1].astype(np.float64)

    if kind == "c4":
        # the headline step on `rows` query rows of the owned Q partition against all 8 KV partitions
        wid, P = 4, MESH_P
        kparts = [MESH_G % MESH_A + MESH_A * t for t in range(MESH_B)]
        kall = np.concatenate([bf(wid, synthetic.T_K, j, (1, P, HKV, D)) for j in kparts], axis=1)
        vall = np.concatenate([bf(wid, synthetic.T_V, j, (1, P, HKV, D)) for j in kparts], axis=1)
        q = bf(wid, synthetic.T_Q, 1000 + MESH_G, (1, rows, HQ, D))
        do = bf(wid, synthetic.T_DO, 1000 + MESH_G, (1, rows, HQ, D))
        mu = np.float32(math.log(MESH_B * P) + 0.5)
        inc = [(bf(wid, synthetic.T_O_IN, 1000 + r, (1, rows, HQ, D)),
                (synthetic.normal_f32(wid, synthetic.T_LSE_IN, 1000 + r, (1, HQ, rows)) + mu).astype(np.float64))
               for r in range(MESH_A - 1)]
        t0 = time.perf_counter()
        O, L = attn_tile(q, kall, vall, scale)
        Om, Lm = merge([(O, L)] + inc)
        attn_tile_bwd(q, kall, vall, Om, do, Lm, scale)
        dt = time.perf_counter() - t0
        nk = kall.shape[1]
        return dt, 14.0 * D * HQ * rows * nk, (f"{rows} query rows x {HQ} heads of the owned Q partition against "
                                                f"all {nk} keys: forward, 15-way merge, backward")
    if kind == "c1":
        wid, S, n, d = 1, 256, 4, 64
        P = S // n
        q = synthetic.normal_f32(wid, synthetic.T_Q, 0, (1, S, 1, d)).astype(np.float64)
        k = synthetic.normal_f32(wid, synthetic.T_K, 0, (1, S, 1, d)).astype(np.float64)
        v = synthetic.normal_f32(wid, synthetic.T_V, 0, (1, S, 1, d)).astype(np.float64)
        s1 = np.float32(1.0 / math.sqrt(d))
        t0 = time.perf_counter()
        for i in range(n):
            parts = [attn_tile(q[:, i * P:(i + 1) * P], k[:, j * P:(j + 1) * P], v[:, j * P:(j + 1) * P], s1)
                     for j in range(n)]
            merge(parts)
        dt = time.perf_counter() - t0
        return dt, 4.0 * d * S * S, "the whole configuration: 16 tiles and 4 merges"
    if kind == "c2":
        wid, S = 2, 8192
        q = bf(wid, synthetic.T_Q, 0, (1, S, HQ, D))[:, :rows]
        k = bf(wid, synthetic.T_K, 0, (1, S, HKV, D))
        v = bf(wid, synthetic.T_V, 0, (1, S, HKV, D))
        t0 = time.perf_counter()
        attn_tile(q, k, v, scale)
        dt = time.perf_counter() - t0
        return dt, 4.0 * D * HQ * rows * S, f"{rows} of {S} query rows x {HQ} heads against all {S} keys (forward)"
    if kind == "c3":
        wid, C = 3, 4096
        c = 26  # the chunk with 27 KV chunks
        nk = (c + 1) * C
        k = np.concatenate([bf(wid, synthetic.T_K, j, (1, C, HKV, D)) for j in range(c + 1)], axis=1)
        v = np.concatenate([bf(wid, synthetic.T_V, j, (1, C, HKV, D)) for j in range(c + 1)], axis=1)
        q = bf(wid, synthetic.T_Q, c, (1, C, HQ, D))[:, :rows]
        qpos = c * C + np.arange(rows)
        t0 = time.perf_counter()
        attn_tile(q, k, v, scale, None, True, qpos, np.arange(nk))
        dt = time.perf_counter() - t0
        allowed = int(np.sum(qpos + 1))
        return dt, 4.0 * D * HQ * allowed, (f"{rows} of {C} query rows x {HQ} heads of chunk 26 against its "
                                            f"{nk} causal keys (forward)")
    if kind == "c5":
        wid, S = 5, 8192
        k = bf(wid, synthetic.T_K, 0, (1, S, HKV, D))
        v = bf(wid, synthetic.T_V, 0, (1, S, HKV, D))
        q = bf(wid, synthetic.T_Q, 0, (1, S, HQ, D))[:, :rows]
        do = bf(wid, synthetic.T_DO, 0, (1, S, HQ, D))[:, :rows]
        O, L = attn_tile(q, k, v, scale)
        t0 = time.perf_counter()
        attn_tile_bwd(q, k, v, O, do, L, scale)
        dt = time.perf_counter() - t0
        return dt, 10.0 * D * HQ * rows * S, (f"{rows} query rows x {HQ} heads of one Q partition against all {S} "
                                              f"keys (backward: dQ rows and their dK/dV contributions)")
    raise ValueError(kind)


def cpu_baseline(kind, rows, scale):
    dt, flop, what = oracle_sample(kind, rows, scale)
    model, nproc = cpu_info()
    return {"value": round(flop / dt / 1e12, 5), "unit": "TFLOP/s", "cores": int(blas_threads()), "kind": "oracle",
            "sample": f"{what}; float64 NumPy, {dt:.1f} s", "cpu": model, "host_cores_visible": nproc,
            "seconds": round(dt, 2)}


# -------------------------------------------------------------- the headline --

def mesh_share_inputs(gen, dev):
    """Device-resident inputs of the Mesh 8x8 share: Q of the 8 Q partitions, the 8 KV partitions in
    one gathered buffer (K[j], V[j] are views into it), N(0,1) from the seeded device generator."""
    import torch
    import distributed_long_context_amd as ma
    P = MESH_P
    qparts, kparts = ma.mesh_attn_map_mesh_tile(MESH_N, MESH_A, MESH_B, MESH_G, True)

    def randn(shape):
        return torch.randn(shape, generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)

    Q = {i: randn((1, P, HQ, D)) for i in qparts}
    kg = randn((1, MESH_B * P, HKV, D))
    vg = randn((1, MESH_B * P, HKV, D))
    K = {j: kg[:, t * P:(t + 1) * P] for t, j in enumerate(kparts)}
    V = {j: vg[:, t * P:(t + 1) * P] for t, j in enumerate(kparts)}
    return qparts, kparts, Q, kg, vg, K, V


def headline(args, dev, scale):
    import torch
    import distributed_long_context_amd as ma
    from distributed_long_context_amd import BwdTile, Tile

    gen = torch.Generator(device=dev)
    gen.manual_seed(4)
    P = MESH_P
    qparts, kparts, Q, kg, vg, K, V = mesh_share_inputs(gen, dev)
    mu = math.log(MESH_B * P) + 0.5
    # 7 incoming partials for the owned partition (O ~ N(0,1) in bf16, LSE = mu + N(0,1))
    inc = [(torch.randn((1, P, HQ, D), generator=gen, device=dev).to(torch.bfloat16),
            torch.randn((1, HQ, P), generator=gen, device=dev) + mu) for _ in range(MESH_A - 1)]
    dO = {i: torch.randn((1, P, HQ, D), generator=gen, device=dev).to(torch.bfloat16) for i in qparts}
    part_o = {(i, j): torch.empty((1, P, HQ, D), dtype=torch.bfloat16, device=dev) for i in qparts for j in kparts}
    part_l = {(i, j): torch.empty((1, HQ, P), dtype=torch.float32, device=dev) for i in qparts for j in kparts}
    mo = {i: torch.empty((1, P, HQ, D), dtype=torch.bfloat16, device=dev) for i in qparts}
    ml = {i: torch.empty((1, HQ, P), dtype=torch.float32, device=dev) for i in qparts}
    dq = {i: torch.empty((1, P, HQ, D), dtype=torch.float32, device=dev) for i in qparts}
    dk = {j: torch.empty((1, P, HKV, D), dtype=torch.float32, device=dev) for j in kparts}
    dv = {j: torch.empty_like(dk[j]) for j in kparts}
    ftiles = [Tile(Q[i], K[j], V[j], part_o[(i, j)], part_l[(i, j)]) for i in qparts for j in kparts]
    btiles = [BwdTile(Q[i], K[j], V[j], mo[i], dO[i], ml[i], dq[i], dk[j], dv[j]) for i in qparts for j in kparts]
    ws = torch.empty(max(256, ma.mesh_attn_tile_bwd_workspace_size(btiles, scale, ma.MA_MASK_NONE)), dtype=torch.uint8,
                     device=dev)
    merge_lists = []
    for i in qparts:
        os_ = [part_o[(i, j)] for j in kparts]
        ls_ = [part_l[(i, j)] for j in kparts]
        if i == MESH_G:
            os_ += [x[0] for x in inc]
            ls_ += [x[1] for x in inc]
        merge_lists.append((os_, ls_, mo[i], ml[i]))
    pos0 = ma.mesh_attn_pos_contiguous(0)
    pairs = MESH_A * MESH_B * P * P
    fwd_flop = 4.0 * D * HQ * pairs
    bwd_flop = 10.0 * D * HQ * pairs
    part_bytes = P * HQ * D * 2 + HQ * P * 4
    merge_bytes = sum((len(x[0]) + 1) * part_bytes for x in merge_lists)
    stream = torch.cuda.current_stream()
    evs, host_ms = [], []

    def step(record):
        h0 = time.perf_counter()
        # (1) host mapping: this GPU's partitions, groups and pair work list
        qp_, kp_ = ma.mesh_attn_map_mesh_tile(MESH_N, MESH_A, MESH_B, MESH_G, True)
        ma.mesh_attn_map_groups(MESH_N, MESH_A, MESH_B, MESH_G)
        wl = ma.mesh_attn_build_worklist([pos0] * MESH_A, [P] * MESH_A, [pos0] * MESH_B, [P] * MESH_B,
                                         ma.MA_MASK_NONE)
        assert qp_ == qparts and kp_ == kparts and len(wl) == MESH_A * MESH_B
        if record:
            host_ms.append((time.perf_counter() - h0) * 1e3)
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)] if record else None
        if record:
            e[0].record(stream)
        ma.mesh_attn_tile_fwd(ftiles, scale, ma.MA_MASK_NONE)                 # (2)
        if record:
            e[1].record(stream)
        for os_, ls_, o, l in merge_lists:                                    # (3)
            ma.mesh_attn_merge(os_, ls_, o, l)
        if record:
            e[2].record(stream)
        ma.mesh_attn_tile_bwd(btiles, scale, ma.MA_MASK_NONE, workspace=ws)  # (4)
        if record:
            e[3].record(stream)
            evs.append(e)

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps

    def part_ms(i):
        ts = [e[i].elapsed_time(e[i + 1]) for e in evs]
        return _median(ts), sum(ts) / len(ts)

    (fm, fa), (mm, mma), (bm, ba) = part_ms(0), part_ms(1), part_ms(2)
    parts = {"map_host": {"ms": round(_median(host_ms), 4), "note": "mapper + work list, host C++ through the C ABI"},
             "tile_fwd": tf(fwd_flop, fa, reps=args.steps), "merge": gb(merge_bytes, mma, reps=args.steps),
             "tile_bwd": tf(bwd_flop, ba, reps=args.steps)}
    parts["tile_fwd"].update({"ms_median": round(fm, 4), "launches": "64 tiles in one call (3 launches of the "
                                                                      "30-tile table)"})
    parts["merge"].update({"ms_median": round(mm, 4), "calls": "7 x 8-way + 1 x 15-way"})
    parts["tile_bwd"].update({"ms_median": round(bm, 4), "includes": "8 x bwd_pre (D = rowsum(dO*O)), bwd_dq, bwd_dkv"})
    value = (fwd_flop + bwd_flop) / (ms_step * 1e-3) / 1e12
    # dominant part by time: the tile backward; its rate is the events' mean over the timed steps
    rl = roofline_mfma(parts["tile_bwd"], "tile_bwd: one mesh_attn_tile_bwd call over the 64 pairs "
                                          "(8 bwd_pre + bwd_dq + bwd_dkv launches)", stored_traffic())
    rl.update(flop_per_launch=bwd_flop, ms_per_launch=round(ba, 4))
    power = None
    if args.power_sample > 0:
        power = power_clock([("tile_fwd", lambda: ma.mesh_attn_tile_fwd(ftiles, scale, ma.MA_MASK_NONE)),
                             ("tile_bwd", lambda: ma.mesh_attn_tile_bwd(btiles, scale, ma.MA_MASK_NONE, workspace=ws))],
                            args.power_sample)
        for name in ("tile_fwd", "tile_bwd"):
            pw = power.get(name, {})
            if "gfx_mhz_median" in pw:
                pk = PEAK_BF16_TFLOPS * pw["gfx_mhz_median"] / 2400.0
                pw["bf16_peak_at_held_clock_tflops"] = round(pk, 1)
                pw["frac_of_peak_at_held_clock"] = round(parts[name]["TFLOP/s"] / pk, 4)
    return value, ms_step, parts, rl, power


# --------------------------------------------------------------- per config --

def config_c1(args, dev):
    """fp32, 1 head, d = 64, S = 256 in 4 partitions of 64: all 16 tiles in one call, then four
    4-way merges (launch-bound; the fp32 forward is bound by fp32 VALU arithmetic)."""
    import torch
    import distributed_long_context_amd as ma
    from distributed_long_context_amd import Tile
    gen = torch.Generator(device=dev)
    gen.manual_seed(1)
    S, n, d = 256, 4, 64
    P = S // n
    q, k, v = (torch.randn((1, S, 1, d), generator=gen, device=dev) for _ in range(3))
    outs = [(torch.empty((1, P, 1, d), device=dev), torch.empty((1, 1, P), device=dev)) for _ in range(n * n)]
    t16 = [Tile(q[:, i * P:(i + 1) * P], k[:, j * P:(j + 1) * P], v[:, j * P:(j + 1) * P], *outs[i * n + j])
           for i in range(n) for j in range(n)]
    mo = [(torch.empty((1, P, 1, d), device=dev), torch.empty((1, 1, P), device=dev)) for _ in range(n)]
    s1 = float(1.0 / math.sqrt(d))

    def merges():
        for i in range(n):
            row = outs[i * n:(i + 1) * n]
            ma.mesh_attn_merge([x[0] for x in row], [x[1] for x in row], mo[i][0], mo[i][1])

    flop = 4.0 * d * S * S
    r = {"workload": "fp32, 1 head, d=64, S=256 in 4 partitions: 16 tiles (one call) + 4 x 4-way merges"}
    reps = reps_of(100, args)
    fwd = timed(lambda: ma.mesh_attn_tile_fwd(t16, s1, ma.MA_MASK_NONE), reps, 20)
    r["tile_fwd"] = {"ms": round(fwd[0], 4), "ms_mean": round(fwd[1], 4), "reps": reps, "flop": flop,
                     "TFLOP/s": round(flop / (fwd[0] * 1e-3) / 1e12, 4)}
    mg = timed(merges, reps, 20)
    r["merges"] = gb(n * (n + 1) * (P * d * 4 + P * 4), mg[0], mg[1], reps)
    r["roofline"] = {"bound": "alu", "achieved": r["tile_fwd"]["TFLOP/s"], "peak": PEAK_F32_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(r["tile_fwd"]["TFLOP/s"] / PEAK_F32_TFLOPS, 6), "traffic": None,
                     "kernel": "fwd_f32_kernel (16 tiles of 64 x 64: launch-bound, a correctness configuration)"}
    return r


def config_c2(args, dev, scale):
    import torch
    import distributed_long_context_amd as ma
    from distributed_long_context_amd import Tile
    gen = torch.Generator(device=dev)
    gen.manual_seed(2)
    S = 8192
    q = torch.randn((1, S, HQ, D), generator=gen, device=dev).to(torch.bfloat16)
    k, v = (torch.randn((1, S, HKV, D), generator=gen, device=dev).to(torch.bfloat16) for _ in range(2))
    o = torch.empty((1, S, HQ, D), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((1, HQ, S), dtype=torch.float32, device=dev)
    t = [Tile(q, k, v, o, lse)]
    r = {"workload": "one non-causal tile, Q 8192 x KV 8192, 32/8 heads, d=128, bf16"}
    r["tile_fwd"] = timed_tf(4.0 * D * HQ * S * S, lambda: ma.mesh_attn_tile_fwd(t, scale, ma.MA_MASK_NONE),
                             reps_of(100, args), 20)
    r["roofline"] = roofline_mfma(r["tile_fwd"], "fwd_bf16_kernel<128, false, 8> (one launch)")
    return r


def config_c3(args, dev, scale):
    import torch
    import distributed_long_context_amd as ma
    from distributed_long_context_amd import BwdTile, Tile
    gen = torch.Generator(device=dev)
    gen.manual_seed(3)
    N, rk, C = 16, 5, 4096
    qchunks = ma.mesh_attn_map_zigzag(N, rk)
    nkv = max(qchunks) + 1

    def randn(shape, dtype=torch.bfloat16, mul=1.0, add=0.0):
        return (torch.randn(shape, generator=gen, device=dev) * mul + add).to(dtype)

    def out(sq):
        return (torch.empty((1, sq, HQ, D), dtype=torch.bfloat16, device=dev),
                torch.empty((1, HQ, sq), dtype=torch.float32, device=dev))

    Q = {c: randn((1, C, HQ, D)) for c in qchunks}
    kg, vg = randn((1, nkv * C, HKV, D)), randn((1, nkv * C, HKV, D))
    K = [kg[:, j * C:(j + 1) * C] for j in range(nkv)]
    V = [vg[:, j * C:(j + 1) * C] for j in range(nkv)]
    qpos = [ma.mesh_attn_pos_contiguous(c * C) for c in qchunks]
    kpos = [ma.mesh_attn_pos_contiguous(j * C) for j in range(nkv)]
    wl = ma.mesh_attn_build_worklist(qpos, [C, C], kpos, [C] * nkv, ma.MA_MASK_CAUSAL)
    pairs = sum(ma.mesh_attn_count_allowed(qpos[i], C, kpos[j], C, ma.MA_MASK_CAUSAL) for i, j, _ in wl)
    tiles = [Tile(Q[qchunks[i]], K[j], V[j], *out(C), qpos[i], kpos[j]) for i, j, _ in wl]
    groups = [[t for t, (ii, _, _) in zip(tiles, wl) if ii == i] for i in range(2)]
    merged = [out(C) for _ in qchunks]
    fused = [out(C) for _ in qchunks]
    ftiles = [Tile(Q[c], kg[:, :(c + 1) * C], vg[:, :(c + 1) * C], *fused[i], qpos[i], ma.mesh_attn_pos_contiguous(0))
              for i, c in enumerate(qchunks)]
    part_bytes = C * HQ * D * 2 + HQ * C * 4
    merge_bytes = sum((len(g) + 1) * part_bytes for g in groups)

    def merges():
        for g, m in zip(groups, merged):
            ma.mesh_attn_merge([t.o for t in g], [t.lse for t in g], m[0], m[1])

    fwd_flop = 4.0 * D * HQ * pairs
    r = {"workload": "causal zigzag share of S=131072 in 32 chunks of 4096, rank 5 of 16 (chunks 5 and 26): "
                     "33 tiles (31 FULL, 2 diagonal PARTIAL, 31 EMPTY skipped), then 6-way and 27-way merges",
         "tiles": len(wl), "allowed_pairs_per_head": pairs}
    r["tile_fwd"] = timed_tf(fwd_flop, lambda: ma.mesh_attn_tile_fwd(tiles, scale, ma.MA_MASK_CAUSAL),
                             reps_of(30, args), 5)
    scratch = torch.empty(1 << 29, dtype=torch.uint8, device=dev)
    ts = []
    for it in range(reps_of(20, args) + 1):
        mall_flush(scratch, it)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        merges()
        e1.record()
        e1.synchronize()
        ts.append(e0.elapsed_time(e1))
    del scratch
    r["merge_6_and_27"] = gb(merge_bytes, _median(ts[1:]), sum(ts[1:]) / len(ts[1:]), len(ts) - 1)
    r["merge_6_and_27"]["note"] = "MALL flushed before each rep"
    r["tile_fwd_fused_gathered_kv"] = timed_tf(fwd_flop, lambda: ma.mesh_attn_tile_fwd(ftiles, scale, ma.MA_MASK_CAUSAL),
                                               reps_of(30, args), 5)
    # backward of the share: dQ of both chunks, partial dK/dV of KV chunks 0..26
    dO = {c: randn((1, C, HQ, D)) for c in qchunks}
    O = {c: randn((1, C, HQ, D), mul=math.sqrt(math.e / (c * C + C / 2))) for c in qchunks}
    L = {c: randn((1, HQ, C), torch.float32, 0.3, math.log(c * C + C / 2) + 0.5) for c in qchunks}
    dq = {c: torch.empty((1, C, HQ, D), dtype=torch.float32, device=dev) for c in qchunks}
    dk = [torch.empty((1, C, HKV, D), dtype=torch.float32, device=dev) for _ in range(nkv)]
    dv = [torch.empty_like(x) for x in dk]
    btiles = [BwdTile(Q[qchunks[i]], K[j], V[j], O[qchunks[i]], dO[qchunks[i]], L[qchunks[i]], dq[qchunks[i]],
                      dk[j], dv[j], qpos[i], kpos[j]) for i, j, _ in wl]
    ws = torch.empty(max(256, ma.mesh_attn_tile_bwd_workspace_size(btiles, scale, ma.MA_MASK_CAUSAL)), dtype=torch.uint8,
                     device=dev)
    r["tile_bwd"] = timed_tf(10.0 * D * HQ * pairs,
                             lambda: ma.mesh_attn_tile_bwd(btiles, scale, ma.MA_MASK_CAUSAL, workspace=ws),
                             reps_of(20, args), 3)
    r["roofline"] = roofline_mfma(r["tile_fwd"], "tile_fwd: one mesh_attn_tile_fwd call over the 33 tiles "
                                                 "(fwd_bf16_kernel masked and unmasked launches)")
    return r


def config_c4(args, dev, scale):
    """The Mesh share's other entries: the fused forward over the gathered KV buffer, the merges
    with the MALL flushed, the GOO replay and the gradient add-reduce."""
    import torch
    import distributed_long_context_amd as ma
    from distributed_long_context_amd import Tile
    gen = torch.Generator(device=dev)
    gen.manual_seed(40)
    P = MESH_P
    qparts, kparts, Q, kg, vg, K, V = mesh_share_inputs(gen, dev)

    def out(sq):
        return (torch.empty((1, sq, HQ, D), dtype=torch.bfloat16, device=dev),
                torch.empty((1, HQ, sq), dtype=torch.float32, device=dev))

    pairs = MESH_A * MESH_B * P * P
    flop = 4.0 * D * HQ * pairs
    mu = math.log(MESH_B * P) + 0.5
    inc = [(torch.randn((1, P, HQ, D), generator=gen, device=dev).to(torch.bfloat16),
            torch.randn((1, HQ, P), generator=gen, device=dev) + mu) for _ in range(MESH_A - 1)]
    r = {"workload": "Mesh 8x8 share of GPU 9 of n=64 at S=1,048,576 (16384-token partitions), non-causal"}
    fused = {i: out(P) for i in qparts}
    ftiles = [Tile(Q[i], kg, vg, *fused[i]) for i in qparts]

    def fused_step():
        ma.mesh_attn_tile_fwd(ftiles, scale, ma.MA_MASK_NONE)
        ma.mesh_attn_merge([fused[MESH_G][0]] + [x[0] for x in inc], [fused[MESH_G][1]] + [x[1] for x in inc],
                           fused[MESH_G][0], fused[MESH_G][1])

    r["fwd_fused_gathered_kv_plus_owned_merge"] = timed_tf(flop, fused_step, reps_of(5, args), 1)
    tiles = {(i, j): Tile(Q[i], K[j], V[j], *out(P)) for i in qparts for j in kparts}
    ma.mesh_attn_tile_fwd(list(tiles.values()), scale, ma.MA_MASK_NONE)
    merged = {i: out(P) for i in qparts}
    part_bytes = P * HQ * D * 2 + HQ * P * 4

    def merges():
        for i in qparts:
            os_ = [tiles[(i, j)].o for j in kparts]
            ls_ = [tiles[(i, j)].lse for j in kparts]
            if i == MESH_G:
                os_ += [x[0] for x in inc]
                ls_ += [x[1] for x in inc]
            ma.mesh_attn_merge(os_, ls_, merged[i][0], merged[i][1])

    r["merge_7x8_and_15"] = timed_gb((7 * 9 + 16) * part_bytes, merges, reps_of(10, args), 2)
    r["merge_7x8_and_15"]["note"] = "10.8 GB per rep, far beyond the 256 MB MALL"
    del tiles, merged, fused, ftiles
    torch.cuda.empty_cache()
    # GOO replay: k_Q = k_KV = 4 chunks per partition; C-i-j in the greedy plan's order, each folded into
    # its Q chunk's (O, LSE) with the forward's accumulate mode
    kq = kkv = 4
    cq, ck = P // kq, P // kkv
    gq = [torch.cat([Q[i][:, c * cq:(c + 1) * cq] for i in qparts], dim=1) for c in range(kq)]
    gk = [torch.cat([K[j][:, c * ck:(c + 1) * ck] for j in kparts], dim=1) for c in range(kkv)]
    gv = [torch.cat([V[j][:, c * ck:(c + 1) * ck] for j in kparts], dim=1) for c in range(kkv)]
    acc = [out(MESH_A * cq) for _ in range(kq)]
    plan = ma.mesh_attn_goo_plan(kq, kkv, 0.5, 1.0, 0.5, 0.5, 1.0)
    order = [(i, j) for _, comp in plan for _, i, j in comp]

    def goo_replay():
        first = set()
        for i, j in order:
            ma.mesh_attn_tile_fwd([Tile(gq[i], gk[j], gv[j], acc[i][0], acc[i][1])], scale, ma.MA_MASK_NONE,
                                  accumulate=i in first)
            first.add(i)

    r["fwd_goo_replay_4x4"] = timed_tf(flop, goo_replay, reps_of(5, args), 1)
    r["fwd_goo_replay_4x4"]["tasks"] = len(order)
    del gq, gk, gv, acc
    # the addition of the gradient reduce-scatter: 8 partial dQ of one Q partition (fp32, 256 MiB each)
    parts = [torch.randn((1, P, HQ, D), generator=gen, device=dev) for _ in range(8)]
    red = torch.empty_like(parts[0])
    r["reduce_add_8_dq"] = timed_gb(9 * parts[0].numel() * 4, lambda: ma.mesh_attn_reduce_add(parts, red),
                                    reps_of(20, args), 3)
    r["roofline"] = "the headline step's (top-level roofline)"
    return r


def config_c5(args, dev, scale):
    import torch
    import distributed_long_context_amd as ma
    from distributed_long_context_amd import BwdTile
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)
    S, nq = 8192, 4

    def randn(shape, dtype=torch.bfloat16, mul=1.0, add=0.0):
        return (torch.randn(shape, generator=gen, device=dev) * mul + add).to(dtype)

    k, v = randn((1, S, HKV, D)), randn((1, S, HKV, D))
    dk = torch.empty((1, S, HKV, D), dtype=torch.float32, device=dev)
    dv = torch.empty_like(dk)
    btiles = [BwdTile(randn((1, S, HQ, D)), k, v, randn((1, S, HQ, D), mul=math.sqrt(math.e / S)), randn((1, S, HQ, D)),
                      randn((1, HQ, S), torch.float32, 0.3, math.log(S) + 0.5),
                      torch.empty((1, S, HQ, D), dtype=torch.float32, device=dev), dk, dv) for _ in range(nq)]
    ws = torch.empty(max(256, ma.mesh_attn_tile_bwd_workspace_size(btiles, scale, ma.MA_MASK_NONE)), dtype=torch.uint8,
                     device=dev)
    r = {"workload": "backward of 4 Q partitions of 8192 x one KV partition of 8192, 32/8 heads, d=128, bf16"}
    r["tile_bwd"] = timed_tf(10.0 * D * HQ * nq * S * S,
                             lambda: ma.mesh_attn_tile_bwd(btiles, scale, ma.MA_MASK_NONE, workspace=ws),
                             reps_of(20, args), 3)
    r["tile_bwd"]["includes"] = "4 x bwd_pre, bwd_dq, bwd_dkv"
    r["roofline"] = roofline_mfma(r["tile_bwd"], "tile_bwd: one mesh_attn_tile_bwd call (4 bwd_pre + bwd_dq + bwd_dkv)")
    return r


def config_striped(args, dev, scale):
    import torch
    import distributed_long_context_amd as ma
    from distributed_long_context_amd import BwdTile, Tile
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    P = MESH_P
    qparts, kparts, Q, kg, vg, K, V = mesh_share_inputs(gen, dev)
    qpos = {i: ma.mesh_attn_pos_striped(MESH_N, i) for i in qparts}
    kpos = {j: ma.mesh_attn_pos_striped(MESH_N, j) for j in kparts}
    mode = ma.MA_MASK_STRIPED_ZIGZAG
    pairs = sum(ma.mesh_attn_count_allowed(qpos[i], P, kpos[j], P, mode) for i in qparts for j in kparts)
    outs = [(torch.empty((1, P, HQ, D), dtype=torch.bfloat16, device=dev),
             torch.empty((1, HQ, P), dtype=torch.float32, device=dev)) for _ in range(MESH_A * MESH_B)]
    tiles = [Tile(Q[i], K[j], V[j], *outs[x * MESH_B + y], qpos[i], kpos[j])
             for x, i in enumerate(qparts) for y, j in enumerate(kparts)]
    r = {"workload": "the Mesh 8x8 share under the causal mask with striped positions (partition p holds "
                     "p + 64 t; every pair PARTIAL)", "allowed_pairs_per_head": pairs}
    r["tile_fwd"] = timed_tf(4.0 * D * HQ * pairs, lambda: ma.mesh_attn_tile_fwd(tiles, scale, mode), reps_of(5, args), 1)
    del tiles, outs
    torch.cuda.empty_cache()
    dO = {i: torch.randn((1, P, HQ, D), generator=gen, device=dev).to(torch.bfloat16) for i in qparts}
    O = {i: (torch.randn((1, P, HQ, D), generator=gen, device=dev) * math.sqrt(2 * math.e / (MESH_B * P))).to(
        torch.bfloat16) for i in qparts}
    L = {i: torch.randn((1, HQ, P), generator=gen, device=dev) * 0.3 + (math.log(MESH_B * P / 2) + 0.5) for i in qparts}
    dq = {i: torch.empty((1, P, HQ, D), dtype=torch.float32, device=dev) for i in qparts}
    dk = {j: torch.empty((1, P, HKV, D), dtype=torch.float32, device=dev) for j in kparts}
    dv = {j: torch.empty_like(dk[j]) for j in kparts}
    btiles = [BwdTile(Q[i], K[j], V[j], O[i], dO[i], L[i], dq[i], dk[j], dv[j], qpos[i], kpos[j])
              for i in qparts for j in kparts]
    ws = torch.empty(max(256, ma.mesh_attn_tile_bwd_workspace_size(btiles, scale, mode)), dtype=torch.uint8, device=dev)
    r["tile_bwd"] = timed_tf(10.0 * D * HQ * pairs, lambda: ma.mesh_attn_tile_bwd(btiles, scale, mode, workspace=ws),
                             reps_of(3, args), 1)
    r["roofline"] = roofline_mfma(r["tile_bwd"], "tile_bwd: one mesh_attn_tile_bwd call over the 64 masked pairs")
    return r


def config_small(args, dev, scale):
    """A 13440 x 13440 share (32/8 heads, d = 128, non-causal) cut into (13440/P)^2 tiles of P x P
    tokens, all in one forward call (mesh_attn_tile_fwd_tabled: the resident-KV tiles from a tile
    table in device memory), for the partition sizes of [CHARM+]'s scaling table.  Compulsory bytes
    per tile = Q, K, V read once + O, LSE written once."""
    import torch
    import distributed_long_context_amd as ma
    from distributed_long_context_amd import Tile
    gen = torch.Generator(device=dev)
    gen.manual_seed(6)
    S = 13440
    q = torch.randn((1, S, HQ, D), generator=gen, device=dev).to(torch.bfloat16)
    k, v = (torch.randn((1, S, HKV, D), generator=gen, device=dev).to(torch.bfloat16) for _ in range(2))
    o_all = torch.empty((S // 210) * S * HQ * D, dtype=torch.bfloat16, device=dev)
    l_all = torch.empty((S // 210) * HQ * S, dtype=torch.float32, device=dev)
    r = {"workload": "13440 x 13440 share cut into P x P tiles, one forward call"}
    for P in (13440, 3360, 840, 210):
        n = S // P
        tiles = []
        for i in range(n):
            for j in range(n):
                part = i * n + j
                o = o_all[part * P * HQ * D:(part + 1) * P * HQ * D].view(1, P, HQ, D)
                lse = l_all[part * HQ * P:(part + 1) * HQ * P].view(1, HQ, P)
                tiles.append(Tile(q[:, i * P:(i + 1) * P], k[:, j * P:(j + 1) * P], v[:, j * P:(j + 1) * P], o, lse))
        flop = 4.0 * D * HQ * S * S
        # argument packing (and the tile table's upload) outside the timing
        prep = ma.prepare_tile_fwd(tiles, scale, ma.MA_MASK_NONE, table=True)
        e = timed_tf(flop, lambda: ma.launch_prepared_tile_fwd(prep), reps_of(20, args), 3)
        if P == 210:  # the same call through mesh_attn_tile_fwd (tiles in kernel arguments, 30 a launch)
            prep_ka = ma.prepare_tile_fwd(tiles, scale, ma.MA_MASK_NONE)
            r["fwd_P210_kernel_arguments"] = timed_tf(flop, lambda: ma.launch_prepared_tile_fwd(prep_ka),
                                                      reps_of(20, args), 3)
        tile_bytes = P * HQ * D * 2 * 2 + 2 * P * HKV * D * 2 + HQ * P * 4
        g = n * n * tile_bytes / (e["ms"] * 1e-3) / 1e9
        e.update({"tiles": n * n, "compulsory_bytes": n * n * tile_bytes, "hbm_GB/s_of_compulsory_bytes": round(g, 1),
                  "frac_hbm_peak": round(g / PEAK_HBM_GBPS, 4),
                  "flop_per_compulsory_byte": round(flop / (n * n * tile_bytes), 1)})
        r[f"fwd_P{P}"] = e
    small = r["fwd_P210"]
    r["roofline"] = {"bound": "hbm", "achieved": small["hbm_GB/s_of_compulsory_bytes"], "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": small["frac_hbm_peak"],
                     "traffic": stored_traffic(SMALL_TRAFFIC_FILE, "fwd_p210_bytes_per_call"),
                     "kernel": "the forward at P = 210 (4096 tiles, one mesh_attn_tile_fwd_tabled call: one "
                               "resident-KV launch; 168 FLOP per compulsory byte, below the chip's balance of about "
                               "315)"}
    return r


# --------------------------------------------------------------------- main --

def main():
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-pmc-small":
        # bench.py --summarize-pmc-small FETCH_CSV WRITE_CSV COPY_MIB CALLS "COMMAND (with PMC for the counter)"
        summarize_pmc_small(sys.argv[2], sys.argv[3], int(sys.argv[4]), int(sys.argv[5]), sys.argv[6])
        return
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-pmc":
        # bench.py --summarize-pmc FETCH_CSV WRITE_CSV COPY_MIB "COMMAND (with PMC for the counter)"
        summarize_pmc(sys.argv[2], sys.argv[3], int(sys.argv[4]), sys.argv[5])
        return
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's share on one MI355X; --gpus above 1 is not supported "
              "(the path runs on a single GPU, with no collectives).", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    import distributed_long_context_amd as ma

    ma.lib()  # fails loudly without the HIP library
    dev = "cuda:0"
    torch.cuda.set_device(0)
    scale = float(np.float32(1.0 / math.sqrt(D)))
    out = {"metric": METRIC, "value": None, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": None, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic: N(0,1) inputs from seeded device generators; incoming partials and dO seeded",
           "config": {"workload": "mesh-8x8-1m-g9: Mesh-Attention share of GPU 9 of n=64 at S=1,048,576 "
                                  "(8 Q x 8 KV partitions of 16384 tokens, KV rotation), non-causal, 32/8 heads, "
                                  "d=128, bf16; step = host mapping + tile forward (64 tiles) + LSE merges "
                                  "(7 x 8-way, 1 x 15-way with 7 incoming) + tile backward (64 pairs)",
                      "batch": 1, "seq_len": MESH_N * MESH_P, "partition_tokens": MESH_P, "q_partitions": MESH_A,
                      "kv_partitions": MESH_B, "q_heads": HQ, "kv_heads": HKV, "head_dim": D, "mask": "none"}}
    if not args.no_step:
        value, ms_step, parts, rl, power = headline(args, dev, scale)
        out.update(value=round(value, 2), ms_per_step=round(ms_step, 4), roofline=rl, parts=parts)
        if power is not None:
            out["power_clock"] = power
        torch.cuda.empty_cache()
        if not args.no_cpu_baseline:
            out["cpu_baseline"] = cpu_baseline("c4", args.cpu_rows, np.float32(scale))
    names = [c for c in args.configs.split(",") if c and c != "none"]
    runners = {"c1": lambda: config_c1(args, dev), "c2": lambda: config_c2(args, dev, scale),
               "c3": lambda: config_c3(args, dev, scale), "c4": lambda: config_c4(args, dev, scale),
               "c5": lambda: config_c5(args, dev, scale), "striped": lambda: config_striped(args, dev, scale),
               "small": lambda: config_small(args, dev, scale)}
    oracle_rows = {"c1": 0, "c2": 512, "c3": 64, "c5": 256}
    blocks = {}
    for name in names:
        blocks[name] = runners[name]()
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        if not args.no_cpu_baseline and name in oracle_rows:
            blocks[name]["cpu_baseline"] = cpu_baseline(name, oracle_rows[name], np.float32(scale))
    if blocks:
        out["configs"] = blocks
    if args.calib_copy_mb > 0:
        # a plain device copy of known size, the reference for the HBM byte counters
        n = args.calib_copy_mb * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
