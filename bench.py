"""Bench of one GPU's share: tile forward + LSE merge + tile backward on MI355X.

One step is one pass of the whole hot path over one batch of synthetic input,
at the single-tile GQA shape (Q partition 8192 x KV partition 8192 tokens,
32 query / 8 KV heads, head_dim 128, bf16, non-causal):

  1. host mapping and tile classification (C++ mapper through the C ABI);
  2. mesh_attn_tile_fwd  -> partial O (bf16) and LSE (fp32);
  3. mesh_attn_merge     -> folds the partial with one incoming seeded partial
                            (the rest of the row's KV, as another GPU would send);
  4. mesh_attn_tile_bwd  -> dQ, dK, dV (fp32) from the merged O and LSE and a
                            seeded dO (this KV partition's share of the gradient).

Prints ONE JSON line.  `value` is the whole step's algorithmic tile FLOPs per
second (forward 4*d*Hq and backward 10*d*Hq per allowed pair), inputs already
resident in HBM.  Per-kernel times come from events recorded on the stream the
kernels are launched on (torch's current stream, which the binding passes).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "tile fwd/bwd TFLOP/s + % bf16 MFMA peak; merge GB/s + % HBM peak (1 GPU)"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E

SQ = SK = 8192
HQ, HKV, D = 32, 8, 128
WORKLOAD_ID = 2


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=4096, help="query rows in the oracle sample")
    ap.add_argument("--parts", default="fwd,merge,bwd", help="kernels in the step (all by default)")
    ap.add_argument("--workloads", default="fp32,zigzag,mesh,striped,small,bwd4",
                    help="the other workloads timed after the step (comma list; 'none' for none): "
                         "fp32 = 1 head, d=64, S=256 in 4 partitions (16 tiles + 4 merges), "
                         "zigzag = causal zigzag share of S=131072, mesh = Mesh 8x8 tile of S=1048576, "
                         "striped = the same Mesh tile under the causal mask with striped positions, "
                         "small = a 13440-token share cut into tiles of 13440 down to 210 tokens, "
                         "bwd4 = backward of 4 Q partitions x one KV partition of 8192")
    ap.add_argument("--workload-reps", type=int, default=3, help="timed repetitions per workload entry (median)")
    ap.add_argument("--power-sample", type=float, default=5.0,
                    help="after the timed steps (outside the timed region), run the forward and then the backward "
                         "back to back for this many seconds each while sampling socket power and shader clocks "
                         "with amd-smi (0: off)")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="after the timed steps, one plain device copy of this many MiB (outside the timed "
                         "region): the reference launch for scaling HBM byte counters")
    return ap.parse_args()


def cpu_baseline(rows, scale):
    """The fp64 oracle on a bounded sample of the same workload: `rows` query rows x 32 heads,
    forward over all 8192 keys, the merge with the incoming partial, and the backward."""
    import numpy as np
    import synthetic
    from oracle import attn_tile, merge, attn_tile_bwd
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    _, qv = synthetic.normal_bf16(WORKLOAD_ID, synthetic.T_Q, 0, (1, SQ, HQ, D))
    _, kv = synthetic.normal_bf16(WORKLOAD_ID, synthetic.T_K, 0, (1, SK, HKV, D))
    _, vv = synthetic.normal_bf16(WORKLOAD_ID, synthetic.T_V, 0, (1, SK, HKV, D))
    _, dov = synthetic.normal_bf16(WORKLOAD_ID, synthetic.T_DO, 0, (1, SQ, HQ, D))
    _, oin = synthetic.normal_bf16(WORKLOAD_ID, synthetic.T_O_IN, 0, (1, SQ, HQ, D))
    lin = incoming_lse()
    sel = np.arange(rows)
    q = qv[:, sel]
    t0 = time.perf_counter()
    O, L = attn_tile(q, kv, vv, scale)
    Om, Lm = merge([(O, L), (oin[:, sel], lin[:, :, sel])])
    attn_tile_bwd(q, kv, vv, Om, dov[:, sel], Lm, scale)
    dt = time.perf_counter() - t0
    flops = (4 + 10) * D * HQ * rows * SK
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{rows} of {SQ} query rows x {HQ} heads against all {SK} keys: forward, 2-way merge, "
                      f"backward in float64 NumPy ({dt:.1f} s; cpu {platform.processor() or platform.machine()}, "
                      f"{len(os.sched_getaffinity(0))} host cores visible)"}


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
    import statistics
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
            for _ in range(20):
                fn()
            n += 20
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


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_tile_bwd_gqa_tile_8k.md")
KERNEL_SOURCES = ["bwd.hip", "fwd_bf16.hip", "merge.hip", "api.hip", "ma_device.h", "ma_internal.h"]


def kernel_source_hash():
    """sha256 over the HIP sources the measured kernels are built from (changes invalidate stored counters)."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "distributed_long_context_amd", "csrc")
    for name in KERNEL_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def stored_traffic():
    """HBM bytes per tile-backward launch from the committed counter summary, or None when the
    summary is missing or was taken on other kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
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
        return int(vals["tile_bwd_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def summarize_pmc(fetch_csv, write_csv, copy_mib, command):
    """Write the HBM-traffic summary of the tile backward from two rocprofv3 --pmc runs
    (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), each scaled by what the same counter
    reads for the plain device copy of copy_mib MiB made by --calib-copy-mb."""
    import csv
    import collections

    def per_kernel(path):
        by_dispatch = collections.OrderedDict()
        for r in csv.DictReader(open(path)):
            key = (int(r["Dispatch_Id"]), r["Kernel_Name"])
            by_dispatch[key] = by_dispatch.get(key, 0.0) + float(r["Counter_Value"])
        agg = collections.OrderedDict()
        for (_, name), v in by_dispatch.items():
            agg.setdefault(name, []).append(v)
        return {k: sum(v) / len(v) for k, v in agg.items()}

    fetch, write = per_kernel(fetch_csv), per_kernel(write_csv)
    copy_kib = copy_mib * 1024.0
    copy_name = next(k for k in fetch if "copyBuffer" in k or "copy" in k.lower())
    f_scale, w_scale = copy_kib / fetch[copy_name], copy_kib / write[copy_name]
    short = lambda n: n.replace("ma::(anonymous namespace)::", "").replace("void ", "").split("(")[0]
    bwd = [k for k in fetch if any(t in k for t in ("bwd_pre_kernel", "bwd_dq_kernel", "bwd_dkv_kernel"))]
    total = sum(fetch[k] * f_scale + write[k] * w_scale for k in bwd) * 1024
    lines = ["# HBM traffic of the tile backward, gqa-tile-8k (counters)", "",
             "Workload: one non-causal tile, Q 8192 x KV 8192 tokens, 32/8 heads, head_dim 128, bf16.",
             "Two rocprofv3 runs of the same command, one counter each (KiB per dispatch, averaged over",
             "the dispatches of each kernel):", "",
             "    " + command.replace("PMC", "FETCH_SIZE"), "    " + command.replace("PMC", "WRITE_SIZE"), "",
             f"Calibration: the plain device copy of {copy_mib} MiB ({short(copy_name)}) reads FETCH_SIZE "
             f"{fetch[copy_name]:.0f} KiB and WRITE_SIZE {write[copy_name]:.0f} KiB, so the factors are "
             f"{f_scale:.4f} (fetch) and {w_scale:.4f} (write).", "",
             "| Kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled MiB read | scaled MiB written |",
             "|---|---|---|---|---|"]
    for k in fetch:
        if k == copy_name or k not in write:
            continue
        lines.append(f"| {short(k)} | {fetch[k]:.0f} | {write[k]:.0f} | {fetch[k] * f_scale / 1024:.1f} | "
                     f"{write[k] * w_scale / 1024:.1f} |")
    lines += ["", "The tile backward entry point launches bwd_pre, bwd_dq and bwd_dkv once each; their sum is "
              "the traffic per launch that bench.py reports while the kernel sources are unchanged:", "",
              f"    tile_bwd_bytes_per_launch: {int(round(total))}",
              f"    source_sha256: {kernel_source_hash()}", ""]
    with open(TRAFFIC_FILE, "w") as f:
        f.write("\n".join(lines))
    print(f"wrote {TRAFFIC_FILE}: {total / 2**20:.1f} MiB per launch")


def incoming_lse():
    """LSE of the incoming partial: ln(8192) + 0.5 + N(0,1), float32 (seeded)."""
    import numpy as np
    import synthetic
    mu = math.log(SK) + 0.5
    return (synthetic.normal_f32(WORKLOAD_ID, synthetic.T_LSE_IN, 0, (1, HQ, SQ)) + np.float32(mu)).astype(np.float32)


def _timed(fn, reps, warmup=1):
    """Median milliseconds of fn() over `reps` runs after `warmup`, from events on the current stream.

    The runs are enqueued back to back and the host synchronises once at the end, so a host-side
    pause between recording an event and launching the work (seen as rare 30-40 ms outliers when
    every run synchronised) is hidden behind the queued work; the median drops any that remain."""
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
    ts = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
    mid = len(ts) // 2
    return ts[mid] if len(ts) % 2 else 0.5 * (ts[mid - 1] + ts[mid])


def _tf(flop, ms):
    t = flop / (ms * 1e-3) / 1e12
    return {"ms": round(ms, 4), "TFLOP/s": round(t, 1), "frac_bf16_peak": round(t / PEAK_BF16_TFLOPS, 4), "flop": flop}


def _gb(nbytes, ms):
    g = nbytes / (ms * 1e-3) / 1e9
    return {"ms": round(ms, 4), "GB/s": round(g, 1), "frac_hbm_peak": round(g / PEAK_HBM_GBPS, 4), "bytes": nbytes}


def measure_workloads(names, reps):
    """Times the other workloads of the hot path on the device, inputs resident in HBM.

    Inputs are N(0,1) drawn on the device from a seeded generator (the same distributions as the parity
    tests' host-drawn inputs, a different stream of numbers); O and LSE given to the backward have a real
    forward's magnitudes.  Algorithmic work counts allowed pairs only (4*d*Hq forward, 10*d*Hq backward)
    and merge/reduce bytes as each input read once plus each output written once."""
    import torch
    import distributed_long_context_amd as ma
    from distributed_long_context_amd import BwdTile, Tile

    dev = "cuda:0"
    gen = torch.Generator(device=dev)
    gen.manual_seed(1234)
    scale = float(1.0 / math.sqrt(D))

    def randn(shape, dtype=torch.bfloat16, mul=1.0, add=0.0):
        return (torch.randn(shape, generator=gen, device=dev, dtype=torch.float32) * mul + add).to(dtype)

    def out(sq):
        return (torch.empty((1, sq, HQ, D), dtype=torch.bfloat16, device=dev),
                torch.empty((1, HQ, sq), dtype=torch.float32, device=dev))

    res = {}
    if "zigzag" in names:
        N, r, C = 16, 5, 4096
        qchunks = ma.mesh_attn_map_zigzag(N, r)
        nkv = max(qchunks) + 1
        Q = {c: randn((1, C, HQ, D)) for c in qchunks}
        kg = randn((1, nkv * C, HKV, D))
        vg = randn((1, nkv * C, HKV, D))
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

        w = {"tiles": len(wl), "allowed_pairs_per_head": pairs}
        w["fwd_tiles"] = _tf(4.0 * D * HQ * pairs, _timed(lambda: ma.mesh_attn_tile_fwd(tiles, scale, ma.MA_MASK_CAUSAL), reps))
        w["merge_6_and_27"] = _gb(merge_bytes, _timed(merges, reps))
        w["fwd_fused_gathered_kv"] = _tf(4.0 * D * HQ * pairs,
                                         _timed(lambda: ma.mesh_attn_tile_fwd(ftiles, scale, ma.MA_MASK_CAUSAL), reps))
        # backward of the share: dQ of both chunks, partial dK/dV of KV chunks 0..26
        dO = {c: randn((1, C, HQ, D)) for c in qchunks}
        O = {c: randn((1, C, HQ, D), mul=0.02) for c in qchunks}
        L = {c: randn((1, HQ, C), torch.float32, 0.3, math.log(c * C + C / 2) + 0.5) for c in qchunks}
        dq = {c: torch.empty((1, C, HQ, D), dtype=torch.float32, device=dev) for c in qchunks}
        dk = [torch.empty((1, C, HKV, D), dtype=torch.float32, device=dev) for _ in range(nkv)]
        dv = [torch.empty_like(x) for x in dk]
        btiles = [BwdTile(Q[qchunks[i]], K[j], V[j], O[qchunks[i]], dO[qchunks[i]], L[qchunks[i]], dq[qchunks[i]],
                          dk[j], dv[j], qpos[i], kpos[j]) for i, j, _ in wl]
        ws = torch.empty(max(256, ma.mesh_attn_tile_bwd_workspace_size(btiles, scale, ma.MA_MASK_CAUSAL)), dtype=torch.uint8, device=dev)
        w["bwd_tiles"] = _tf(10.0 * D * HQ * pairs,
                             _timed(lambda: ma.mesh_attn_tile_bwd(btiles, scale, ma.MA_MASK_CAUSAL, workspace=ws), reps))
        res["zigzag-causal-128k-r5"] = w
        del Q, kg, vg, K, V, tiles, groups, merged, fused, ftiles, dO, O, L, dq, dk, dv, btiles, ws
        torch.cuda.empty_cache()
    if "mesh" in names:
        n, a, b, g, P = 64, 8, 8, 9, 16384
        qparts, kparts = ma.mesh_attn_map_mesh_tile(n, a, b, g, True)
        Q = {i: randn((1, P, HQ, D)) for i in qparts}
        kg = randn((1, b * P, HKV, D))
        vg = randn((1, b * P, HKV, D))
        K = {j: kg[:, t * P:(t + 1) * P] for t, j in enumerate(kparts)}
        V = {j: vg[:, t * P:(t + 1) * P] for t, j in enumerate(kparts)}
        tiles = {(i, j): Tile(Q[i], K[j], V[j], *out(P)) for i in qparts for j in kparts}
        mu = math.log(b * P) + 0.5
        inc = [(randn((1, P, HQ, D), mul=0.01), randn((1, HQ, P), torch.float32, 1.0, mu)) for _ in range(a - 1)]
        merged = {i: out(P) for i in qparts}
        pairs = len(tiles) * P * P
        part_bytes = P * HQ * D * 2 + HQ * P * 4
        merge_bytes = (7 * (8 + 1) + (15 + 1)) * part_bytes

        def merges():
            for i in qparts:
                os_ = [tiles[(i, j)].o for j in kparts]
                ls_ = [tiles[(i, j)].lse for j in kparts]
                if i == g:
                    os_ += [x[0] for x in inc]
                    ls_ += [x[1] for x in inc]
                ma.mesh_attn_merge(os_, ls_, merged[i][0], merged[i][1])

        fused = {i: out(P) for i in qparts}
        ftiles = [Tile(Q[i], kg, vg, *fused[i]) for i in qparts]

        def fused_step():
            ma.mesh_attn_tile_fwd(ftiles, scale, ma.MA_MASK_NONE)
            ma.mesh_attn_merge([fused[g][0]] + [x[0] for x in inc], [fused[g][1]] + [x[1] for x in inc],
                               fused[g][0], fused[g][1])

        w = {"tiles": len(tiles), "allowed_pairs_per_head": pairs}
        w["fwd_tiles"] = _tf(4.0 * D * HQ * pairs,
                             _timed(lambda: ma.mesh_attn_tile_fwd(list(tiles.values()), scale, ma.MA_MASK_NONE), reps))
        w["merge_7x8_and_15"] = _gb(merge_bytes, _timed(merges, reps))
        w["fwd_fused_gathered_kv_plus_owned_merge"] = _tf(4.0 * D * HQ * pairs, _timed(fused_step, reps))
        del tiles, merged, fused, ftiles
        torch.cuda.empty_cache()
        # GOO replay: k_Q = k_KV = 4 chunks per partition; the compute tasks C-i-j (gathered Q chunk i of
        # 8 x 4096 rows against gathered KV chunk j of 8 x 4096 keys) run in the greedy plan's order, each
        # folded into its Q chunk's (O, LSE) by the forward's accumulate mode
        kq = kkv = 4
        cq, ck = P // kq, P // kkv
        gq = [torch.cat([Q[i][:, c * cq:(c + 1) * cq] for i in qparts], dim=1) for c in range(kq)]
        gk = [torch.cat([K[j][:, c * ck:(c + 1) * ck] for j in kparts], dim=1) for c in range(kkv)]
        gv = [torch.cat([V[j][:, c * ck:(c + 1) * ck] for j in kparts], dim=1) for c in range(kkv)]
        acc = [out(a * cq) for _ in range(kq)]
        plan = ma.mesh_attn_goo_plan(kq, kkv, 0.5, 1.0, 0.5, 0.5, 1.0)
        order = [(i, j) for _, comp in plan for _, i, j in comp]

        def goo_replay():
            first = set()
            for i, j in order:
                ma.mesh_attn_tile_fwd([Tile(gq[i], gk[j], gv[j], acc[i][0], acc[i][1])], scale, ma.MA_MASK_NONE,
                                      accumulate=i in first)
                first.add(i)

        w["fwd_goo_replay_4x4"] = _tf(4.0 * D * HQ * pairs, _timed(goo_replay, reps))
        w["fwd_goo_replay_4x4"]["tasks"] = len(order)
        del gq, gk, gv, acc
        torch.cuda.empty_cache()
        # backward of the 8 x 8 tile: dQ_i over the 8 KV partitions, dK/dV_j over the 8 Q partitions
        dO = {i: randn((1, P, HQ, D)) for i in qparts}
        O = {i: randn((1, P, HQ, D), mul=0.01) for i in qparts}
        L = {i: randn((1, HQ, P), torch.float32, 0.3, mu) for i in qparts}
        dq = {i: torch.empty((1, P, HQ, D), dtype=torch.float32, device=dev) for i in qparts}
        dk = {j: torch.empty((1, P, HKV, D), dtype=torch.float32, device=dev) for j in kparts}
        dv = {j: torch.empty_like(dk[j]) for j in kparts}
        btiles = [BwdTile(Q[i], K[j], V[j], O[i], dO[i], L[i], dq[i], dk[j], dv[j]) for i in qparts for j in kparts]
        ws = torch.empty(max(256, ma.mesh_attn_tile_bwd_workspace_size(btiles, scale, ma.MA_MASK_NONE)), dtype=torch.uint8, device=dev)
        w["bwd_tiles"] = _tf(10.0 * D * HQ * pairs,
                             _timed(lambda: ma.mesh_attn_tile_bwd(btiles, scale, ma.MA_MASK_NONE, workspace=ws), 1))
        # the addition of the gradient reduce-scatter: 8 partial dQ of one Q partition (fp32) summed
        parts = [dq[i] for i in qparts]
        red = torch.empty_like(parts[0])
        w["reduce_add_8_dq"] = _gb(9 * parts[0].numel() * 4, _timed(lambda: ma.mesh_attn_reduce_add(parts, red), reps))
        res["mesh-8x8-1m-g9"] = w
        del Q, kg, vg, K, V, inc, dO, O, L, dq, dk, dv, btiles, ws, parts, red
        torch.cuda.empty_cache()
    if "striped" in names:
        # Mesh 8 x 8 share at S = 1,048,576 under the causal mask with the striped layout of [Mesh]
        # section 3.7: partition p holds tokens p + 64 t, so every (Q, KV) pair is PARTIAL
        n, a, b, g, P = 64, 8, 8, 9, 16384
        qparts, kparts = ma.mesh_attn_map_mesh_tile(n, a, b, g, True)
        Q = {i: randn((1, P, HQ, D)) for i in qparts}
        kg = randn((1, b * P, HKV, D))
        vg = randn((1, b * P, HKV, D))
        K = {j: kg[:, t * P:(t + 1) * P] for t, j in enumerate(kparts)}
        V = {j: vg[:, t * P:(t + 1) * P] for t, j in enumerate(kparts)}
        qpos = {i: ma.mesh_attn_pos_striped(n, i) for i in qparts}
        kpos = {j: ma.mesh_attn_pos_striped(n, j) for j in kparts}
        mode = ma.MA_MASK_STRIPED_ZIGZAG
        pairs = sum(ma.mesh_attn_count_allowed(qpos[i], P, kpos[j], P, mode) for i in qparts for j in kparts)
        tiles = [Tile(Q[i], K[j], V[j], *out(P), qpos[i], kpos[j]) for i in qparts for j in kparts]
        w = {"tiles": len(tiles), "allowed_pairs_per_head": pairs}
        w["fwd_tiles"] = _tf(4.0 * D * HQ * pairs, _timed(lambda: ma.mesh_attn_tile_fwd(tiles, scale, mode), reps))
        del tiles
        torch.cuda.empty_cache()
        dO = {i: randn((1, P, HQ, D)) for i in qparts}
        O = {i: randn((1, P, HQ, D), mul=0.01) for i in qparts}
        L = {i: randn((1, HQ, P), torch.float32, 0.3, math.log(b * P / 2) + 0.5) for i in qparts}
        dq = {i: torch.empty((1, P, HQ, D), dtype=torch.float32, device=dev) for i in qparts}
        dk = {j: torch.empty((1, P, HKV, D), dtype=torch.float32, device=dev) for j in kparts}
        dv = {j: torch.empty_like(dk[j]) for j in kparts}
        btiles = [BwdTile(Q[i], K[j], V[j], O[i], dO[i], L[i], dq[i], dk[j], dv[j], qpos[i], kpos[j])
                  for i in qparts for j in kparts]
        ws = torch.empty(max(256, ma.mesh_attn_tile_bwd_workspace_size(btiles, scale, mode)), dtype=torch.uint8, device=dev)
        w["bwd_tiles"] = _tf(10.0 * D * HQ * pairs, _timed(lambda: ma.mesh_attn_tile_bwd(btiles, scale, mode, workspace=ws), 1))
        res["mesh-8x8-1m-g9-striped-causal"] = w
        del Q, kg, vg, K, V, dO, O, L, dq, dk, dv, btiles, ws
        torch.cuda.empty_cache()
    if "small" in names:
        # Small-tile efficiency: one Q x KV share of 13440 x 13440 tokens (GQA 32/8, d = 128,
        # non-causal) cut into (13440 / P)^2 tiles of P x P tokens, all in one forward call, for
        # the partition sizes of [CHARM+]'s scaling table (13440 down to 210 tokens)
        S = 13440
        q = randn((1, S, HQ, D))
        k = randn((1, S, HKV, D))
        v = randn((1, S, HKV, D))
        o_all = torch.empty((S // 210) * S * HQ * D, dtype=torch.bfloat16, device=dev)
        l_all = torch.empty((S // 210) * HQ * S, dtype=torch.float32, device=dev)
        w = {}
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
            prep = ma.prepare_tile_fwd(tiles, scale, ma.MA_MASK_NONE)  # argument checks outside the timing
            w[f"fwd_P{P}"] = _tf(flop, _timed(lambda: ma.launch_prepared_tile_fwd(prep), reps))
            w[f"fwd_P{P}"]["tiles"] = n * n
        res["small-tiles-13440"] = w
        del q, k, v, o_all, l_all, tiles
        torch.cuda.empty_cache()
    if "fp32" in names:
        # the fp32 correctness configuration: 1 head, d = 64, S = 256 in 4 partitions of 64, all 16 tiles
        # in one call, then a 4-way merge per Q partition (launch-bound; reported, not a roofline target)
        S1, n1, d1 = 256, 4, 64
        P1 = S1 // n1
        q1 = torch.randn((1, S1, 1, d1), generator=gen, device=dev)
        k1 = torch.randn((1, S1, 1, d1), generator=gen, device=dev)
        v1 = torch.randn((1, S1, 1, d1), generator=gen, device=dev)
        outs = [(torch.empty((1, P1, 1, d1), device=dev), torch.empty((1, 1, P1), device=dev)) for _ in range(n1 * n1)]
        t16 = [Tile(q1[:, i * P1:(i + 1) * P1], k1[:, j * P1:(j + 1) * P1], v1[:, j * P1:(j + 1) * P1], *outs[i * n1 + j])
               for i in range(n1) for j in range(n1)]
        mo = [(torch.empty((1, P1, 1, d1), device=dev), torch.empty((1, 1, P1), device=dev)) for _ in range(n1)]
        s1 = float(1.0 / math.sqrt(d1))

        def c1():
            ma.mesh_attn_tile_fwd(t16, s1, ma.MA_MASK_NONE)
            for i in range(n1):
                row = outs[i * n1:(i + 1) * n1]
                ma.mesh_attn_merge([x[0] for x in row], [x[1] for x in row], mo[i][0], mo[i][1])

        ms = _timed(c1, max(reps, 5))
        res["fp32-s256-n4"] = {"fwd_and_merge": {"ms": round(ms, 4), "flop": 4.0 * d1 * S1 * S1,
                                                 "note": "launch-bound correctness configuration"}}
    if "bwd4" in names:
        S, nq = 8192, 4
        k = randn((1, S, HKV, D))
        v = randn((1, S, HKV, D))
        dk = torch.empty((1, S, HKV, D), dtype=torch.float32, device=dev)
        dv = torch.empty_like(dk)
        btiles = []
        for _ in range(nq):
            btiles.append(BwdTile(randn((1, S, HQ, D)), k, v, randn((1, S, HQ, D), mul=0.02), randn((1, S, HQ, D)),
                                  randn((1, HQ, S), torch.float32, 0.3, math.log(S) + 0.5),
                                  torch.empty((1, S, HQ, D), dtype=torch.float32, device=dev), dk, dv))
        ws = torch.empty(max(256, ma.mesh_attn_tile_bwd_workspace_size(btiles, scale, ma.MA_MASK_NONE)), dtype=torch.uint8, device=dev)
        res["gqa-bwd-4x8k"] = {"bwd_tiles": _tf(10.0 * D * HQ * nq * S * S, _timed(
            lambda: ma.mesh_attn_tile_bwd(btiles, scale, ma.MA_MASK_NONE, workspace=ws), reps))}
        del k, v, dk, dv, btiles, ws
        torch.cuda.empty_cache()
    return res


def main():
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
    import synthetic
    import distributed_long_context_amd as ma
    from distributed_long_context_amd import Pos, Tile, BwdTile

    parts = set(args.parts.split(","))
    dev = "cuda:0"
    torch.cuda.set_device(0)

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    scale = float(np.float32(1.0 / math.sqrt(D)))
    q = bf16(synthetic.normal_bf16(WORKLOAD_ID, synthetic.T_Q, 0, (1, SQ, HQ, D))[0])
    k = bf16(synthetic.normal_bf16(WORKLOAD_ID, synthetic.T_K, 0, (1, SK, HKV, D))[0])
    v = bf16(synthetic.normal_bf16(WORKLOAD_ID, synthetic.T_V, 0, (1, SK, HKV, D))[0])
    dO = bf16(synthetic.normal_bf16(WORKLOAD_ID, synthetic.T_DO, 0, (1, SQ, HQ, D))[0])
    o_in = bf16(synthetic.normal_bf16(WORKLOAD_ID, synthetic.T_O_IN, 0, (1, SQ, HQ, D))[0])
    lse_in = torch.from_numpy(incoming_lse()).to(dev)
    o = torch.empty((1, SQ, HQ, D), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((1, HQ, SQ), dtype=torch.float32, device=dev)
    o_m = torch.empty_like(o)
    lse_m = torch.empty_like(lse)
    dq = torch.empty((1, SQ, HQ, D), dtype=torch.float32, device=dev)
    dk = torch.empty((1, SK, HKV, D), dtype=torch.float32, device=dev)
    dv = torch.empty((1, SK, HKV, D), dtype=torch.float32, device=dev)
    q_pos, k_pos = ma.mesh_attn_pos_contiguous(0), ma.mesh_attn_pos_contiguous(0)
    bwd_tiles = [BwdTile(q, k, v, o_m, dO, lse_m, dq, dk, dv, q_pos, k_pos)]
    ws = None
    if "bwd" in parts:
        ws = torch.empty(max(256, ma.mesh_attn_tile_bwd_workspace_size(bwd_tiles, scale, ma.MA_MASK_NONE)), dtype=torch.uint8, device=dev)

    pairs = ma.mesh_attn_count_allowed(q_pos, SQ, k_pos, SK, ma.MA_MASK_NONE)
    fwd_flop = 4.0 * D * HQ * pairs
    bwd_flop = 10.0 * D * HQ * pairs
    merge_bytes = 2 * (SQ * HQ * D * 2 + HQ * SQ * 4) + (SQ * HQ * D * 2 + HQ * SQ * 4)

    stream = torch.cuda.current_stream()
    evs = []

    def step(record):
        # (1) host mapping: the tile list for this GPU's share (one non-causal pair)
        wl = ma.mesh_attn_build_worklist([q_pos], [SQ], [k_pos], [SK], ma.MA_MASK_NONE)
        assert wl == [(0, 0, ma.MA_TILE_FULL)]
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)] if record else None
        if record:
            e[0].record(stream)
        if "fwd" in parts:
            ma.mesh_attn_tile_fwd([Tile(q, k, v, o, lse, q_pos, k_pos)], scale, ma.MA_MASK_NONE)
        if record:
            e[1].record(stream)
        if "merge" in parts:
            ma.mesh_attn_merge([o, o_in], [lse, lse_in], o_m, lse_m)
        if record:
            e[2].record(stream)
        if "bwd" in parts:
            ma.mesh_attn_tile_bwd(bwd_tiles, scale, ma.MA_MASK_NONE, workspace=ws)
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
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps

    # the merge again with the 256 MB MALL flushed before each run (a 512 MiB write), so that its
    # inputs come from HBM (in the step they partly hit the MALL: the forward has just written one)
    merge_cold_ms = None
    if "merge" in parts:
        scratch = torch.empty(1 << 29, dtype=torch.uint8, device=dev)
        ts = []
        for it in range(6):
            scratch.fill_(it)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            ma.mesh_attn_merge([o, o_in], [lse, lse_in], o_m, lse_m)
            e1.record(stream)
            e1.synchronize()
            ts.append(e0.elapsed_time(e1))
        merge_cold_ms = sum(ts[1:]) / len(ts[1:])
        del scratch

    power = None
    if args.power_sample > 0:
        runs = []
        if "fwd" in parts:
            runs.append(("tile_fwd", lambda: ma.mesh_attn_tile_fwd([Tile(q, k, v, o, lse, q_pos, k_pos)], scale,
                                                                  ma.MA_MASK_NONE)))
        if "bwd" in parts:
            runs.append(("tile_bwd", lambda: ma.mesh_attn_tile_bwd(bwd_tiles, scale, ma.MA_MASK_NONE, workspace=ws)))
        power = power_clock(runs, args.power_sample)

    if args.calib_copy_mb > 0:
        n = args.calib_copy_mb * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def mean_median(i):
        ts = sorted(e[i].elapsed_time(e[i + 1]) for e in evs)
        mid = len(ts) // 2
        return sum(ts) / len(ts), (ts[mid] if len(ts) % 2 else 0.5 * (ts[mid - 1] + ts[mid]))

    (fwd_ms, fwd_med), (merge_ms, merge_med), (bwd_ms, bwd_med) = mean_median(0), mean_median(1), mean_median(2)
    step_flop = (fwd_flop if "fwd" in parts else 0) + (bwd_flop if "bwd" in parts else 0)
    value = step_flop / (ms_step * 1e-3) / 1e12

    res_parts = {}
    if "fwd" in parts:
        t = fwd_flop / (fwd_ms * 1e-3) / 1e12
        res_parts["tile_fwd"] = {"ms": round(fwd_ms, 4), "ms_median": round(fwd_med, 4), "TFLOP/s": round(t, 1),
                                 "frac_bf16_peak": round(t / PEAK_BF16_TFLOPS, 4), "flop": fwd_flop}
    if "merge" in parts:
        g = merge_bytes / (merge_ms * 1e-3) / 1e9
        res_parts["merge"] = {"ms": round(merge_ms, 4), "ms_median": round(merge_med, 4), "GB/s": round(g, 1),
                              "frac_hbm_peak": round(g / PEAK_HBM_GBPS, 4), "bytes": merge_bytes, "k": 2}
        gc = merge_bytes / (merge_cold_ms * 1e-3) / 1e9
        res_parts["merge_mall_flushed"] = {"ms": round(merge_cold_ms, 4), "GB/s": round(gc, 1),
                                           "frac_hbm_peak": round(gc / PEAK_HBM_GBPS, 4), "bytes": merge_bytes, "k": 2}
    if "bwd" in parts:
        t = bwd_flop / (bwd_ms * 1e-3) / 1e12
        res_parts["tile_bwd"] = {"ms": round(bwd_ms, 4), "ms_median": round(bwd_med, 4), "TFLOP/s": round(t, 1),
                                 "frac_bf16_peak": round(t / PEAK_BF16_TFLOPS, 4), "flop": bwd_flop,
                                 "includes": "D=rowsum(dO*O) preprocessing"}
    # dominant kernel by time
    dom = max(((n, p["ms"]) for n, p in res_parts.items() if n != "merge_mall_flushed"), key=lambda x: x[1])[0]
    if dom == "merge":
        rl = {"bound": "hbm", "achieved": res_parts["merge"]["GB/s"], "peak": PEAK_HBM_GBPS, "unit": "GB/s",
              "frac": res_parts["merge"]["frac_hbm_peak"], "traffic": None, "kernel": "merge"}
    else:
        rl = {"bound": "mfma", "achieved": res_parts[dom]["TFLOP/s"], "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
              "frac": res_parts[dom]["frac_bf16_peak"], "traffic": None, "kernel": dom}
        if dom == "tile_bwd":
            rl["kernel"] = "tile_bwd (mesh_attn_tile_bwd: bwd_pre + bwd_dq + bwd_dkv)"
            rl["traffic"] = stored_traffic()

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "gqa-tile-8k: one non-causal (Q 8192 x KV 8192) tile, 32/8 heads, d=128, bf16; "
                               "fwd + 2-way LSE merge + bwd", "batch": 1, "q_tokens": SQ, "kv_tokens": SK,
                   "q_heads": HQ, "kv_heads": HKV, "head_dim": D, "mask": "none", "steps_parts": sorted(parts)},
        "roofline": rl, "parts": res_parts,
    }
    if power is not None:
        # the dense bf16 peak scales with the shader clock: the rate each part reaches against the
        # peak at the clock the chip held while it ran
        for name in ("tile_fwd", "tile_bwd"):
            pw = power.get(name, {})
            if "gfx_mhz_median" in pw and name in res_parts:
                pk = PEAK_BF16_TFLOPS * pw["gfx_mhz_median"] / 2400.0
                pw["bf16_peak_at_held_clock_tflops"] = round(pk, 1)
                pw["frac_of_peak_at_held_clock"] = round(res_parts[name]["TFLOP/s"] / pk, 4)
        out["power_clock"] = power
    names = set(args.workloads.split(",")) - {"none", ""}
    if names:
        del q, k, v, dO, o_in, lse_in, o, lse, o_m, lse_m, dq, dk, dv, bwd_tiles, ws
        torch.cuda.empty_cache()
        out["workloads"] = measure_workloads(names, args.workload_reps)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.cpu_rows, np.float32(scale))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
