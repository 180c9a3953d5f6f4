"""Build libmesh_attn.so in-tree with hipcc for gfx950.

Usage: ``python -m distributed_long_context_amd.build`` (or ``build()``).
Every call recompiles; objects go to ``_build/`` at the repository root and the
library to ``distributed_long_context_amd/libmesh_attn.so``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "libmesh_attn.so")
BUILD_DIR = os.path.join(ROOT, "_build")

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed fp32 VALU forms are kept out of the device code on purpose.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# Kernels never produce or consume NaN on purpose (masked scores are -inf); this lets
# fmaxf lower to plain v_max/v_max3 without NaN canonicalisation.
FAST_FLAGS = {"fwd_bf16.hip": ["-fno-honor-nans"], "bwd.hip": ["-fno-honor-nans"]}
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC, "-Wno-unused-command-line-argument"]

SOURCES = ["api.hip", "fwd_bf16.hip", "fwd_f32.hip", "merge.hip", "reduce.hip", "bwd.hip", "mapper.cpp", "goo.cpp"]


def _compile(src: str) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD_DIR, src + ".o")
    cmd = [HIPCC] + COMMON + DEVICE_FLAGS + FAST_FLAGS.get(src, [])
    if src.endswith(".cpp"):
        cmd += ["-x", "c++"]
    cmd += ["-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    workers = max(1, min(len(srcs), 8, os.cpu_count() or 1))
    with cf.ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}", file=sys.stderr)
    return OUT


if __name__ == "__main__":
    build()
