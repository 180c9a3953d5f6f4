"""Host-only build of the library with AddressSanitizer and UndefinedBehaviorSanitizer (test infrastructure).

Compiles the ABI layer (csrc/api.hip; sanitizers on its host side only), the mapper and the GOO planner with
-fsanitize=address,undefined and links them with launch stubs that report "no device", into
tests/sanitize/_build/libmesh_attn_host_asan.so.  The CPU tests of the ABI, the mapper and the
planner then run against it (tests/test_host_sanitizers.py).  The sanitizer flags apply to host
code only; nothing here is built for or run on a GPU.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
CSRC = os.path.join(ROOT, "distributed_long_context_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT_DIR = os.path.join(HERE, "_build")
OUT = os.path.join(OUT_DIR, "libmesh_attn_host_asan.so")

CLANG = os.environ.get("MA_HOST_CLANG", "/opt/rocm/llvm/bin/clang++")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]
# the HIP source also has a device part (a device array, no kernels): the sanitizers go to the
# host side only
SAN_HOST_ONLY = [x for f in SAN for x in ("-Xarch_host", f)]
COMMON = ["-O1", "-g", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC, "-Wno-unused-command-line-argument"]
# (source, extra flags): the ABI layer as HIP host code, the rest as plain C++
SOURCES = [
    (os.path.join(CSRC, "api.hip"), ["-x", "hip", "--offload-arch=gfx950"]),
    (os.path.join(CSRC, "mapper.cpp"), ["-x", "c++"]),
    (os.path.join(CSRC, "goo.cpp"), ["-x", "c++"]),
    (os.path.join(HERE, "launch_stubs.cpp"), ["-x", "c++", "-D__HIP_PLATFORM_AMD__"]),
]


def runtime() -> str:
    """Path of the shared AddressSanitizer runtime that a host process must preload."""
    r = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True,
                       check=True)
    return r.stdout.strip()


def build() -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    objs = []
    for src, extra in SOURCES:
        obj = os.path.join(OUT_DIR, os.path.basename(src) + ".o")
        san = SAN_HOST_ONLY if src.endswith(".hip") else SAN
        cmd = [CLANG] + COMMON + san + extra + ["-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"sanitizer build failed for {src}:\n{r.stderr}")
        objs.append(obj)
    hip_lib = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "lib")
    tmp = OUT + ".tmp"
    cmd = [CLANG, "-shared", "-shared-libsan"] + SAN + ["-o", tmp] + objs + \
          ["-L", hip_lib, "-Wl,-rpath," + hip_lib, "-lamdhip64"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitizer link failed:\n{r.stderr}")
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(), file=sys.stderr)
