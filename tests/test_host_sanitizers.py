"""The host C++ under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

tests/sanitize/build.py compiles the ABI layer's host code (argument validation, launch planning,
parameter packing, segment expansion), the mapper and the GOO planner with both sanitizers, linked
with launch stubs that report "no device".  The CPU tests of the ABI, the mapper and the planner then
run in a child process against that library, with the sanitizer runtime preloaded; any report
fails the child and so this test.
"""
import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BUILD = os.path.join(ROOT, "tests", "sanitize", "build.py")


def _builder():
    spec = importlib.util.spec_from_file_location("ma_sanitize_build", BUILD)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_host_code_under_address_and_ub_sanitizers():
    b = _builder()
    lib = b.build()
    env = dict(os.environ)
    env.update(LD_PRELOAD=b.runtime(), MESH_ATTN_TEST_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0:exitcode=86",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1:exitcode=87")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                        "tests/test_abi_host.py", "tests/test_mapper.py", "tests/test_goo.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, out
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, out
    assert " passed" in r.stdout, out
