import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    # the host-only sanitizer build (tests/test_host_sanitizers.py) reruns the CPU tests of the ABI,
    # the mapper and the planner against its own library, named here
    alt = os.environ.get("MESH_ATTN_TEST_LIB")
    if alt:
        from distributed_long_context_amd import _abi
        _abi.LIB_PATH = alt


def pytest_collection_modifyitems(config, items):
    # GPU tests run only where a GPU is visible; on a CPU-only host they are skipped.
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for it in items:
        if "gpu" in it.keywords:
            it.add_marker(skip)
