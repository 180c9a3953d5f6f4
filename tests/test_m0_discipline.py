"""The kernels load global memory straight into LDS with inline assembly that writes M0 (the LDS
address of global_load_lds) and declares it clobbered.  M0 is a reserved register: the compiler
does not promise to preserve a value of its own in M0 across such a statement.  The kernels are
correct only while the compiler keeps nothing in M0, so this test compiles every HIP source to
gfx950 assembly with the build's flags and checks that M0 appears only in the helper's own
sequence (s_mov_b32 m0, <sgpr>; s_nop 0; global_load_lds_dwordx4) and nowhere else."""
import os
import re
import shutil
import subprocess

import pytest

from distributed_long_context_amd import build as B

M0 = re.compile(r"\bm0\b")
# instructions that read or write M0 without naming it
IMPLICIT_M0 = re.compile(r"^(v_movrel|s_movrel|s_set_gpr_idx|s_sendmsg|s_ttracedata|ds_gws|ds_ordered_count|v_interp|"
                         r"ds_\w*addtid|buffer_\w*lds|global_load_lds|scratch_load_lds)")


def _device_asm(src, out):
    cmd = [B.HIPCC] + [f for f in B.COMMON if f != "-fPIC"] + B.DEVICE_FLAGS + B.FAST_FLAGS.get(src, []) + \
        ["--cuda-device-only", "-S", "-o", out, os.path.join(B.CSRC, src)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    with open(out) as f:
        return [ln.split(";")[0].strip() for ln in f]


def _instructions(lines):
    return [ln for ln in lines if ln and not ln.startswith(".") and not ln.endswith(":")]


@pytest.mark.skipif(shutil.which(B.HIPCC) is None and not os.path.exists(B.HIPCC), reason="hipcc not found")
@pytest.mark.parametrize("src", [s for s in B.SOURCES if s.endswith(".hip")])
def test_m0_is_written_only_by_the_lds_dma_helper(src, tmp_path):
    ins = _instructions(_device_asm(src, str(tmp_path / (src + ".s"))))
    writes = 0
    for i, ln in enumerate(ins):
        if IMPLICIT_M0.match(ln):
            # only the helper's own load, right after its M0 write
            assert ln.startswith("global_load_lds_dwordx4") and i >= 2 and ins[i - 1] == "s_nop 0" and \
                re.fullmatch(r"s_mov_b32\s+m0,\s*s\d+", ins[i - 2]), f"{src}: instruction using M0: {ins[i - 2:i + 1]!r}"
            continue
        if not M0.search(ln):
            continue
        assert re.fullmatch(r"s_mov_b32\s+m0,\s*s\d+", ln), f"{src}: M0 used outside the DMA helper: {ln!r}"
        assert ins[i + 1] == "s_nop 0" and ins[i + 2].startswith("global_load_lds_dwordx4"), \
            f"{src}: M0 written without the helper's load after it: {ins[i:i + 3]!r}"
        writes += 1
    if src in ("fwd_bf16.hip", "bwd.hip"):
        assert writes > 0  # these kernels do use the helper
