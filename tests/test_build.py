"""Build-level checks of the kernels' register use (no GPU needed).

The fused kernels keep each wave's fp32 state slice in registers for a whole run; a change that
pushes one of them past its register budget makes the compiler spill to scratch memory, which
costs far more than the change gains (it has happened: one shape's fused scan went from 0.64 ms
to 0.95 ms). The unfused and quadratic kernels are tuned for occupancy and have spilled silently
when a change held values across their main loops. These tests read the kernel descriptors of
the built device code and fail on any scratch use or register spill.
"""

import os
import re
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BUILD = os.path.join(ROOT, "mamba_ssd_chunked_cumsum_amd", "_build")
OBJ = os.path.join(BUILD, "ssd_fused.o")
LLVM = "/opt/rocm/llvm/bin"


def _tool(name):
    p = os.path.join(LLVM, name)
    return p if os.path.exists(p) else shutil.which(name)


def _kernel_descriptors(obj=OBJ):
    objcopy, bundler, readelf = _tool("llvm-objcopy"), _tool("clang-offload-bundler"), _tool(
        "llvm-readelf")
    if not (os.path.exists(obj) and objcopy and bundler and readelf):
        pytest.skip("kernels not built here, or the ROCm LLVM tools are missing")
    with tempfile.TemporaryDirectory() as tmp:
        fat, dev = os.path.join(tmp, "fatbin"), os.path.join(tmp, "dev.o")
        subprocess.run([objcopy, f"--dump-section=.hip_fatbin={fat}", obj, os.path.join(tmp, "x")],
                       check=True, capture_output=True)
        subprocess.run([bundler, "--unbundle", "--type=o", f"--input={fat}",
                        "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", f"--output={dev}"],
                       check=True, capture_output=True)
        notes = subprocess.run([readelf, "--notes", dev], check=True, capture_output=True,
                               text=True).stdout
    kernels, cur = {}, None
    for line in notes.splitlines():
        m = re.match(r"\s+\.name:\s+(\S+)", line)
        if m:
            cur = m.group(1)
            kernels[cur] = {}
            continue
        m = re.match(r"\s+\.(private_segment_fixed_size|vgpr_spill_count|sgpr_spill_count|"
                     r"vgpr_count):\s+(\d+)", line)
        if m and cur is not None:
            kernels[cur][m.group(1)] = int(m.group(2))
    return kernels


def test_fused_kernels_use_no_scratch():
    kernels = _kernel_descriptors()
    fused = {k: v for k, v in kernels.items()
             if any(n in k for n in ("k_run_states", "k_state_chain", "k_fused_scan"))}
    # 6 (headdim, dstate) shapes: run states and the fused scan; one chain kernel
    assert len(fused) == 13, sorted(kernels)
    bad = {k: v for k, v in fused.items()
           if v.get("private_segment_fixed_size", 0) or v.get("vgpr_spill_count", 0)}
    assert not bad, f"fused kernels spilling to scratch: {bad}"


@pytest.mark.parametrize("source", ["ssd_unfused", "ssd_quad", "ssd_step", "ssd_backward"])
def test_other_kernels_use_no_scratch(source):
    kernels = _kernel_descriptors(os.path.join(BUILD, source + ".o"))
    assert kernels, source
    bad = {k: v for k, v in kernels.items()
           if v.get("private_segment_fixed_size", 0) or v.get("vgpr_spill_count", 0)}
    assert not bad, f"{source} kernels spilling to scratch: {bad}"
