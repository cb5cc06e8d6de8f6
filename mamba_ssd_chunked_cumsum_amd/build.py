"""Build libssd.so (HIP kernels for gfx950 + the C-ABI host code) in-tree with hipcc.

    python -m mamba_ssd_chunked_cumsum_amd.build

Always recompiles. Objects go to mamba_ssd_chunked_cumsum_amd/_build/, the library to
mamba_ssd_chunked_cumsum_amd/_lib/libssd.so.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIBDIR = os.path.join(PKG, "_lib")
LIB = os.path.join(LIBDIR, "libssd.so")

SOURCES = ["ssd_api.cpp", "ssd_unfused.hip", "ssd_fused.hip", "ssd_step.hip", "ssd_backward.hip",
           "ssd_quad.hip", "ssd_scratch.hip"]
ARCH = "gfx950"

# Packed-fp32 VALU forms stay disabled in device code (the compiler would otherwise fuse pairs of
# fp32 adds/multiplies into them).
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Xclang", "-target-feature",
          "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include")]


# Per-source extras. The fused kernels keep their matrix-core accumulators in ordinary VGPRs
# (their VALU work reads the carried state every sub-chunk); AGPRs then hold what does not fit.
EXTRA = {"ssd_fused.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found; the ROCm toolchain is required to build libssd")
    return p


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    cc = hipcc()
    procs, objs = [], []
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        if not os.path.exists(path):
            continue
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [cc, *COMMON, *EXTRA.get(src, []), *lang, "-c", path, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                            text=True)))
        objs.append(obj)
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        noise = "is not a recognized feature for this target"
        text = "\n".join(l for l in out.splitlines() if noise not in l)
        if text.strip() and (verbose or p.returncode):
            print(text, file=sys.stderr)
        if p.returncode:
            failed.append(src)
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    tmp = LIB + ".tmp"
    cmd = [cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    write_build_info(cc)
    return LIB


BUILD_INFO = os.path.join(LIBDIR, "build_info.json")


def write_build_info(cc: str) -> None:
    """Record what the library was built from (it travels with the library to hosts without the
    git history): the git revision and whether the tree differed from it, and the compiler."""
    import json

    def run(args):
        try:
            return subprocess.run(args, cwd=ROOT, capture_output=True, text=True,
                                  timeout=30).stdout.strip()
        except (OSError, subprocess.SubprocessError):
            return ""

    info = {
        "git_rev": run(["git", "rev-parse", "HEAD"]) or None,
        "git_dirty": bool(run(["git", "status", "--porcelain", "--untracked-files=no"])),
        "hipcc": (run([cc, "--version"]).splitlines() or [""])[0],
        "arch": ARCH,
    }
    with open(BUILD_INFO, "w") as f:
        json.dump(info, f, indent=1)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
