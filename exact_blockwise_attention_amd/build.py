"""Build libra.so (the C-ABI library) for gfx950 with hipcc, in-tree.

Usage: python -m exact_blockwise_attention_amd.build   (or build() from Python)

Every source is compiled on each call (object files go to _build/ next to
this file), then linked into exact_blockwise_attention_amd/libra.so.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB = os.path.join(HERE, "libra.so")
SOURCES = ["ra_api.cpp", "ra_fwd.hip", "ra_misc.hip", "ra_bwd.hip", "ra_dq.hip", "ra_dqds.hip", "ra_gemm.hip"]
ARCH = "gfx950"

# Packed fp32 VALU instructions are disabled for all device code.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r


def _check_launch_stubs(lib):
    """Fail the build when a kernel's host launch stub is undefined in the
    library: hipcc drops it without a diagnostic when the host pass cannot
    instantiate a kernel template, and the library then fails only at load."""
    r = subprocess.run(["nm", lib], capture_output=True, text=True)
    if r.returncode != 0:
        return  # no nm: nothing to check with
    missing = [ln.split()[-1] for ln in r.stdout.splitlines() if " U " in ln and "__device_stub__" in ln]
    if missing:
        raise RuntimeError(f"{lib}: undefined kernel launch stubs: {missing}")


def build(verbose: bool = False) -> str:
    cc = hipcc()
    out_dir = os.path.join(HERE, "_build")
    os.makedirs(out_dir, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(out_dir, src + ".o")
        cmd = [cc, *HIP_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
        if src.endswith(".cpp"):
            cmd[1:1] = ["-x", "hip"]
        _run(cmd)
        return obj

    workers = min(len(SOURCES), max(1, (os.cpu_count() or 4)))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    _check_launch_stubs(tmp)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
