"""Build libcoc.so (gfx950) in-tree with hipcc.

    python -m tensor_gemm_collective_amd.csrc.build [-v]

Objects go to tensor_gemm_collective_amd/csrc/_build/, the library to
tensor_gemm_collective_amd/libcoc.so.  Always recompiles.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
ROOT = os.path.dirname(PKG)
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(PKG, "libcoc.so")
ARCH = "gfx950"

# coc_api.cpp holds host code and one device array (the allocation-free entry
# point's scratch memory), so it takes the device pass as well; diag.hip holds
# the MFMA-rate diagnostic.
DEVICE_SOURCES = ["kernels.hip", "coc_api.cpp", "diag.hip"]
HOST_SOURCES = ["coc_plan.cpp"]

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{HERE}"]
# Device code: gfx950 only, packed-fp32 instructions disabled.
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wno-unused-command-line-argument", "-Wno-inline-asm"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if verbose and (r.stdout or r.stderr):
        print(r.stdout + r.stderr, flush=True)


def build(verbose: bool = False, defines=(), lib_path: str = LIB_PATH, build_dir: str = BUILD_DIR) -> str:
    """Compile and link libcoc.so.  `defines` (e.g. ["COC_RING_MIN_TILES=128"]) override
    the build-time tuning knobs of kernels.hip."""
    cc = hipcc()
    os.makedirs(build_dir, exist_ok=True)
    dflags = [f"-D{d}" for d in defines]
    jobs = []
    for s in DEVICE_SOURCES:
        obj = os.path.join(build_dir, s + ".o")
        jobs.append([cc, *COMMON, *DEVICE, *dflags, "-x", "hip", "-c", os.path.join(HERE, s), "-o", obj])
    for s in HOST_SOURCES:
        obj = os.path.join(build_dir, s + ".o")
        # host code only: no device pass (it holds no kernels)
        jobs.append([cc, *COMMON, "--offload-host-only", *dflags, "-c", os.path.join(HERE, s), "-o", obj])
    with ThreadPoolExecutor(max_workers=min(4, len(jobs))) as ex:
        list(ex.map(lambda c: _run(c, verbose), jobs))
    objs = [j[-1] for j in jobs]
    tmp = lib_path + ".tmp"
    _run([cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp], verbose)
    os.replace(tmp, lib_path)
    return lib_path


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
