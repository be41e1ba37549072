"""Build librhtq.so in-tree with hipcc for gfx950.

    python randomized_hadamard_rotation_amd/build.py

(run as a script: importing the package itself needs the library this builds)

Every HIP translation unit is compiled with packed-FP32 instruction selection
disabled; objects are compiled in parallel and linked into one shared library next
to this file.
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "librhtq.so")
OBJDIR = os.path.join(ROOT, "_build")

ARCH = os.environ.get("RHTQ_OFFLOAD_ARCH", "gfx950")
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          # keep MFMA results in ordinary VGPRs (no AGPR round trips)
          "-mllvm", "-amdgpu-mfma-vgpr-form",
          "-Wall", "-Wno-unused-function"]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


# Per-source flags.  The order-172 kernels run with the hardware's IEEE mode off
# (-mno-amdgpu-ieee, which requires -fno-honor-nans): inputs are finite by contract, and without
# signalling-NaN quieting the compiler no longer canonicalises each matrix-core result with an
# extra max before taking maxima of absolute values.
PER_FILE = {"rhtq_fast172.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee"]}


def _compile(src: str, hipcc: str, verbose: bool) -> str:
    obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [hipcc, *COMMON, *PER_FILE.get(os.path.basename(src), []), *lang, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return obj


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, hipcc, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
