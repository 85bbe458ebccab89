"""Build the C-ABI library libfa_mi355x.so in-tree with hipcc for gfx950.

Usage: ``python io_aware_attention_fa_amd/build.py`` (or ``__graft_entry__.build()``).  Run it as
a file, not as ``-m io_aware_attention_fa_amd.build``: importing the package loads the library,
which fails while it is missing or older than its header.  Every call compiles from source;
objects go to ``_build/`` and the library next to this file.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libfa_mi355x.so"

SOURCES = ["fa_validate.cpp", "fa_host.cpp", "fa_fwd_kernel.hip", "fa_decode_kernel.hip",
           "fa_bwd_kernel.hip", "fa_softmax_kernel.hip",
           "fa_elementwise_kernel.hip", "fa_noalloc.hip"]

ARCH = "gfx950"
# Packed-fp32 VALU instructions are kept out of every kernel.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
                "-Wno-unused-command-line-argument"]
# The forward kernel never produces or consumes NaN (masked scores are -inf), so it runs with the
# IEEE mode bit off: min/max then need no quieting of their inputs (no canonicalising moves).
PER_SOURCE_FLAGS = {"fa_fwd_kernel.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee"]}


def library_path() -> str:
    return os.path.join(PKG, LIB_NAME)


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the ROCm toolchain is required to build the library")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r


def build_library(verbose: bool = False) -> str:
    """Compile every source and link libfa_mi355x.so; returns its path."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        _run([hipcc, *COMMON_FLAGS, *DEVICE_FLAGS, *PER_SOURCE_FLAGS.get(src, []), "-I", INCLUDE,
              "-I", CSRC, *lang, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        return obj

    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    out = library_path()
    tmp = out + ".tmp"
    _run([hipcc, "-shared", f"--offload-arch={ARCH}", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, out)
    build_calibration(verbose)
    return out


def calibration_library_path() -> str:
    return os.path.join(PKG, "libfa_calib.so")


def build_calibration(verbose: bool = False) -> str:
    """The gfx950 calibration microbenchmarks (libfa_calib.so, see calibrate.py)."""
    out = calibration_library_path()
    tmp = out + ".tmp"
    _run([_hipcc(), *COMMON_FLAGS, *DEVICE_FLAGS, "-shared", "-x", "hip",
          os.path.join(PKG, "calib", "fa_calib.hip"), "-o", tmp], verbose)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv))
