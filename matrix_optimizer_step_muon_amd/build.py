"""Builds libmuon.so for gfx950 with hipcc, in-tree.

    python -m matrix_optimizer_step_muon_amd.build

The library goes to ``matrix_optimizer_step_muon_amd/_lib/libmuon.so``, and
objects go to ``_build/`` at the repository root (git-ignored). It always
compiles from scratch.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBDIR = os.path.join(PKG, "_lib")
LIB = os.path.join(LIBDIR, "libmuon.so")
BUILD = os.path.join(ROOT, "_build")

ARCH = "gfx950"
# Packed-fp32 instructions stay off in device code. hipcc's host pass warns
# that it does not know the feature; the warning is harmless.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", f"-I{INCLUDE}", f"-I{CSRC}",
          "-Wall", "-Wno-unused-function"]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found")
    return path


def _run(cmd):
    print("+", " ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if out.strip():
        print(out, flush=True)
    if res.returncode != 0:
        raise RuntimeError(f"build step failed ({res.returncode}): {' '.join(cmd)}")


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    cc = hipcc()
    k_obj = os.path.join(BUILD, "muon_kernels.o")
    a_obj = os.path.join(BUILD, "muon_api.o")
    p_obj = os.path.join(BUILD, "muon_partition.o")
    _run([cc, *COMMON, *DEVICE_FLAGS, "-c", os.path.join(CSRC, "muon_kernels.hip"), "-o", k_obj])
    _run([cc, *COMMON, "-c", os.path.join(CSRC, "muon_api.cpp"), "-o", a_obj])
    _run([cc, *COMMON, "-c", os.path.join(CSRC, "muon_partition.cpp"), "-o", p_obj])
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, k_obj, a_obj, p_obj,
          "-Wl,-soname,libmuon.so", "-Wl,-rpath,/opt/rocm/lib"])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
