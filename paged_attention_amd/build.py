"""Builds libpkv.so in-tree: HIP kernels for gfx950 plus the host allocator.

``python paged_attention_amd/build.py`` (or ``build()``) compiles every source
under ``csrc/`` with hipcc and links ``paged_attention_amd/libpkv.so``.  The
shared library is what the Python binding loads; nothing is compiled at import
time.  This file imports nothing from the package, so it runs even when no
library (or a stale one) is present.
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
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libpkv.so")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
ROCM = os.environ.get("ROCM_PATH", os.path.dirname(os.path.dirname(os.path.realpath(HIPCC))))

COMMON = ["-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-DPKV_BUILDING_LIBRARY", f"-I{INCLUDE}", f"-I{CSRC}"]
# Device code: gfx950 only; packed FP32 instructions disabled.
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]

HIP_SOURCES = ["kernels.hip", "kernels_q8.hip", "block_kernels.hip"]
HOST_SOURCES = ["allocator.cpp", "status.cpp", "prefix_groups.cpp"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"build step failed ({res.returncode}): {' '.join(cmd)}")
    return res


def build(verbose: bool = False) -> str:
    """Compile all sources and link libpkv.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        jobs.append([HIPCC, *COMMON, *DEVICE, "-c", os.path.join(CSRC, src), "-o", obj])
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        # Host-only C++ (no device code): compiled by hipcc's clang as plain C++.
        jobs.append([HIPCC, *COMMON, f"-I{ROCM}/include", "-D__HIP_PLATFORM_AMD__", "-x", "c++", "-c",
                     os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        list(ex.map(lambda c: _run(c, verbose), jobs))
    objs = [os.path.join(BUILD, s + ".o") for s in HIP_SOURCES + HOST_SOURCES]
    tmp = LIB + ".tmp"
    _run([HIPCC, *DEVICE, "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
