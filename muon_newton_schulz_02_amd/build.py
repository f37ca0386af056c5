"""Build the HIP libraries in-tree for gfx950.

    python -m muon_newton_schulz_02_amd.build        # or build() from Python

libmuon_adamw.so is the optimizer (the C ABI of include/muon_adamw.h);
libma_peaks.so holds the ceiling probes the benchmark measures beside it
(csrc/peaks.hip).  Every source is compiled by hipcc with
--offload-arch=gfx950; packed-fp32 instruction selection is disabled for
device code.  The shared objects land next to this file, where the binding
loads them.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB = os.path.join(HERE, "libmuon_adamw.so")
BUILD_DIR = os.path.join(HERE, "_build")

SOURCES = ["plan.cpp", "step.cpp", "elementwise.hip", "ns_gemm.hip", "noalloc.hip"]
PEAKS_SOURCES = ["peaks.hip"]
PEAKS_LIB = os.path.join(HERE, "libma_peaks.so")

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
    "-I", INCLUDE, "-I", CSRC,
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def _compile(hipcc: str, src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [hipcc, *COMMON, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s\n%s" % (" ".join(cmd), res.stdout, res.stderr))
    return obj


def _link(hipcc: str, objs, out: str):
    tmp = out + ".tmp"
    cmd = [hipcc, "-shared", "--offload-arch=gfx950", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed: %s\n%s\n%s" % (" ".join(cmd), res.stdout, res.stderr))
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Compile every source and link both shared libraries; returns the
    optimizer library's path."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(5, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(hipcc, s), SOURCES + PEAKS_SOURCES))
    _link(hipcc, objs[:len(SOURCES)], LIB)
    _link(hipcc, objs[len(SOURCES):], PEAKS_LIB)
    if verbose:
        print("built", LIB)
        print("built", PEAKS_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
