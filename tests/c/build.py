"""Compile the plain-C driver of the C ABI (tests/c/abi_step.c) against the
built library: gcc, C99, the HIP runtime API headers and libamdhip64 only.

    python tests/c/build.py
"""

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PKG = os.path.join(ROOT, "muon_newton_schulz_02_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
EXE = os.path.join(HERE, "abi_step")


def build(verbose: bool = False) -> str:
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no C compiler for the C ABI driver")
    if not os.path.exists(os.path.join(PKG, "libmuon_adamw.so")):
        raise RuntimeError("build libmuon_adamw.so first")
    cmd = [cc, "-std=c99", "-O2", "-Wall", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
           os.path.join(HERE, "abi_step.c"), "-o", EXE + ".tmp",
           "-L", PKG, "-l:libmuon_adamw.so", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../muon_newton_schulz_02_amd",
           "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("C driver build failed: %s\n%s%s" % (" ".join(cmd), res.stdout,
                                                               res.stderr))
    os.replace(EXE + ".tmp", EXE)
    if verbose:
        print("built", EXE)
    return EXE


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
