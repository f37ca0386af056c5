"""The library's host code (plan building, argument validation, the overlap
check, descriptor tables) under AddressSanitizer and UndefinedBehaviorSanitizer.

plan.cpp and step.cpp are compiled by g++ with both sanitizers and linked
with the library's device objects as built for gfx950; the ABI's CPU tests
(tests/test_abi_cpu.py) then run in a child Python process with that library
loaded and the sanitizer runtimes preloaded, halting on the first report.
No GPU is touched: those tests only call host entry points or make calls
that validation rejects before any launch.
"""

import glob
import os
import shutil
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
PKG = os.path.join(ROOT, "muon_newton_schulz_02_amd")
CSRC = os.path.join(PKG, "csrc")
HOST_SOURCES = ("plan.cpp", "step.cpp")


def _gcc_runtime(name):
    out = subprocess.run(["g++", "-print-file-name=%s" % name], capture_output=True, text=True)
    path = out.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_host_code_under_asan_and_ubsan(tmp_path):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    asan, ubsan = _gcc_runtime("libasan.so"), _gcc_runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("sanitizer runtimes not available")
    build_dir = os.path.join(PKG, "_build")
    if not glob.glob(os.path.join(build_dir, "*.o")):
        sys.path.insert(0, ROOT)
        from muon_newton_schulz_02_amd import build as B
        B.build()
    flags = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fPIC",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
             "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I", CSRC,
             "-I", os.path.join(ROOT, "include")]
    objs = []
    for src in HOST_SOURCES:
        obj = str(tmp_path / (src + ".o"))
        subprocess.run(["g++", *flags, "-c", os.path.join(CSRC, src), "-o", obj], check=True)
        objs.append(obj)
    # the device objects, as the package build made them (copied under
    # neutral names)
    for k, obj in enumerate(sorted(glob.glob(os.path.join(build_dir, "*.o")))):
        if os.path.basename(obj).split(".")[0] + ".cpp" in HOST_SOURCES:
            continue
        dst = str(tmp_path / ("device_%d.o" % k))
        shutil.copy(obj, dst)
        objs.append(dst)
    lib = str(tmp_path / "libmuon_adamw_sanitized.so")
    subprocess.run(["g++", "-shared", "-fsanitize=address,undefined", "-o", lib, *objs,
                    "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"], check=True)
    env = dict(os.environ)
    env["LD_PRELOAD"] = "%s %s" % (asan, ubsan)
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    driver = ("import sys; sys.path.insert(0, %r)\n"
              "import muon_newton_schulz_02_amd._abi as A\n"
              "A.load(%r)\n"
              "import pytest\n"
              "sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', %r]))\n"
              % (ROOT, lib, os.path.join(HERE, "test_abi_cpu.py")))
    res = subprocess.run([sys.executable, "-c", driver], cwd=ROOT, env=env, capture_output=True,
                         text=True, timeout=600)
    report = res.stdout[-3000:] + res.stderr[-3000:]
    assert res.returncode == 0, report
    assert "ERROR: AddressSanitizer" not in res.stderr and "runtime error" not in res.stderr, report
    assert " passed" in res.stdout, report
