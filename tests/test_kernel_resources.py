"""Resource budgets of the Newton-Schulz kernels, read from the gfx950
assembly the compiler writes for csrc/ns_gemm.hip (no GPU needed).

The bf16 GEMM kernels run eight waves per workgroup, two per SIMD, and in
the overlapped step one AdamW wave shares each SIMD with them: each GEMM
wave must stay within 216 registers (2 x 216 + the AdamW kernel's 80 = 512,
a SIMD's register file), with no spills, and the workgroup's LDS within the
160 KB of a compute unit."""

import os
import re
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "muon_newton_schulz_02_amd", "csrc")


def _hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    pytest.skip("hipcc not available")


def _kernels(src, tmp_path):
    out = str(tmp_path / (os.path.basename(src) + ".s"))
    subprocess.run([_hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                    "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-x", "hip",
                    "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", out],
                   check=True, capture_output=True)
    text = open(out).read()
    meta = text[text.index("amdhsa.kernels:"):]
    res = {}
    for block in meta.split("\n  - ")[1:]:
        name = re.search(r"\.name:\s+(\S+)", block)
        if not name:
            continue
        get = lambda key: int(re.search(r"\.%s:\s+(\d+)" % key, block).group(1))
        res[name.group(1)] = dict(vgpr=get("vgpr_count"), agpr=get("agpr_count"),
                                  spill=get("vgpr_spill_count"),
                                  lds=get("group_segment_fixed_size"))
    return res


def test_bf16_gemm_register_and_lds_budget(tmp_path):
    ks = _kernels("ns_gemm.hip", tmp_path)
    bf16 = {n: r for n, r in ks.items() if "_bf16" in n and "k_ns_" in n and "lds" not in n}
    assert len(bf16) == 4, sorted(ks)
    # the one-workgroup kernel for small bf16 matrices holds a whole matrix
    # in LDS (and still leaves a SIMD room for a side AdamW wave)
    lds = [r for n, r in ks.items() if "k_ns_lds_bf16" in n]
    assert len(lds) == 1 and lds[0]["lds"] <= 160 * 1024, lds
    assert lds[0]["vgpr"] + lds[0]["agpr"] <= 512 - 80, lds
    for name, r in bf16.items():
        assert r["vgpr"] + r["agpr"] <= 216, (name, r)
        assert r["spill"] == 0, (name, r)
        assert r["lds"] <= 160 * 1024, (name, r)
    for name, r in ks.items():
        assert r["spill"] == 0, (name, r)


def test_adamw_side_kernel_fits_beside_two_gemm_waves(tmp_path):
    ks = _kernels("elementwise.hip", tmp_path)
    claim = [r for n, r in ks.items() if "k_adamw_claim" in n]
    assert claim, sorted(ks)
    for r in claim:
        assert r["vgpr"] + r["agpr"] <= 512 - 2 * 216, r
