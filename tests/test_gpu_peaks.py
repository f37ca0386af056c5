"""The ceiling probes the benchmark reports beside its rates (csrc/peaks.hip
through muon_newton_schulz_02_amd/peaks.py) run on the GPU and return
plausible figures: positive, the matrix-core rates below the datasheet
peaks, and the copy into LDS faster from L2 than from beyond it.  Small
launches (arrays of 256 MiB may partly stay in the memory-side cache, so the
stream rates are not bounded by the HBM peak here): this checks that the
probes work, it does not measure."""

import math

import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from muon_newton_schulz_02_amd import peaks
    peaks.load()
    return torch, peaks


def _ok(x):
    return isinstance(x, float) and math.isfinite(x) and x > 0.0


def test_mfma_and_lds_probes(env):
    torch, peaks = env
    bf = peaks.mfma(torch, False, iters=2000, reps=1)
    f32 = peaks.mfma(torch, True, iters=1000, reps=1)
    assert _ok(bf["tflops"]) and bf["tflops"] < 2600.0, bf
    assert _ok(f32["tflops"]) and f32["tflops"] < 170.0, f32
    assert 500.0 < bf["sclk_mhz"] < 3000.0, bf
    for tr in (False, True):
        r = peaks.lds(torch, tr, iters=200, reps=1)
        assert _ok(r["gbps"]) and _ok(r["bytes_per_clk_per_cu"]), r


def test_stream_and_dma_probes(env):
    torch, peaks = env
    for kind in ("read", "copy", "adamw_mix"):
        r = peaks.stream(torch, kind, 0.25, reps=1)
        assert _ok(r["gbps"]), (kind, r)
    near = peaks.dma(torch, 4, stages=256, reps=1)
    far = peaks.dma(torch, 256, stages=256, reps=1)
    for r in (near, far):
        assert _ok(r["gbps"]) and _ok(r["bytes_per_clk_per_cu"]), r
    assert near["gbps"] > far["gbps"], (near, far)
