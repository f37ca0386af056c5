"""The allocation-free step (muon_adamw_step_noalloc) against the step with
a caller-owned workspace (muon_adamw_step), through the C ABI on the GPU.

Two calls in a row on one GPU, the second with a smaller parameter table
(the scratch then holds the first call's data), each compared bit for bit
with muon_adamw_step on identical inputs: both run the same kernels, and
each matrix's phases in the same order, so every output must be equal.
Both Newton-Schulz precisions; two steps per table.  A captured call is
refused.
"""

import numpy as np
import pytest

import workloads as W
from tests import _harness as H

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
M = pytest.importorskip("muon_newton_schulz_02_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    M.load_library()
    yield
    torch.cuda.synchronize()


def _small(w):
    """The first action-expert layer's matrices, two norms and a bias of the
    tiny hybrid table: a smaller table than the whole one."""
    keep = [p for p in w.params
            if p.name.startswith("action_expert.layers.0.") or "embed" in p.name][:9]
    return W.Workload(w.name + "_small", seed=w.seed + 1, steps=2, ns_precision=w.ns_precision,
                      params=keep, grad_std=w.grad_std)


def _outputs(run):
    st = run.state
    return [H.host(x).copy() for x in run.params + st.muon_momentum + st.adam_m + st.adam_v +
            run.deltas + [run.norm_out] if x is not None]


def _steps(w, prec, noalloc):
    hp = H.oracle_hparams(w)
    run = H.setup_gpu(M, torch, w, hp, prec)
    for t in (1, 2):
        H.fill_grads(run, torch, t)
        H.say("%s %s noalloc=%s step %d" % (w.name, prec, noalloc, t))
        if noalloc:
            M.muon_adamw_step_noalloc(run.plan, run.params, run.grads, run.state, run.hp,
                                      grad_norm_out=run.norm_out, muon_update_out=run.deltas)
        else:
            M.muon_adamw_step(run.plan, run.params, run.grads, run.state, run.hp, run.workspace,
                              grad_norm_out=run.norm_out, muon_update_out=run.deltas)
        torch.cuda.synchronize()
    assert run.state.step == 2
    need = M.muon_adamw_workspace_size(run.plan, run.hp.ns_precision)
    return _outputs(run), need


@pytest.mark.parametrize("prec", ["fp32", "bf16"])
def test_noalloc_matches_workspace_step_on_two_tables(prec):
    big = W.tiny_hybrid_fp32()
    small = _small(big)
    sizes = []
    for w in (big, small):
        want, need = _steps(w, prec, noalloc=False)
        got, _ = _steps(w, prec, noalloc=True)
        sizes.append(need)
        assert need <= M.MA_NOALLOC_SCRATCH_BYTES
        assert len(got) == len(want)
        for k, (a, b) in enumerate(zip(got, want)):
            assert np.array_equal(a, b), "%s %s: output %d differs (max |diff| %g)" % (
                w.name, prec, k, float(np.max(np.abs(a.astype(np.float64) - b.astype(np.float64)))))
    assert sizes[1] < sizes[0]


def test_noalloc_refuses_capture():
    w = _small(W.tiny_hybrid_fp32())
    hp = H.oracle_hparams(w)
    run = H.setup_gpu(M, torch, w, hp, "bf16")
    run.state.device_step = torch.zeros(1, dtype=torch.int64, device="cuda")
    H.fill_grads(run, torch, 1)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with pytest.raises(M.MuonAdamWError) as e:
        with torch.cuda.graph(g):
            M.muon_adamw_step_noalloc(run.plan, run.params, run.grads, run.state, run.hp)
    assert e.value.code == M.MA_ERR_CAPTURE
    torch.cuda.synchronize()
    assert int(run.state.device_step.item()) == 0
