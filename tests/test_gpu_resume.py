"""Resume equivalence (checkpoint/resume of the optimizer state).

The optimizer state is caller-owned: parameters, Muon momentum, AdamW
moments and the step counter (host or device).  A run that saves them to host
memory after two steps and continues in a fresh plan, workspace and set of
tensors loaded from that copy must give, bit for bit, what four
uninterrupted steps give.  The workspace carries nothing from one step to
the next.
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


def _workload(storage):
    w = H.ragged_workload()
    w.param_storage = storage
    w.params.append(W.ParamSpec("vlm.model.layers.0.mlp.up_proj.weight", (512, 300)))
    return w


def _run(w, hp, prec, overlap, counter):
    run = H.setup_gpu(M, torch, w, hp, prec, overlap=overlap)
    if counter == "device":
        run.state.device_step = torch.zeros(1, dtype=torch.int64, device="cuda")
    return run


def _step(run, t):
    H.fill_grads(run, torch, t)
    H.gpu_step(M, torch, run)


def _save(run):
    """What a checkpoint holds: every caller-owned tensor, copied to host
    memory bit for bit (bf16 stays bf16), and the step counter."""
    cpu = lambda xs: [None if x is None else x.detach().cpu().clone() for x in xs]
    st = run.state
    step = int(st.device_step.item()) if st.device_step is not None else st.step
    return dict(params=cpu(run.params), mom=cpu(st.muon_momentum), m=cpu(st.adam_m),
                v=cpu(st.adam_v), step=step)


def _load(run, ck):
    for dst, src in ((run.params, ck["params"]), (run.state.muon_momentum, ck["mom"]),
                     (run.state.adam_m, ck["m"]), (run.state.adam_v, ck["v"])):
        for d, s in zip(dst, src):
            if d is not None:
                d.copy_(s.to(d.device))
    if run.state.device_step is not None:
        run.state.device_step.fill_(ck["step"])
    else:
        run.state.step = ck["step"]
    torch.cuda.synchronize()


def _outputs(run):
    st = run.state
    return [H.host(x).copy() for x in run.params + st.muon_momentum + st.adam_m + st.adam_v +
            run.deltas + [run.norm_out] if x is not None]


@pytest.mark.parametrize("prec,overlap,storage,counter", [
    ("bf16", False, "fp32", "host"), ("bf16", True, "fp32", "device"),
    ("fp32", False, "fp32", "device"), ("bf16", True, "bf16", "host")])
def test_resume_from_saved_state_is_bitwise(prec, overlap, storage, counter):
    """Four steps of a cosine schedule with warmup (so the step number
    matters at every step) against two steps, a save to host memory, a fresh
    plan/workspace/tensors loaded from it, and two more steps."""
    w = _workload(storage)
    hp = H.oracle_hparams(w, lr_schedule="cosine_with_min_lr", warmup_steps=1, total_steps=5)
    ref = _run(w, hp, prec, overlap, counter)
    for t in range(1, 5):
        H.say("resume ref prec=%s overlap=%s storage=%s counter=%s step %d"
              % (prec, overlap, storage, counter, t))
        _step(ref, t)
    want = _outputs(ref)
    del ref
    first = _run(w, hp, prec, overlap, counter)
    for t in (1, 2):
        H.say("resume first half step %d" % t)
        _step(first, t)
    ck = _save(first)
    assert ck["step"] == 2
    del first
    torch.cuda.empty_cache()
    second = _run(w, hp, prec, overlap, counter)
    _load(second, ck)
    for t in (3, 4):
        H.say("resume second half step %d" % t)
        _step(second, t)
    got = _outputs(second)
    assert len(got) == len(want)
    for k, (a, b) in enumerate(zip(got, want)):
        assert np.array_equal(a, b), "tensor %d differs after resume (max |diff| %g)" % (
            k, float(np.max(np.abs(a.astype(np.float64) - b.astype(np.float64)))))
    if counter == "host":
        assert second.state.step == 4
    else:
        assert int(second.state.device_step.item()) == 4
