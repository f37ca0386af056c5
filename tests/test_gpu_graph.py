"""Device-resident step counter and graph capture of the whole step.

With state.device_step set, every value that depends on the step number (the
scheduled rate, AdamW's bias corrections and decays, the Muon rate) is formed
on the GPU; a captured step reads the descriptor tables the last eager step
put in the workspace, so a step captured once replays as the following
steps.  These
tests compare bit for bit: the device-counter path with the host-counter path
(which the parity tests check against the oracle), and graph replays with
eager steps on identical inputs.
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


def _workload(storage="fp32"):
    w = H.ragged_workload()
    w.param_storage = storage
    # an AdamW matrix large enough that the overlapped launch has chunks to claim
    w.params.append(W.ParamSpec("vlm.model.layers.0.mlp.up_proj.weight", (512, 300)))
    return w


def _hparams(w):
    # a schedule whose rate changes at every step checked here
    return H.oracle_hparams(w, lr_schedule="cosine_with_min_lr", warmup_steps=1, total_steps=4)


def _setup(w, hp, overlap, device_counter):
    run = H.setup_gpu(M, torch, w, hp, "bf16", overlap=overlap)
    if device_counter:
        run.state.device_step = torch.zeros(1, dtype=torch.int64, device="cuda")
    return run


def _snapshot(run):
    return [H.host(x).copy() for x in run.params + run.deltas + run.state.muon_momentum +
            run.state.adam_m + run.state.adam_v + [run.norm_out] if x is not None]


def _assert_same(a, b, where):
    assert len(a) == len(b)
    for k, (x, y) in enumerate(zip(a, b)):
        assert np.array_equal(x, y), "%s: tensor %d differs (max |diff| %g)" % (
            where, k, float(np.max(np.abs(x.astype(np.float64) - y.astype(np.float64)))))


def _step(run):
    M.muon_adamw_step(run.plan, run.params, run.grads, run.state, run.hp, run.workspace,
                      grad_norm_out=run.norm_out, muon_update_out=run.deltas)


@pytest.mark.parametrize("overlap", [False, True])
def test_device_counter_matches_host_counter_bitwise(overlap):
    """Four scheduled steps (warmup, cosine, held at the floor) give the same
    bits with the step number on the device as with it on the host; the
    device counter ends at 4 and the host counter is left alone."""
    w = _workload()
    hp = _hparams(w)
    outs = []
    for dev_counter in (False, True):
        run = _setup(w, hp, overlap, dev_counter)
        snaps = []
        for t in range(1, 5):
            H.fill_grads(run, torch, t)
            H.say("device counter=%s overlap=%s step %d" % (dev_counter, overlap, t))
            _step(run)
            torch.cuda.synchronize()
            snaps.append(_snapshot(run))
        if dev_counter:
            assert int(run.state.device_step.item()) == 4
            assert run.state.step == 0
        else:
            assert run.state.step == 4
        outs.append(snaps)
    for t, (a, b) in enumerate(zip(*outs), start=1):
        _assert_same(a, b, "step %d" % t)


def test_eager_steps_reupload_after_the_workspace_was_overwritten():
    """The workspace is scratch between eager steps: with the device counter
    set, a caller that overwrites it (or frees it and gets the same memory
    back from the caching allocator holding other data) between two eager
    steps still gets exactly the results of an untouched workspace, since
    every eager step uploads its descriptor tables again."""
    w = _workload()
    hp = _hparams(w)
    outs = []
    for clobber in (False, True):
        run = _setup(w, hp, False, True)
        snaps = []
        for t in range(1, 4):
            H.fill_grads(run, torch, t)
            if clobber and t > 1:
                run.workspace.fill_(0xA5)      # garbage where the tables were
                torch.cuda.synchronize()
            H.say("workspace clobber=%s step %d" % (clobber, t))
            _step(run)
            torch.cuda.synchronize()
            snaps.append(_snapshot(run))
        outs.append(snaps)
    for t, (a, b) in enumerate(zip(*outs), start=1):
        _assert_same(a, b, "step %d" % t)


@pytest.mark.parametrize("overlap,storage", [(False, "fp32"), (True, "fp32"), (True, "bf16")])
def test_graph_replays_match_eager_steps(overlap, storage):
    """Step 1 eager, then one step captured in a graph and replayed as steps
    2..5, with eager work (new gradients, unrelated kernels, host syncs)
    between replays: after every replay the state equals that of eager steps
    on the same inputs, bit for bit (float32 or bfloat16 parameters)."""
    w = _workload(storage)
    hp = _hparams(w)
    eager = _setup(w, hp, overlap, True)
    ref = []
    for t in range(1, 6):
        H.fill_grads(eager, torch, t)
        H.say("eager overlap=%s step %d" % (overlap, t))
        _step(eager)
        torch.cuda.synchronize()
        ref.append(_snapshot(eager))

    run = _setup(w, hp, overlap, True)
    H.fill_grads(run, torch, 1)
    H.say("graph run overlap=%s: eager step 1" % overlap)
    _step(run)
    torch.cuda.synchronize()
    _assert_same(_snapshot(run), ref[0], "eager step 1")

    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    H.say("graph run overlap=%s: capture" % overlap)
    with torch.cuda.graph(g, stream=cap):
        _step(run)
    torch.cuda.synchronize()
    # capturing ran nothing: state and counter are still those of step 1
    assert int(run.state.device_step.item()) == 1
    _assert_same(_snapshot(run), ref[0], "after capture")

    junk = torch.randn(1 << 20, device="cuda")
    for t in range(2, 6):
        H.fill_grads(run, torch, t)
        junk.mul_(0.5).add_(1.0)  # unrelated eager work between replays
        torch.cuda.synchronize()
        H.say("graph run overlap=%s: replay as step %d" % (overlap, t))
        g.replay()
        torch.cuda.synchronize()
        assert int(run.state.device_step.item()) == t
        _assert_same(_snapshot(run), ref[t - 1], "replay as step %d" % t)
    del g


@pytest.mark.filterwarnings("ignore:The CUDA Graph is empty")
def test_capture_without_device_counter_is_refused():
    """A captured step with the host counter would replay a frozen step
    number: the library refuses it before recording anything."""
    w = _workload()
    hp = _hparams(w)
    run = _setup(w, hp, False, False)
    H.fill_grads(run, torch, 1)
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    code = None
    H.say("capture with the host counter")
    with torch.cuda.graph(g, stream=cap):
        try:
            _step(run)
        except M.MuonAdamWError as e:
            code = e.code
    torch.cuda.synchronize()
    assert code == M.MA_ERR_CAPTURE
    assert run.state.step == 0


@pytest.mark.filterwarnings("ignore:The CUDA Graph is empty")
def test_capture_needing_new_tables_is_refused():
    """Capturing a step whose pointers differ from the last eager step's
    (here: no eager step at all) would record a host upload; refused."""
    w = _workload()
    hp = _hparams(w)
    run = _setup(w, hp, False, True)
    H.fill_grads(run, torch, 1)
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    code = None
    H.say("capture before any eager step")
    with torch.cuda.graph(g, stream=cap):
        try:
            _step(run)
        except M.MuonAdamWError as e:
            code = e.code
    torch.cuda.synchronize()
    assert code == M.MA_ERR_CAPTURE
    assert int(run.state.device_step.item()) == 0


def test_graph_replays_with_batched_newton_schulz():
    """The 126 full-size action-expert matrices plus one AdamW tensor, AdamW
    beside the Muon group: Newton-Schulz runs as several batches over two
    streams, all forked from and joined into the captured stream.  Replays
    equal eager steps bit for bit."""
    w = W.ae18_muon_bf16()
    w.params.append(W.ParamSpec("vlm.model.norm.weight", (2048,)))
    hp = _hparams(w)

    def setup():
        run = H.setup_gpu(M, torch, w, hp, "bf16", "torch", deltas="none", overlap=True)
        run.state.device_step = torch.zeros(1, dtype=torch.int64, device="cuda")
        return run

    def snap(run):
        return [H.host(x).copy() for x in run.params + run.state.muon_momentum +
                run.state.adam_m + run.state.adam_v + [run.norm_out] if x is not None]

    eager = setup()
    ref = []
    for t in (1, 2, 3):
        H.fill_grads(eager, torch, t, "torch")
        H.say("batched NS eager step %d" % t)
        _step(eager)
        torch.cuda.synchronize()
        ref.append(snap(eager))
    del eager
    torch.cuda.empty_cache()

    run = setup()
    H.fill_grads(run, torch, 1, "torch")
    H.say("batched NS graph run: eager step 1")
    _step(run)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    H.say("batched NS graph run: capture")
    with torch.cuda.graph(g, stream=cap):
        _step(run)
    torch.cuda.synchronize()
    for t in (2, 3):
        H.fill_grads(run, torch, t, "torch")
        torch.cuda.synchronize()
        H.say("batched NS graph run: replay as step %d" % t)
        g.replay()
        torch.cuda.synchronize()
        assert int(run.state.device_step.item()) == t
        _assert_same(snap(run), ref[t - 1], "replay as step %d" % t)
    del g
