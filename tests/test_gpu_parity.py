"""GPU parity of the HIP MuonAdamW step against the CPU oracle.

Each test seeds the same inputs for both sides (workloads module), runs the
GPU path through the C ABI and the oracle independently for several steps,
and compares after every step (tolerances in tests/_harness.py).  Sizes span
several GEMM tiles with ragged tails; the full-size workloads run in the
launch configuration the benchmark times and are compared on sampled
tensors, since the oracle cannot afford every matrix.
"""

import math
from dataclasses import replace

import numpy as np
import pytest

import oracle as O
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


def _run_parity(w, ns_precision, steps, hp=None, sampled=None, backend="numpy",
                check_params=True, say_every=1, overlap=False, prepare=None):
    """Run `steps` steps on both sides; compare the whole table (or only the
    entries in `sampled`).

    With bf16 parameter storage a parameter rounds to one of two bfloat16
    neighbours where the unrounded value lies near their midpoint, and a
    one-spacing difference would then persist; so each step starts the
    oracle from the GPU's parameters of the step before (states, which do
    not depend on the parameters, keep their own trajectories), and the
    parameters are checked against the rounding window of the gate."""
    hp = hp or H.oracle_hparams(w)
    bf16 = w.param_storage == "bf16"
    assert hp.param_storage == w.param_storage
    tol = H.BF16_TOL if ns_precision == "bf16" else H.FP32_TOL
    deltas = "all" if sampled is None else set(sampled)
    run = H.setup_gpu(M, torch, w, hp, ns_precision, backend, deltas=deltas, overlap=overlap)
    if prepare is not None:
        prepare(run)
    idx = range(len(w.params)) if sampled is None else sorted(sampled)
    # oracle-side state of the compared entries, from the same seeded inputs
    op, obuf, om, ov, omabs = {}, {}, {}, {}, {}
    for i in idx:
        if run.groups[i] == O.NONE:
            continue
        op[i] = H.host(run.params[i]).copy()
        if run.groups[i] == O.MUON:
            obuf[i] = H.host(run.state.muon_momentum[i]).copy()
        else:
            om[i] = np.zeros(w.params[i].shape, np.float32)
            ov[i] = np.zeros(w.params[i].shape, np.float32)
            omabs[i] = np.zeros(w.params[i].shape, np.float64)
    worst = 0.0
    errs = []
    for t in range(1, steps + 1):
        H.say("%s ns=%s step %d: inputs" % (w.name, ns_precision, t))
        H.fill_grads(run, torch, t, backend)
        torch.cuda.synchronize()
        H.say("%s step %d: oracle norm" % (w.name, t))
        norm = H.oracle_norm_of_device_grads(run)
        coef = O.clip_coefficient(norm, hp.max_grad_norm)
        if bf16:
            for i in op:
                op[i] = H.host(run.params[i]).copy()
        H.say("%s step %d: gpu step" % (w.name, t))
        H.gpu_step(M, torch, run)
        gnorm = float(H.host(run.norm_out)[0])
        assert abs(gnorm - norm) <= 1e-5 * norm, (gnorm, norm)
        assert run.state.step == t
        H.say("%s step %d: oracle updates (norm %.6g)" % (w.name, t, norm))
        hp_t = replace(hp, lr=O.scheduled_lr(hp, t))  # this step's scheduled rate
        for i in idx:
            g = run.groups[i]
            if g == O.NONE:
                continue
            grad = H.host(run.grads[i])
            if g == O.ADAMW:
                p, m, v = O.adamw_update(op[i], grad, om[i], ov[i], t, coef, hp_t)
                omabs[i] = hp.beta1 * omabs[i] + (1 - hp.beta1) * np.abs(coef * grad.astype(np.float64))
                where = "%s[%d] step %d" % (w.name, i, t)
                if bf16:
                    p32, _, _ = O.adamw_update(op[i], grad, om[i], ov[i], t, coef,
                                               replace(hp_t, param_storage="fp32"))
                    same = H.check_adamw_bf16(H.host(run.params[i]), H.host(run.state.adam_m[i]),
                                              H.host(run.state.adam_v[i]), p32, m, v, p, where,
                                              m_terms=omabs[i])
                    assert same >= 0.98, "%s: only %.4f of p equal the oracle's" % (where, same)
                else:
                    H.check_adamw(H.host(run.params[i]), H.host(run.state.adam_m[i]),
                                  H.host(run.state.adam_v[i]), p, m, v, where, m_terms=omabs[i])
                op[i], om[i], ov[i] = p, m, v
            else:
                m_, n_ = w.params[i].shape
                if m_ * n_ >= (1 << 24):
                    H.say("  oracle NS of %s %dx%d" % (w.names[i], m_, n_))
                scale = O.lr_shape_scale(m_, n_, hp.moonlight_coefficient)
                p, buf, delta = O.muon_matrix_update(op[i], grad, obuf[i], coef, hp_t, scale)
                gbuf = H.host(run.state.muon_momentum[i])
                np.testing.assert_allclose(gbuf, buf, rtol=1e-5, atol=1e-7 * (np.abs(buf).max() + 1e-30))
                err = H.rel_fro(H.host(run.deltas[i]), delta)
                worst = max(worst, err)
                errs.append(err)
                assert err <= tol, "%s[%d] %s step %d: delta rel err %.3g > %.1g" % (
                    w.name, i, w.params[i].shape, t, err, tol)
                if check_params and bf16:
                    # p = RNE_bf16(p_before - delta) in float32, with the delta the
                    # GPU reports (gated above); Muon decay 0 makes it exact
                    assert hp.muon_weight_decay == 0.0
                    gd = H.host(run.deltas[i])
                    want = O.bf16_round((op[i] - gd).astype(np.float32))
                    np.testing.assert_array_equal(H.host(run.params[i]), want)
                elif check_params:
                    gp = H.host(run.params[i]).astype(np.float64)
                    # parameter error = update error + one fp32 rounding per step
                    slack = t * (tol * np.linalg.norm(delta) + 6e-8 * np.linalg.norm(p)) + 1e-30
                    assert np.linalg.norm(gp - p.astype(np.float64)) <= 2 * slack
                op[i], obuf[i] = p, buf
        H.say("%s step %d ok (worst muon rel err %.3g)" % (w.name, t, worst))
    if errs:
        H.say("%s ns=%s: Muon update rel err over %d matrix-steps: max %.3g, median %.3g"
              % (w.name, ns_precision, len(errs), max(errs), float(np.median(errs))))
    return worst


def test_tiny_hybrid_fp32_all_entries():
    """14 Muon matrices (256..1024, both orientations) + 13 AdamW tensors,
    fp32 NS, 3 steps, every entry compared."""
    _run_parity(W.tiny_hybrid_fp32(), "fp32", 3)


@pytest.mark.parametrize("prec", ["fp32", "bf16"])
def test_small_matrix_tiles(prec):
    """Matrices of at most 256 rows after orientation, in both stored
    orientations, from 1 x 1 up to reductions of 4352 padded columns: under
    fp32 every one runs on the 32 x 32 small tiles with the four-way split
    reduction; under bf16 the thin ones (fewer than 16 rows) do, beside bf16
    matrices on the large tiles.  3 steps, every entry compared."""
    shapes = [(1, 1), (2, 300), (300, 2), (31, 33), (200, 4100), (4100, 200), (256, 256),
              (255, 1024), (1024, 255), (64, 256), (17, 17), (7, 2000)]
    params = [W.ParamSpec("action_expert.layers.%d.s.weight" % i, sh)
              for i, sh in enumerate(shapes)]
    params += [W.ParamSpec("vlm.norm", (300,))]
    w = W.Workload("small_tiles_" + prec, seed=13, steps=3, ns_precision=prec, params=params,
                   grad_std=1e-3)
    _run_parity(w, prec, 3)


_ragged_workload = H.ragged_workload


@pytest.mark.parametrize("prec,steps", [("bf16", 5), ("fp32", 5), ("bf16", 1), ("fp32", 2)])
def test_ragged_shapes(prec, steps):
    """Ragged Muon shapes (1xn, nx1, odd sizes around tile edges, both
    orientations) and odd AdamW sizes (tails of a chunk, non-multiples of 4),
    with 1, 2 and 5 NS steps."""
    w = _ragged_workload()
    hp = H.oracle_hparams(w, ns_steps=steps)
    _run_parity(w, prec, 2, hp=hp)


def test_ragged_published_coefficients_no_nesterov_with_decay():
    w = _ragged_workload()
    hp = H.oracle_hparams(w, ns_coeffs=O.PUBLISHED_NS_COEFFS, muon_nesterov=False,
                          muon_weight_decay=0.1, lr=1e-3, max_grad_norm=0.0)
    _run_parity(w, "fp32", 2, hp=hp)


@pytest.mark.parametrize("prec", ["bf16", "fp32"])
def test_ragged_cubic_coefficients(prec):
    """c = 0 (the classic cubic iteration 1.5 X - 0.5 X X^T X): the polynomial
    step reduces to B = b A, which the bf16 kernels cannot fold into the
    product's accumulators and take from the A operand in the epilogue."""
    w = _ragged_workload()
    hp = H.oracle_hparams(w, ns_coeffs=(1.5, -0.5, 0.0))
    _run_parity(w, prec, 2, hp=hp)


@pytest.mark.parametrize("std,clip,prec", [(1e-20, 1.0, "bf16"), (1e-20, 1.0, "fp32"),
                                           (1e-9, 1.0, "bf16"), (1e15, 0.0, "bf16"),
                                           (1e15, 0.0, "fp32")])
def test_extreme_gradient_scales(std, clip, prec):
    """Muon matrices whose momentum direction u has a Frobenius norm far from
    1.  The GPU path writes u unnormalised as the Newton-Schulz input and
    applies 1 / (||u|| + eps) in the first Gram and X-update epilogues; for a
    norm outside [2^-40, 2^40] (here ~1e-17 and ~1e18) it scales the operands
    themselves first, so products stay inside the fp32 range.  Both paths
    must match the oracle, which normalises before iterating."""
    shapes = [(1, 7), (33, 65), (65, 33), (300, 130), (257, 513), (3, 1000), (129, 129)]
    params = [W.ParamSpec("action_expert.layers.%d.x.weight" % i, s) for i, s in enumerate(shapes)]
    w = W.Workload("extreme_%g" % std, seed=11, steps=2, ns_precision=prec, params=params,
                   grad_std=std)
    hp = H.oracle_hparams(w, max_grad_norm=clip)
    _run_parity(w, prec, 2, hp=hp)


@pytest.mark.parametrize("prec", ["bf16", "fp32"])
def test_cosine_schedule(prec):
    """The defaults table's cosine_with_min_lr (min_lr_rate 0.1) over five
    steps of a 4-step schedule with one warmup step: the rates are 0 (warmup
    start), the base rate, two points down the cosine and the minimum held
    past the end, for both groups."""
    w = _ragged_workload()
    hp = H.oracle_hparams(w, lr_schedule="cosine_with_min_lr", warmup_steps=1, total_steps=4,
                          lr=1e-3)
    assert [O.schedule_factor(hp, k) for k in range(5)] == pytest.approx(
        [0.0, 1.0, 0.775, 0.325, 0.1])
    _run_parity(w, prec, 5, hp=hp)


def test_adamw_mode_and_misaligned_views():
    """Plain-AdamW mode sends every trainable tensor through the AdamW kernel;
    a view starting one float into its storage takes the scalar path."""
    dev = torch.device("cuda", 0)
    table = [("action_expert.layers.0.q.weight", (64, 48), True),
             ("vlm.x", (1000,), True), ("vlm.y", (20001,), True)]
    plan = M.muon_adamw_plan(table, mode=M.MA_MODE_ADAMW)
    assert all(M.muon_adamw_plan_entry(plan, i)["group"] == M.MA_GROUP_ADAMW for i in range(3))
    rng = np.random.default_rng(3)
    store = torch.zeros(20002, device=dev)
    p_host = [rng.standard_normal(s).astype(np.float32) * np.float32(0.02) for _, s, _ in table]
    params = [torch.from_numpy(p_host[0]).to(dev), torch.from_numpy(p_host[1]).to(dev), store[1:]]
    params[2].copy_(torch.from_numpy(p_host[2]))
    assert params[2].data_ptr() % 16 == 4
    st = M.State(3)
    for i, (_, s, _) in enumerate(table):
        st.adam_m[i] = torch.zeros(s, device=dev)
        st.adam_v[i] = torch.zeros(s, device=dev)
    hp = O.HParams()
    lhp = H.lib_hparams(M, hp, "bf16")
    ws = torch.empty(M.muon_adamw_workspace_size(plan, 0), dtype=torch.uint8, device=dev)
    om = [np.zeros(s, np.float32) for _, s, _ in table]
    ov = [np.zeros(s, np.float32) for _, s, _ in table]
    op = [p.copy() for p in p_host]
    mabs = [np.zeros(s, np.float64) for _, s, _ in table]
    for t in (1, 2, 3):
        g_host = [rng.standard_normal(s).astype(np.float32) * np.float32(0.05) for _, s, _ in table]
        grads = [torch.from_numpy(g).to(dev) for g in g_host]
        H.say("adamw mode step", t)
        M.muon_adamw_step(plan, params, grads, st, lhp, ws)
        torch.cuda.synchronize()
        coef = O.clip_coefficient(O.global_grad_norm(g_host), hp.max_grad_norm)
        for i in range(3):
            mabs[i] = hp.beta1 * mabs[i] + (1 - hp.beta1) * np.abs(coef * g_host[i].astype(np.float64))
            op[i], om[i], ov[i] = O.adamw_update(op[i], g_host[i], om[i], ov[i], t, coef, hp)
            H.check_adamw(H.host(params[i]), H.host(st.adam_m[i]), H.host(st.adam_v[i]),
                          op[i], om[i], ov[i], "adamw-mode[%d] step %d" % (i, t), m_terms=mabs[i])
    assert float(store[0]) == 0.0


@pytest.mark.filterwarnings("ignore:invalid value encountered")
@pytest.mark.parametrize("kind", ["nan_in_adamw", "inf_in_muon"])
def test_non_finite_gradients_propagate(kind):
    """Non-finite gradients are not skipped: a NaN makes the global norm and
    the clip factor NaN, so every updated tensor turns NaN; an infinity makes
    the norm infinite and the factor 0, so the infinite element turns NaN
    (0 * inf), its matrix's whole update turns NaN through Newton-Schulz,
    and the rest is updated with a zero gradient.  The NaN pattern of every
    tensor equals the oracle's; finite values pass the usual gates."""
    w = _ragged_workload()
    hp = H.oracle_hparams(w)
    run = H.setup_gpu(M, torch, w, hp, "bf16")
    H.fill_grads(run, torch, 1)
    names = w.names
    if kind == "nan_in_adamw":
        run.grads[names.index("vlm.big")][7] = float("nan")
    else:
        run.grads[names.index("action_expert.layers.4.r.weight")][3, 5] = float("inf")
    torch.cuda.synchronize()
    p0 = [None if p is None else H.host(p).copy() for p in run.params]
    b0 = [None if b is None else H.host(b).copy() for b in run.state.muon_momentum]
    g0 = [None if g is None else H.host(g).copy() for g in run.grads]
    z = [None if p is None else np.zeros_like(p) for p in p0]
    H.say("non-finite gradients: %s" % kind)
    H.gpu_step(M, torch, run)
    res = O.optimizer_step(names, p0, g0, w.trainable, b0, z, z, 1, hp, groups=run.groups)
    gnorm = float(H.host(run.norm_out)[0])
    if kind == "nan_in_adamw":
        assert math.isnan(gnorm) and math.isnan(res.grad_norm)
    else:
        assert math.isinf(gnorm) and math.isinf(res.grad_norm) and res.clip_coef == 0.0
    for i, g in enumerate(run.groups):
        if g == O.NONE:
            continue
        pairs = [(H.host(run.params[i]), res.params[i])]
        if g == O.ADAMW:
            pairs += [(H.host(run.state.adam_m[i]), res.adam_m[i]),
                      (H.host(run.state.adam_v[i]), res.adam_v[i])]
        else:
            pairs += [(H.host(run.state.muon_momentum[i]), res.muon_momentum[i]),
                      (H.host(run.deltas[i]), res.deltas[i])]
        for k, (a, b) in enumerate(pairs):
            np.testing.assert_array_equal(np.isnan(a), np.isnan(b), "%s tensor %d" % (names[i], k))
            fin = ~np.isnan(b)
            if g == O.ADAMW or k < 2:
                np.testing.assert_allclose(a[fin], b[fin], rtol=1e-5, atol=1e-9)
            elif fin.all():
                assert H.rel_fro(a, b) <= H.BF16_TOL


def test_degenerate_tables():
    """Edge cases of the table: only frozen entries (the step launches the
    norm finaliser alone: norm 0, nothing else touched, the counter still
    advances); a 1 x 1 Muon matrix next to a one-element AdamW tensor, both
    against the oracle over two steps."""
    dev = torch.device("cuda", 0)
    plan = M.muon_adamw_plan([("vlm.model.embed_tokens.weight", (151, 20), False),
                              ("lm_head.weight", (151, 20), False)])
    st = M.State(2)
    hp = M.muon_adamw_default_hparams()
    ws = torch.empty(max(M.muon_adamw_workspace_size(plan, 0), 256), dtype=torch.uint8, device=dev)
    norm = torch.full((1,), 7.0, device=dev)
    H.say("all-frozen table")
    M.muon_adamw_step(plan, None, None, st, hp, ws, grad_norm_out=norm)
    torch.cuda.synchronize()
    assert float(norm[0]) == 0.0 and st.step == 1

    w = W.Workload("one_by_one", seed=5, steps=2, ns_precision="bf16", grad_std=1e-3,
                   params=[W.ParamSpec("action_expert.layers.0.x.weight", (1, 1)),
                           W.ParamSpec("vlm.scalar", (1,))])
    _run_parity(w, "bf16", 2)
    _run_parity(w, "fp32", 2)


def test_bitwise_deterministic_reruns():
    """Two runs from identical inputs give bit-identical parameters, states,
    deltas and norms (fixed reduction trees, no float atomics)."""
    w = _ragged_workload()
    hp = H.oracle_hparams(w)
    outs = []
    for rep in range(2):
        run = H.setup_gpu(M, torch, w, hp, "bf16")
        for t in (1, 2):
            H.fill_grads(run, torch, t)
            H.say("determinism rep %d step %d" % (rep, t))
            H.gpu_step(M, torch, run)
        outs.append([H.host(x) for x in run.params + run.deltas + run.state.muon_momentum +
                     run.state.adam_m + run.state.adam_v + [run.norm_out] if x is not None])
    for a, b in zip(*outs):
        np.testing.assert_array_equal(a, b)


def test_zero_gradients():
    """Degenerate input: all-zero gradients.  Norm 0, no clipping, Muon deltas
    exactly 0 (NS of the zero matrix), AdamW is pure decay."""
    w = _ragged_workload()
    hp = H.oracle_hparams(w)
    run = H.setup_gpu(M, torch, w, hp, "bf16")
    p0 = [None if p is None else H.host(p).copy() for p in run.params]
    for g in run.grads:
        if g is not None:
            g.zero_()
    H.say("zero gradients")
    H.gpu_step(M, torch, run)
    assert float(H.host(run.norm_out)[0]) == 0.0
    for i, grp in enumerate(run.groups):
        if grp == O.MUON:
            assert np.all(H.host(run.deltas[i]) == 0.0)
            np.testing.assert_array_equal(H.host(run.params[i]), p0[i])
        elif grp == O.ADAMW:
            np.testing.assert_allclose(H.host(run.params[i]), p0[i] * np.float32(1 - 2.5e-7),
                                       rtol=1e-7, atol=0)


def test_ae18_full_size_sampled():
    """The 18-layer action-expert Muon group at full size (126 matrices),
    bf16 NS, per-row-scaled gradients, 10 steps; the oracle follows one
    matrix of every shape (q 1024^2, k 256x1024, gate 4096x1024 transposed,
    down 1024x4096) and the global norm over all gradients."""
    w = W.ae18_muon_bf16()
    sampled = {0, 1, 4, 6 + 7 * 17}
    _run_parity(w, "bf16", w.steps, sampled=sampled, backend="torch")


@pytest.mark.parametrize("overlap", [True, False])
def test_vla_hybrid_full_size_sampled(overlap):
    """The full hybrid step in the benchmark's configuration: 126 Muon
    matrices (bf16 NS) + 253 AdamW tensors (1.88e9 elements) + a frozen
    embedding; clip triggers.  The oracle follows the global norm over all
    2.15e9 gradients, six AdamW tensors of every shape and four Muon
    matrices, over all five configured steps; AdamW beside the Muon group
    (the benchmark's launch, with Newton-Schulz in batches on two streams)
    and serial."""
    w = W.vla_hybrid_bf16()
    names = w.names
    pick = ["vlm.model.layers.0.self_attn.q_proj.weight", "vlm.model.layers.3.mlp.gate_proj.weight",
            "vlm.model.layers.27.mlp.down_proj.weight", "vlm.model.layers.13.input_layernorm.weight",
            "vlm.model.norm.weight", "vlm.model.layers.27.post_attention_layernorm.weight",
            "action_expert.layers.0.self_attn.q_proj.weight",
            "action_expert.layers.5.self_attn.k_proj.weight",
            "action_expert.layers.17.mlp.gate_proj.weight",
            "action_expert.layers.9.mlp.down_proj.weight"]
    sampled = {names.index(n) for n in pick}
    _run_parity(w, "bf16", w.steps, sampled=sampled, backend="torch", overlap=overlap)


def _bf16_ragged():
    w = _ragged_workload()
    w.name = "ragged_small_bf16store"
    w.param_storage = "bf16"
    w.params.append(W.ParamSpec("vlm.model.layers.0.mlp.up_proj.weight", (512, 300)))
    return w


@pytest.mark.parametrize("prec,overlap", [("bf16", False), ("bf16", True), ("fp32", False)])
def test_bf16_storage_ragged(prec, overlap):
    """bf16 parameter storage (the page's bf16_mixed policy): bf16
    parameters and gradients, float32 states.  Ragged shapes take the vector
    paths and the scalar tails of every kernel; AdamW in order or beside the
    Muon group; three steps."""
    _run_parity(_bf16_ragged(), prec, 3, overlap=overlap)


def test_bf16_storage_misaligned_views():
    """bf16 tensors that start 2 or 8 bytes into their storage: the norm,
    AdamW, Muon momentum and update kernels fall back to their narrower
    paths and give the same results."""
    w = _bf16_ragged()
    names = w.names
    shift = {"vlm.big": 1, "vlm.w": 4, "vlm.model.layers.0.mlp.up_proj.weight": 4,
             "action_expert.layers.6.r.weight": 4, "action_expert.layers.9.r.weight": 1}

    def prepare(run):
        for name, k in shift.items():
            i = names.index(name)
            for lst in (run.params, run.grads):
                t = lst[i]
                store = torch.zeros(t.numel() + k, dtype=t.dtype, device=t.device)
                view = store[k:].view(t.shape)
                view.copy_(t)
                assert view.data_ptr() % 16 == 2 * k
                lst[i] = view

    _run_parity(w, "bf16", 2, prepare=prepare)


def test_vla_bf16_mixed_full_size_sampled():
    """The full hybrid step with bf16 parameters and gradients (bf16_mixed):
    the global norm over all 2.15e9 bf16 gradients, six AdamW tensors and
    four Muon matrices followed for two steps."""
    w = W.vla_hybrid_bf16_mixed()
    names = w.names
    pick = ["vlm.model.layers.0.self_attn.q_proj.weight", "vlm.model.layers.3.mlp.gate_proj.weight",
            "vlm.model.layers.27.mlp.down_proj.weight", "vlm.model.layers.13.input_layernorm.weight",
            "vlm.model.norm.weight", "vlm.model.layers.27.post_attention_layernorm.weight",
            "action_expert.layers.0.self_attn.q_proj.weight",
            "action_expert.layers.5.self_attn.k_proj.weight",
            "action_expert.layers.17.mlp.gate_proj.weight",
            "action_expert.layers.9.mlp.down_proj.weight"]
    sampled = {names.index(n) for n in pick}
    _run_parity(w, "bf16", 2, sampled=sampled, backend="torch", overlap=True)


def test_rank_share_full_size_sampled():
    """One GPU's share of the hybrid step sharded over 8 GPUs by
    owner-compute (11 whole matrices by LPT, 1/8 of the AdamW elements as
    1-D pieces cut at arbitrary offsets), in the configuration the benchmark
    times; two steps."""
    w = W.vla_hybrid_share(0, 8)
    names = w.names
    pieces = [i for i, n in enumerate(names) if "[" in n]
    mats = [i for i, n in enumerate(names) if "[" not in n]
    sampled = {pieces[0], pieces[len(pieces) // 2], pieces[-1], mats[0], mats[-1]}
    _run_parity(w, "bf16", 2, sampled=sampled, backend="torch", overlap=True)


def test_vla_adamw_full_size_sampled():
    """The page's default optimizer (optim = adamw) over the full hybrid
    table: all 2.15e9 trainable elements through the clip and AdamW (the
    action-expert matrices included), under cosine_with_min_lr over 1000
    steps; the oracle follows the global norm and eight tensors of every
    kind for two steps."""
    w = W.vla_hybrid_adamw()
    names = w.names
    pick = ["vlm.model.layers.0.self_attn.q_proj.weight", "vlm.model.layers.9.mlp.up_proj.weight",
            "vlm.model.norm.weight", "vlm.model.layers.27.input_layernorm.weight",
            "action_expert.layers.0.self_attn.q_proj.weight",
            "action_expert.layers.3.self_attn.v_proj.weight",
            "action_expert.layers.17.mlp.gate_proj.weight",
            "action_expert.layers.8.mlp.down_proj.weight"]
    sampled = {names.index(n) for n in pick}
    _run_parity(w, "bf16", 2, sampled=sampled, backend="torch")


def test_overlapped_groups_match_serial_bitwise():
    """AdamW on the side stream (concurrent with the Muon group) gives the
    same bits as the serial order on one stream, over two steps."""
    w = _ragged_workload()
    w.params.append(W.ParamSpec("vlm.model.layers.0.mlp.up_proj.weight", (512, 300)))
    hp = H.oracle_hparams(w)
    outs = []
    for overlap in (False, True):
        run = H.setup_gpu(M, torch, w, hp, "bf16", overlap=overlap)
        for t in (1, 2):
            H.fill_grads(run, torch, t)
            H.say("overlap=%s step %d" % (overlap, t))
            H.gpu_step(M, torch, run)
        outs.append([H.host(x) for x in run.params + run.deltas + run.state.muon_momentum +
                     run.state.adam_m + run.state.adam_v + [run.norm_out] if x is not None])
    for a, b in zip(*outs):
        np.testing.assert_array_equal(a, b)


def _three_wide_matrices():
    # 3 x 134 MB of bf16 operands: three batches beside AdamW, the last one
    # without a partner on the other stream
    params = [W.ParamSpec("action_expert.layers.%d.mlp.up_proj.weight" % i, (8192, 4096))
              for i in range(3)]
    params.append(W.ParamSpec("vlm.model.norm.weight", (2048,)))
    return W.Workload("three_wide", seed=11, steps=1, ns_precision="bf16", params=params,
                      grad_std=1e-3)


def _ae18_plus_norm():
    w = W.ae18_muon_bf16()
    w.params.append(W.ParamSpec("vlm.model.norm.weight", (2048,)))
    return w


@pytest.mark.parametrize("make", [_ae18_plus_norm, _three_wide_matrices],
                         ids=["ae18_eight_batches", "three_batches"])
def test_batched_newton_schulz_matches_serial_bitwise(make):
    """Full-size Muon matrices plus one AdamW tensor: with the AdamW group
    beside them, Newton-Schulz runs in several batches over two streams
    (eight for the 126 action-expert matrices, an odd three for three
    8192 x 4096 ones); every Muon result equals the serial step's bit for
    bit."""
    w = make()
    hp = H.oracle_hparams(w)
    keys = [i for i, p in enumerate(w.params) if p.trainable]
    ref = None
    for overlap in (False, True):
        run = H.setup_gpu(M, torch, w, hp, "bf16", "torch", deltas="all", overlap=overlap)
        H.fill_grads(run, torch, 1, "torch")
        H.say("batched NS: overlap=%s step" % overlap)
        H.gpu_step(M, torch, run)
        got = [(H.host(run.params[i]).copy(), H.host(run.deltas[i]).copy()
                if run.deltas[i] is not None else None) for i in keys]
        del run
        torch.cuda.empty_cache()
        if ref is None:
            ref = got
            continue
        for i, (a, b) in zip(keys, zip(ref, got)):
            np.testing.assert_array_equal(a[0], b[0], err_msg=w.names[i])
            if a[1] is not None:
                np.testing.assert_array_equal(a[1], b[1], err_msg=w.names[i])


def test_vla_hybrid_fp32ns_full_size_sampled():
    """The full hybrid parameter set with the Newton-Schulz products in fp32
    (true fp32 MFMA): delta relative error <= 1e-4 per matrix and step, on
    four Muon matrices of every shape and four AdamW tensors, over all five
    configured steps."""
    w = W.vla_hybrid_fp32ns()
    names = w.names
    pick = ["vlm.model.layers.1.mlp.down_proj.weight", "vlm.model.layers.20.input_layernorm.weight",
            "vlm.model.norm.weight", "vlm.model.layers.7.self_attn.o_proj.weight",
            "action_expert.layers.2.self_attn.o_proj.weight",
            "action_expert.layers.11.self_attn.v_proj.weight",
            "action_expert.layers.4.mlp.up_proj.weight",
            "action_expert.layers.16.mlp.down_proj.weight"]
    sampled = {names.index(n) for n in pick}
    _run_parity(w, "fp32", w.steps, sampled=sampled, backend="torch")


def test_ragged_stress_noclip_full_size():
    """Large and ragged matrices in one grouped call, clip off so the rank-8
    spike (entry std 100) reaches Newton-Schulz ill-conditioned: every one of
    the 68 matrices (8192^2, 4096x14336, 14336x4096, 128x8192, 64 x 64x256)
    compared with the oracle after the first step, over preloaded momentum."""
    w = W.ragged_stress_bf16(clip=False)
    _run_parity(w, "bf16", 1, backend="torch")


def test_ragged_stress_noclip_three_steps_sampled():
    """Clip off, all three configured steps, with the momentum carried
    forward: the 8192^2 matrix (60 % of the workload's flops), the tall and
    wide 4096/14336 pair, the 128x8192 matrix and three of the 64x256 ones
    compared at every step."""
    w = W.ragged_stress_bf16(clip=False)
    _run_parity(w, "bf16", w.steps, sampled={0, 1, 2, 3, 4, 30, 67}, backend="torch")


def test_ragged_stress_clip_full_size_sampled():
    """The same workload with the clip on (it triggers: the spike makes the
    norm ~1e5), three steps, on the 8192^2 matrix, the tall and wide
    4096/14336 pair, the 128x8192 matrix and four of the 64x256 ones."""
    w = W.ragged_stress_bf16(clip=True)
    _run_parity(w, "bf16", w.steps, sampled={0, 1, 2, 3, 4, 30, 50, 67}, backend="torch")
