"""Pins of the CPU oracle to facts fixed outside the oracle itself.

Each test names what pins it: a closed form, an invariant, a special case that
reduces to a library routine, brute force on tiny inputs (SVD), or a value the
OpenDM training-stack page states.  Chosen so that a dropped term, a wrong
sign, index or coefficient, or a transposed operand in the oracle fails one.
"""

import math
import os

import numpy as np
import pytest

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _phi(s, coeffs, k):
    """k-fold composition of the scalar quintic s -> a s + b s^3 + c s^5."""
    a, b, c = coeffs
    for _ in range(k):
        s = a * s + b * s ** 3 + c * s ** 5
    return s


# --------------------------------------------------------------------------
# Newton-Schulz
# --------------------------------------------------------------------------

@pytest.mark.parametrize("coeffs", [O.DEFAULT_NS_COEFFS, O.PUBLISHED_NS_COEFFS])
@pytest.mark.parametrize("shape", [(5, 9), (9, 5), (7, 7), (1, 6), (6, 1), (16, 64), (40, 24)])
def test_ns_equals_svd_spectral_map(shape, coeffs):
    """Closed form: for X = U S V^T normalised to unit Frobenius norm, k steps
    of X <- aX + (b XX^T + c (XX^T)^2) X give U phi^k(S) V^T, with phi the
    scalar quintic.  SVD from LAPACK, independent of the iteration."""
    rng = np.random.default_rng(sum(shape))
    g = rng.standard_normal(shape)
    for k in (1, 3, 5):
        got = O.newton_schulz(g, k, coeffs, eps=0.0)
        u, s, vt = np.linalg.svd(g, full_matrices=False)
        s = s / math.sqrt(float(np.sum(s * s)))
        want = (u * _phi(s, coeffs, k)) @ vt
        assert np.linalg.norm(got - want) <= 1e-9 * np.linalg.norm(want)


@pytest.mark.parametrize("coeffs", [O.DEFAULT_NS_COEFFS, O.PUBLISHED_NS_COEFFS])
@pytest.mark.parametrize("shape", [(12, 30), (30, 12), (9, 9)])
def test_spectral_map_is_the_iteration_on_singular_values(shape, coeffs):
    """ns_spectral_map applied to the LAPACK singular values of a normalised
    matrix, recombined with its singular vectors, is the matrix iteration."""
    rng = np.random.default_rng(11 + shape[0])
    g = rng.standard_normal(shape)
    u, s, vt = np.linalg.svd(g, full_matrices=False)
    s = s / math.sqrt(float(np.sum(s * s)))
    for k in (1, 2, 5):
        got = O.newton_schulz(g, k, coeffs, eps=0.0)
        want = (u * O.ns_spectral_map(s, k, coeffs)) @ vt
        assert np.linalg.norm(got - want) <= 1e-9 * np.linalg.norm(want)
    assert float(O.ns_spectral_map(1.0, 5, O.DEFAULT_NS_COEFFS)) == pytest.approx(0.984131, abs=2e-6)
    assert float(O.ns_spectral_map(0.0, 5, coeffs)) == 0.0


def test_phi5_values_distinguish_step_count():
    """ns_steps = 5 (hyperparameter table of the page).  The fixed point of
    the map is not reached, so 4, 5 and 6 steps give visibly different gains
    on a unit singular value.  Numbers are the scalar compositions of each
    quintic, evaluated once in double precision by a script separate from
    the oracle, for both triples."""
    d, p = O.DEFAULT_NS_COEFFS, O.PUBLISHED_NS_COEFFS
    assert _phi(1.0, d, 5) == pytest.approx(0.984131, abs=2e-6)
    assert _phi(1.0, d, 4) == pytest.approx(0.996466, abs=2e-6)
    assert _phi(1.0, d, 6) == pytest.approx(0.995206, abs=2e-6)
    assert _phi(1.0, p, 5) == pytest.approx(0.696436, abs=2e-6)
    assert _phi(1.0, p, 4) == pytest.approx(1.089974, abs=2e-6)
    assert _phi(1.0, p, 6) == pytest.approx(1.118768, abs=2e-6)
    hp = O.HParams()
    assert hp.muon_ns_steps == 5


@pytest.mark.parametrize("shape", [(8, 32), (32, 8), (1, 17), (17, 1), (12, 12)])
def test_rank_one_input(shape):
    """Special case: a rank-1 matrix x y^T has one singular value, equal to
    its Frobenius norm, so NS returns phi^5(1) * x y^T / (|x||y|)."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal(shape[0])
    y = rng.standard_normal(shape[1])
    got = O.newton_schulz(np.outer(x, y), 5, eps=0.0)
    want = 0.984131 * np.outer(x / np.linalg.norm(x), y / np.linalg.norm(y))
    np.testing.assert_allclose(got, want, atol=3e-6)


@pytest.mark.parametrize("r,c,gain", [(4, 16, 0.958947), (16, 64, 1.037006), (64, 256, 0.949313)])
def test_orthonormal_rows(r, c, gain):
    """Special case: X = Q with orthonormal rows has r singular values 1, which
    normalisation maps to 1/sqrt(r); the result is phi^5(1/sqrt(r)) Q."""
    rng = np.random.default_rng(r)
    q, _ = np.linalg.qr(rng.standard_normal((c, r)))
    q = q.T
    got = O.newton_schulz(q, 5, eps=0.0)
    np.testing.assert_allclose(got, gain * q, atol=2e-6)
    np.testing.assert_allclose(O.newton_schulz(q.T, 5, eps=0.0), gain * q.T, atol=2e-6)


def test_alignment_with_polar_factor():
    """Brute force on tiny inputs: NS of a Gaussian matrix points along its
    orthogonal polar factor U V^T (SVD), cosine >= 0.99 for shapes with
    r <= c/4, and every output singular value lies in the band of the default
    triple, [0.934, 1.215] for sigma/||X||_F in [1e-2, 1]."""
    rng = np.random.default_rng(11)
    worst = 1.0
    for r in (4, 8, 16, 32, 64):
        for c in (4 * r, 8 * r):
            for t in range(40):
                g = rng.standard_normal((r, c))
                if t % 2:
                    g = g.T
                u, s, vt = np.linalg.svd(g, full_matrices=False)
                polar = u @ vt
                out = O.newton_schulz(g, 5)
                cos = float(np.sum(out * polar) / np.linalg.norm(out) / np.linalg.norm(polar))
                worst = min(worst, cos)
                rel = s / np.linalg.norm(s)
                sv = np.linalg.svd(out, compute_uv=False)
                inside = rel >= 1e-2
                if inside.all():
                    assert sv.min() >= 0.934 and sv.max() <= 1.215
    assert worst >= 0.99


def test_band_of_default_coefficients():
    """The recorded band of the default triple over sigma in [1e-2, 1]."""
    s = np.linspace(1e-2, 1.0, 200001)
    v = _phi(s, O.DEFAULT_NS_COEFFS, 5)
    assert 0.934 <= v.min() <= 0.9345
    assert 1.2145 <= v.max() <= 1.215


@pytest.mark.parametrize("shape", [(6, 20), (20, 6), (9, 9)])
def test_orientation_invariance(shape):
    """Invariant: NS(G^T) = NS(G)^T; the oracle transposes tall matrices, so a
    wrong back-transpose or a Gram on the wrong side breaks it."""
    rng = np.random.default_rng(5)
    g = rng.standard_normal(shape)
    a = O.newton_schulz(g.T, 5)
    b = O.newton_schulz(g, 5).T
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def test_scale_invariance_and_zero():
    """Invariants: NS(alpha G) = NS(G) for alpha > 0 (normalisation), and the
    zero matrix maps to zero (the epsilon guards the division)."""
    rng = np.random.default_rng(6)
    g = rng.standard_normal((10, 30))
    np.testing.assert_allclose(O.newton_schulz(37.5 * g, 5, eps=0.0),
                               O.newton_schulz(g, 5, eps=0.0), atol=1e-12)
    assert np.all(O.newton_schulz(np.zeros((4, 8)), 5) == 0.0)


def test_frobenius_normalise():
    """Special case reducing to a library routine: ||x||_F from numpy."""
    rng = np.random.default_rng(7)
    x = rng.standard_normal((13, 7))
    got = O.frobenius_normalise(x, 1e-7)
    np.testing.assert_allclose(got, x / (np.linalg.norm(x) + 1e-7), rtol=1e-15)


# --------------------------------------------------------------------------
# momentum, learning-rate factor, whole Muon update
# --------------------------------------------------------------------------

def test_nesterov_closed_forms():
    """Closed forms with a zero buffer, mu = 0.95 (hyperparameter table),
    coef 1: step 1 u = 1.95 g1; step 2 u = 1.95 g2 + 0.9025 g1; buffers
    g1 and g2 + 0.95 g1.  Without Nesterov u is the buffer."""
    rng = np.random.default_rng(8)
    g1, g2 = rng.standard_normal((2, 5, 4))
    u1, b1 = O.nesterov_momentum(g1, np.zeros((5, 4)), 1.0, 0.95, True)
    np.testing.assert_allclose(u1, 1.95 * g1, rtol=1e-15)
    np.testing.assert_allclose(b1, g1, rtol=1e-15)
    u2, b2 = O.nesterov_momentum(g2, b1, 1.0, 0.95, True)
    np.testing.assert_allclose(u2, 1.95 * g2 + 0.9025 * g1, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(b2, g2 + 0.95 * g1, rtol=1e-15)
    u3, _ = O.nesterov_momentum(g2, b1, 1.0, 0.95, False)
    np.testing.assert_allclose(u3, g2 + 0.95 * g1, rtol=1e-15)
    u4, b4 = O.nesterov_momentum(g1, np.zeros((5, 4)), 0.25, 0.95, True)
    np.testing.assert_allclose(b4, 0.25 * g1, rtol=1e-15)


def test_lr_shape_scale_values():
    """Closed form 0.2*sqrt(max(m,n)) (the Muon learning-rate sentence of the
    page): exact squares give 3.2, 6.4, 12.8; 8192 and 14336 worked by hand
    (sqrt(8192) = 64 sqrt 2, sqrt(14336) = 32 sqrt 14)."""
    assert O.lr_shape_scale(256, 256) == np.float32(3.2)
    assert O.lr_shape_scale(1024, 256) == np.float32(6.4)
    assert O.lr_shape_scale(256, 1024) == np.float32(6.4)
    assert O.lr_shape_scale(4096, 1024) == np.float32(12.8)
    assert O.lr_shape_scale(8192, 8192) == np.float32(12.8 * math.sqrt(2.0))
    assert O.lr_shape_scale(14336, 4096) == np.float32(6.4 * math.sqrt(14.0))
    assert O.lr_shape_scale(1, 1) == np.float32(0.2)


@pytest.mark.parametrize("shape", [(24, 96), (96, 24)])
def test_muon_update_rank_one(shape):
    """Whole Muon update of a rank-1 gradient at step 1 from a zero buffer:
    delta = lr * 0.2 sqrt(max(m,n)) * phi^5(1) * x y^T / (|x||y|), whatever
    the clip factor and the Nesterov factor 1.95 (both cancel in the
    normalisation); p moves by -delta exactly, the buffer holds coef*g."""
    rng = np.random.default_rng(9)
    x = rng.standard_normal(shape[0])
    y = rng.standard_normal(shape[1])
    g = np.outer(x, y).astype(np.float32)
    p0 = rng.standard_normal(shape).astype(np.float32) * np.float32(0.02)
    hp = O.HParams()
    coef = 0.125
    scale = O.lr_shape_scale(*shape)
    p1, buf, delta = O.muon_matrix_update(p0, g, np.zeros(shape, np.float32), coef, hp, scale)
    want = 2.5e-5 * 0.2 * math.sqrt(max(shape)) * 0.984131 * np.outer(
        x / np.linalg.norm(x), y / np.linalg.norm(y))
    np.testing.assert_allclose(delta, want, rtol=0, atol=2.5e-5 * 5.0 * 3e-6)
    np.testing.assert_allclose(p1, (p0.astype(np.float64) - delta).astype(np.float32), rtol=0, atol=0)
    np.testing.assert_allclose(buf, (coef * g.astype(np.float64)).astype(np.float32), rtol=0, atol=0)


# --------------------------------------------------------------------------
# AdamW and clipping
# --------------------------------------------------------------------------

def _load_adamw_golden():
    rows = []
    with open(os.path.join(GOLDEN, "adamw_one_step.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            rows.append([float(v) for v in line.split()])
    return np.array(rows)


def test_adamw_first_step_worked_values():
    """Closed form of the first AdamW step from zero moments (worked values
    in tests/golden/adamw_one_step.txt); the eps-sensitive row pins where eps
    enters the denominator."""
    rows = _load_adamw_golden()
    hp = O.HParams()
    p0, g, p1, m1, v1 = (rows[:, i] for i in range(5))
    z = np.zeros_like(p0)
    p, m, v = O.adamw_update(p0.astype(np.float32), g.astype(np.float32), z, z, 1, 1.0, hp)
    # inputs pass through float32, so compare to the closed form evaluated on
    # the float32-rounded inputs
    p0f = p0.astype(np.float32).astype(np.float64)
    gf = g.astype(np.float32).astype(np.float64)
    want = p0f * (1 - 2.5e-7) - 2.5e-5 * gf / (np.abs(gf) + 1e-8)
    np.testing.assert_allclose(p, want.astype(np.float32), rtol=0, atol=0)
    np.testing.assert_allclose(p, p1, rtol=2e-7, atol=1e-12)
    np.testing.assert_allclose(m, m1, rtol=2e-7, atol=0)
    np.testing.assert_allclose(v, v1, rtol=4e-7, atol=0)


def test_adamw_constant_gradient_steps():
    """Closed form: with a constant gradient the bias-corrected moments equal
    g and g^2 at every step, so each step is p <- p(1-lr wd) - lr g/(|g|+eps)."""
    hp = O.HParams()
    g = np.array([1e-3, -4e-4, 2e-9, 0.5], np.float32)
    p = np.array([0.02, -0.01, 0.03, 0.0], np.float32)
    m = np.zeros(4, np.float32)
    v = np.zeros(4, np.float32)
    ref = p.astype(np.float64)
    g64 = g.astype(np.float64)
    for t in range(1, 6):
        p, m, v = O.adamw_update(p, g, m, v, t, 1.0, hp)
        ref = ref * (1 - hp.lr * hp.weight_decay) - hp.lr * g64 / (np.abs(g64) + hp.eps)
        np.testing.assert_allclose(p, ref, rtol=1e-6, atol=1e-12)


def test_adamw_zero_gradient_is_pure_decay():
    hp = O.HParams()
    p0 = np.array([0.5, -2.0], np.float32)
    p, m, v = O.adamw_update(p0, np.zeros(2, np.float32), np.zeros(2), np.zeros(2), 1, 1.0, hp)
    np.testing.assert_allclose(p, p0 * (1 - 2.5e-7), rtol=1e-7)
    assert np.all(m == 0) and np.all(v == 0)


def test_global_norm_is_library_norm():
    """Special case reducing to a library routine: the global norm is the
    2-norm of the concatenation of all gradients."""
    rng = np.random.default_rng(12)
    gs = [rng.standard_normal(s).astype(np.float32) for s in [(3, 4), (7,), (2, 2, 2)]]
    flat = np.concatenate([g.ravel().astype(np.float64) for g in gs])
    assert O.global_grad_norm(gs) == pytest.approx(np.linalg.norm(flat), rel=1e-14)


def test_clip_coefficient_closed_forms():
    """max_grad_norm 1.0 (defaults table): no clipping at or below the limit,
    coef*N = 1*N/(N+1e-6) above it, off for max_grad_norm <= 0, NaN
    propagates."""
    assert O.clip_coefficient(0.5, 1.0) == 1.0
    assert O.clip_coefficient(1.0 - 1e-6, 1.0) == 1.0
    n = 464.0
    assert O.clip_coefficient(n, 1.0) * n == pytest.approx(n / (n + 1e-6), rel=1e-15)
    assert O.clip_coefficient(1e9, 0.0) == 1.0
    assert math.isnan(O.clip_coefficient(float("nan"), 1.0))
    assert O.clip_coefficient(float("inf"), 1.0) == 0.0
    assert O.HParams().max_grad_norm == 1.0


def test_step_clip_scope_and_order():
    """Whole-step special case.  A Muon matrix with a rank-1 gradient of norm
    10, a tiny AdamW gradient (1e-8 per element) and a frozen tensor with a
    huge gradient.  The norm must skip the frozen tensor (N = 10 exactly up to
    the AdamW part), the clip must reach AdamW before its moments (then
    coef*g = 1e-9, comparable to eps, so the update is lr*1e-9/(1e-9+1e-8)),
    and the Muon delta is the rank-1 closed form."""
    names = ["action_expert.layers.0.mlp.down_proj.weight", "vlm.model.norm.weight",
             "vlm.model.embed_tokens.weight"]
    x = np.zeros(16); x[3] = 1.0
    y = np.zeros(64); y[10] = 10.0
    gm = np.outer(x, y).astype(np.float32)
    ga = np.full(8, 1e-8, np.float32)
    gn = np.full((4, 4), 1e6, np.float32)
    params = [np.zeros((16, 64), np.float32), np.full(8, 0.1, np.float32), np.zeros((4, 4), np.float32)]
    hp = O.HParams()
    res = O.optimizer_step(names, params, [gm, ga, gn], [True, True, False],
                           [np.zeros((16, 64), np.float32), None, None],
                           [None, np.zeros(8, np.float32), None],
                           [None, np.zeros(8, np.float32), None], 1, hp)
    assert res.groups == [O.MUON, O.ADAMW, O.NONE]
    assert res.grad_norm == pytest.approx(math.sqrt(100.0 + 8 * 1e-16), rel=1e-12)
    coef = 1.0 / (res.grad_norm + 1e-6)
    assert res.clip_coef == pytest.approx(coef, rel=1e-15)
    cg = coef * float(np.float32(1e-8))
    want_a = 0.1 * (1 - 2.5e-7) - 2.5e-5 * cg / (cg + 1e-8)
    np.testing.assert_allclose(res.params[1], np.float32(want_a), rtol=1e-7)
    want_d = 2.5e-5 * 0.2 * 8.0 * 0.984131 * np.outer(x, y / 10.0)
    np.testing.assert_allclose(res.deltas[0], want_d, atol=1e-10)
    np.testing.assert_allclose(res.muon_momentum[0], (coef * gm).astype(np.float32), rtol=1e-7)
    np.testing.assert_array_equal(res.params[2], params[2])


# --------------------------------------------------------------------------
# routing and plan
# --------------------------------------------------------------------------

def _routing_rows():
    rows = []
    with open(os.path.join(GOLDEN, "routing_table.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            grp, tr, shape, name = line.rstrip("\n").split("\t")
            rows.append((grp, tr == "1", tuple(int(s) for s in shape.split(",")), name))
    return rows


def test_routing_table():
    """The page's routing rule on an adversarial table (golden file with its
    reading of every edge)."""
    for grp, tr, shape, name in _routing_rows():
        got = O.GROUP_NAMES[O.route_one(name, shape, tr)]
        assert got == grp, name


def test_routing_adamw_mode():
    """The optim switch: plain AdamW sends every trainable tensor to AdamW."""
    for grp, tr, shape, name in _routing_rows():
        want = "NONE" if not tr else "ADAMW"
        assert O.GROUP_NAMES[O.route_one(name, shape, tr, O.MODE_ADAMW)] == want


def test_workload_group_counts():
    """Group sizes of the synthetic workloads follow from the routing rule:
    tiny 14 Muon / 13 AdamW; 18-layer 126 / 0; full hybrid 126 / 253 / 1
    frozen; stress 68 / 0; the full table in plain-AdamW mode 0 / 379 / 1;
    and the element totals of the workload text."""
    import workloads as W
    expect = {
        "tiny_hybrid_fp32": (14, 13, 0, 2_097_152, 259_072),
        "ae18_muon_bf16": (126, 0, 0, 273_678_336, 0),
        "vla_hybrid_bf16": (126, 253, 1, 273_678_336, 1_879_164_928),
        "ragged_stress_bf16": (68, 0, 0, 186_646_528, 0),
        "vla_hybrid_adamw": (0, 379, 1, 0, 2_152_843_264),
    }
    for name, (nm, na, nn, em, ea) in expect.items():
        w = W.WORKLOADS[name]()
        groups = O.route(w.names, w.shapes, w.trainable, W.mode_id(w))
        assert groups.count(O.MUON) == nm
        assert groups.count(O.ADAMW) == na
        assert groups.count(O.NONE) == nn
        numel = [p.numel for p in w.params]
        assert sum(n for n, g in zip(numel, groups) if g == O.MUON) == em
        assert sum(n for n, g in zip(numel, groups) if g == O.ADAMW) == ea


def test_plan_dump_shape():
    """Plan dump header and bucket lines on the 18-layer table: three
    canonical buckets (1024,1024)x36, (256,1024)x36, (1024,4096)x54 and the
    shape factors 6.4 / 12.8 for max dims 1024 / 4096."""
    import workloads as W
    w = W.ae18_muon_bf16()
    text = O.plan_dump(w.names, w.shapes, w.trainable)
    lines = text.splitlines()
    assert lines[0] == ("muon_adamw_plan v1 mode=0 entries=126 muon=126 adamw=0 none=0 "
                        "buckets=3 adamw_numel=0")
    assert lines[1] == "bucket 0 r=1024 c=1024 count=36"
    assert lines[2] == "bucket 1 r=256 c=1024 count=36"
    assert lines[3] == "bucket 2 r=1024 c=4096 count=54"
    six4 = "%08x" % int(np.array([6.4], np.float32).view(np.uint32)[0])
    t128 = "%08x" % int(np.array([12.8], np.float32).view(np.uint32)[0])
    assert lines[4] == "0 MUON 0 1024 1024 1024 1024 0 %s 1048576 -1" % six4
    assert lines[8] == "4 MUON 2 4096 1024 1024 4096 1 %s 4194304 -1" % t128


# --------------------------------------------------------------------------
# diagnostic bf16 emulation
# --------------------------------------------------------------------------

def test_bf16_round_matches_torch():
    """Special case reducing to a library routine: torch's float32->bfloat16
    conversion rounds to nearest even."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(13)
    x = np.concatenate([rng.standard_normal(10000).astype(np.float32) * 10.0 ** rng.integers(-20, 20, 10000),
                        np.array([0.0, -0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 65504.0], np.float32)]).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(O.bf16_round(x), want)


def test_bf16_split_hand_worked():
    """hi = bf16(x), lo = bf16(x - hi), worked by hand:
    1 + 2^-6 + 2^-12 + 2^-20 -> hi 1 + 2^-6 (the rest is below half a spacing
    2^-8), lo = bf16(2^-12 (1 + 2^-8)) = 2^-12 (a tie, to the even 2^-12);
    -(3 + 2^-9) -> hi -3, lo -2^-9; 0.5 -> (0.5, 0)."""
    x = np.array([1 + 2 ** -6 + 2 ** -12 + 2 ** -20, -(3 + 2 ** -9), 0.5], np.float32)
    hi, lo = O.bf16_split(x)
    np.testing.assert_array_equal(hi, [1 + 2 ** -6, -3.0, 0.5])
    np.testing.assert_array_equal(lo, [2 ** -12, -2 ** -9, 0.0])


# Hand-worked 2 x 3 inputs of the bf16 policy model.  X_LIN needs more than
# 16 significant bits in its first entry; X_POLY's first entry is not a
# bf16 value (1 + 2^-10 rounds to 1), so hi differs from X there, and its
# Gram has an entry that bf16 rounds (9.828125 -> 9.8125).
X_LIN = np.array([[1 + 2 ** -6 + 2 ** -12 + 2 ** -20, 0.5, 0.0],
                  [0.0, 0.25, -(3 + 2 ** -9)]], np.float32)
X_POLY = np.array([[1 + 2 ** -10, 0.5, 0.0],
                   [0.0, 0.25, 3.125]], np.float32)


def test_bf16_policy_linear_term_uses_the_hi_lo_master():
    """Coefficients (2, 0, 0): B = 0, so each step doubles the master hi + lo
    exactly and the result after two steps is 4 (hi + lo) of the input:
    4 (1 + 2^-6 + 2^-12) = 4.0634765625 and -4 (3 + 2^-9) = -12.0078125.
    A float32 master would keep the 2^-20 (4.06348037...), a bf16-only X
    would give 4.0625.  With the lo half used in the first step only, the
    second step doubles hi(2 (1 + 2^-6 + 2^-12)) = 2.03125 -> 4.0625, and
    hi(-(6 + 2^-8)) = -6 -> -12."""
    y = O.ns_bf16_policy_iterate(X_LIN, 2, (2.0, 0.0, 0.0))
    np.testing.assert_array_equal(y, [[4.0634765625, 2.0, 0.0], [0.0, 1.0, -12.0078125]])
    y1 = O.ns_bf16_policy_iterate(X_LIN, 2, (2.0, 0.0, 0.0), lo_iters=1)
    np.testing.assert_array_equal(y1, [[4.0625, 2.0, 0.0], [0.0, 1.0, -12.0]])


def test_bf16_policy_gram_rounding():
    """Coefficients (0, 1, 0): Y = bf16(A) hi with A = hi hi^T, by hand.
    hi = [[1, .5, 0], [0, .25, 3.125]]; A = [[1.25, .125], [.125, 9.828125]],
    and 9.828125 = 1.001110101b x 2^3 rounds to 1.0011101b x 2^3 = 9.8125.
    Y = A hi = [[1.25, .65625, .390625], [.125, 2.515625, 30.6640625]]
    (an unrounded Gram would give 2.51953125 and 30.712890625)."""
    y = O.ns_bf16_policy_iterate(X_POLY, 1, (0.0, 1.0, 0.0))
    np.testing.assert_array_equal(y, [[1.25, 0.65625, 0.390625], [0.125, 2.515625, 30.6640625]])


def test_bf16_policy_square_rounding():
    """Coefficients (0, 0, 1): Y = bf16(A A) hi with the bf16 A above, by
    hand.  A A = [[1.578125, 1.3828125], [1.3828125, 96.30078125]]; the last
    is 1.10000001001101b x 2^6 and rounds up to 96.5.
    Y = [[1.578125, 1.134765625, 4.3212890625], [1.3828125, 24.81640625, 301.5625]]."""
    y = O.ns_bf16_policy_iterate(X_POLY, 1, (0.0, 0.0, 1.0))
    np.testing.assert_array_equal(y, [[1.578125, 1.134765625, 4.3212890625],
                                      [1.3828125, 24.81640625, 301.5625]])


def test_bf16_policy_same_bf16_gram_in_both_terms():
    """Coefficients (0, 1, 1): B = bf16(A + A A) with the same bf16 A in
    both terms, by hand: A + A A = [[2.828125, 1.5078125], [1.5078125,
    106.11328125]], and the last (1.10101000011101b x 2^6) rounds down to
    106.  Y = B hi = [[2.828125, 1.791015625, 4.7119140625],
    [1.5078125, 27.25390625, 331.25]]."""
    y = O.ns_bf16_policy_iterate(X_POLY, 1, (0.0, 1.0, 1.0))
    np.testing.assert_array_equal(y, [[2.828125, 1.791015625, 4.7119140625],
                                      [1.5078125, 27.25390625, 331.25]])


def test_bf16_emulated_orientation_and_scale():
    """The wrapper orients and normalises like newton_schulz: a tall input
    gives the transpose of its wide transpose's result, bit for bit, and a
    power-of-two scaling of the input changes nothing (it commutes with
    every rounding)."""
    rng = np.random.default_rng(15)
    g = rng.standard_normal((24, 96))
    w = O.newton_schulz_bf16_emulated(g, 5)
    np.testing.assert_array_equal(O.newton_schulz_bf16_emulated(g.T.copy(), 5), w.T)
    np.testing.assert_array_equal(O.newton_schulz_bf16_emulated(g * 2.0 ** 20, 5, eps=0.0),
                                  O.newton_schulz_bf16_emulated(g, 5, eps=0.0))


def test_bf16_emulated_error_band_and_thin_matrices():
    """Against the fp64 iteration the bf16 policy costs about 1e-2 on
    Gaussian and row-scaled inputs (0.3-1.6 times the 2e-2 bf16 gate), and
    the matrices with one to three rows reach past the gate: the reason
    very thin Muon matrices run their Newton-Schulz in fp32."""
    rng = np.random.default_rng(5)

    def err(g, **kw):
        a = O.newton_schulz(g, 5)
        return np.linalg.norm(O.newton_schulz_bf16_emulated(g, 5, **kw) - a) / np.linalg.norm(a)

    for shape in ((64, 256), (32, 1024)):
        g = rng.standard_normal(shape) * np.exp(rng.uniform(np.log(0.1), np.log(10), shape[0]))[:, None]
        assert 4e-3 < err(g) < 1.6e-2
    thin = [max(err(rng.standard_normal((r, 1024))) for _ in range(20)) for r in (2, 3)]
    assert max(thin) > 2e-2, thin


# ---------------------------------------------------------------------------
# Learning-rate schedule cosine_with_min_lr (defaults table: min_lr_rate 0.1)
# ---------------------------------------------------------------------------

def test_schedule_special_points():
    """What the schedule's definition fixes: the base rate at the first
    scheduler step, min_lr_rate times it at total_steps and after, the mean
    of the two halfway (cos(pi/2) = 0), 0.5 (1 + 1/sqrt 2) of the way down at
    a quarter, and a linear warmup from 0."""
    hp = O.HParams(lr_schedule="cosine_with_min_lr", total_steps=100, min_lr_rate=0.1)
    assert O.schedule_factor(hp, 0) == 1.0
    assert O.schedule_factor(hp, 50) == pytest.approx(0.55, abs=1e-15)
    assert O.schedule_factor(hp, 25) == pytest.approx(0.1 + 0.9 * 0.8535533905932737, abs=1e-15)
    assert O.schedule_factor(hp, 100) == pytest.approx(0.1, abs=1e-15)
    assert O.schedule_factor(hp, 1000) == pytest.approx(0.1, abs=1e-15)
    warm = O.HParams(lr_schedule="cosine_with_min_lr", total_steps=30, warmup_steps=10)
    assert [O.schedule_factor(warm, k) for k in (0, 1, 5, 9)] == [0.0, 0.1, 0.5, 0.9]
    assert O.schedule_factor(warm, 10) == 1.0
    assert O.schedule_factor(warm, 20) == pytest.approx(0.55, abs=1e-15)
    const = O.HParams()
    assert all(O.schedule_factor(const, k) == 1.0 for k in (0, 7, 10 ** 6))
    with pytest.raises(ValueError):
        O.schedule_factor(O.HParams(lr_schedule="linear"), 0)


def test_schedule_matches_the_trainer_family_scheduler():
    """Special case reducing to a library routine: up to total_steps the
    schedule equals the learning-rate multipliers of transformers'
    get_cosine_with_min_lr_schedule_with_warmup (the scheduler behind the
    name cosine_with_min_lr in the HF-Trainer family the page's trainer
    belongs to), with and without warmup.  Past total_steps that scheduler
    runs on along the cosine; the oracle holds the minimum instead (its own
    reading, pinned in test_schedule_special_points)."""
    torch = pytest.importorskip("torch")
    transformers = pytest.importorskip("transformers")
    for warm, total in ((0, 100), (10, 30), (7, 7), (0, 1)):
        hp = O.HParams(lr_schedule="cosine_with_min_lr", warmup_steps=warm, total_steps=total,
                       min_lr_rate=0.1)
        opt = torch.optim.SGD([torch.zeros(1, requires_grad=True)], lr=1.0)
        sched = transformers.get_cosine_with_min_lr_schedule_with_warmup(
            opt, num_warmup_steps=warm, num_training_steps=total, min_lr_rate=0.1)
        for k in range(total + 1):
            assert O.schedule_factor(hp, k) == pytest.approx(sched.get_last_lr()[0], rel=1e-12,
                                                             abs=1e-15), (warm, total, k)
            opt.step()
            sched.step()


def test_schedule_monotone_and_bounded():
    hp = O.HParams(lr_schedule="cosine_with_min_lr", total_steps=37, warmup_steps=5,
                   min_lr_rate=0.25)
    f = [O.schedule_factor(hp, k) for k in range(60)]
    assert all(a <= b for a, b in zip(f[:5], f[1:6]))          # warmup rises
    assert all(a >= b for a, b in zip(f[5:], f[6:]))           # then falls
    assert min(f[5:]) == pytest.approx(0.25) and max(f) == 1.0


def test_schedule_scales_the_whole_step():
    """One AdamW step from zero moments at optimizer step t = 51 of a
    100-step schedule (factor 0.55): closed form with lr 0.55 * 2.5e-5 and
    the bias corrections of t = 51; and a Muon update scaled by exactly the
    same factor as with a constant rate."""
    hp = O.HParams(lr_schedule="cosine_with_min_lr", total_steps=100)
    g = np.array([1e-3, -2e-6, 0.4], np.float32)
    p0 = np.array([0.02, -0.01, 0.3], np.float32)
    z = np.zeros(3, np.float32)
    names = ["vlm.x", "action_expert.layers.0.q.weight"]
    gm = np.random.default_rng(5).standard_normal((6, 9)).astype(np.float32) * np.float32(1e-3)
    pm = np.random.default_rng(6).standard_normal((6, 9)).astype(np.float32) * np.float32(0.02)
    res = O.optimizer_step(names, [p0, pm], [g, gm], [True, True], [None, np.zeros_like(gm)],
                           [z, None], [z, None], 51, hp)
    lr = 0.55 * 2.5e-5
    coef = res.clip_coef
    gc = coef * g.astype(np.float64)
    m_hat = 0.1 * gc / (1 - 0.9 ** 51)
    v_hat = 0.001 * gc * gc / (1 - 0.999 ** 51)
    want = p0.astype(np.float64) * (1 - lr * 0.01) - lr * m_hat / (np.sqrt(v_hat) + 1e-8)
    np.testing.assert_allclose(res.params[0], want, rtol=3e-7, atol=1e-12)
    flat = O.optimizer_step(names, [p0, pm], [g, gm], [True, True], [None, np.zeros_like(gm)],
                            [z, None], [z, None], 51, O.HParams())
    np.testing.assert_allclose(res.deltas[1], 0.55 * flat.deltas[1], rtol=1e-12, atol=0)


# --------------------------------------------------------------------------
# bfloat16 parameter storage
# --------------------------------------------------------------------------

def _bf16_brute(x: float) -> float:
    """Nearest bfloat16 by search: the bfloat16 values around x (float32 bit
    patterns with the low 16 bits clear), the closest by exact float64
    distance, ties to the even 16-bit pattern."""
    import struct
    if x == 0.0:
        return x
    f = np.float32(x) if abs(x) < 3.0e38 else np.float32(math.copysign(3.0e38, x))
    base = struct.unpack("<I", struct.pack("<f", float(f)))[0] & 0xFFFF0000
    best = None
    for k in range(-2, 3):
        b = (base + (k << 16)) & 0xFFFFFFFF
        if (b & 0x7F800000) == 0x7F800000:
            continue                                # inf / NaN patterns
        v = struct.unpack("<f", struct.pack("<I", b))[0]
        d = abs(x - v)
        key = (d, (b >> 16) & 1)
        if best is None or key < best[0]:
            best = (key, v)
    return best[1]


def test_bf16_round_f64_brute_force():
    """Direct float64 -> bfloat16 rounding against a search over the
    neighbouring bfloat16 values, over many magnitudes and signs."""
    rng = np.random.default_rng(21)
    x = rng.standard_normal(4000) * np.exp(rng.uniform(-60, 60, 4000))
    got = O.bf16_round_f64(x)
    want = np.array([_bf16_brute(float(v)) for v in x], np.float32)
    np.testing.assert_array_equal(got, want)


def test_bf16_round_f64_ties_and_double_rounding():
    """Exact midpoints go to the even neighbour; a value just above a
    midpoint by less than float32 can hold goes up (rounding through float32
    first would land on the tie and go to even instead)."""
    lo = np.float64(1.0)                # bf16 neighbours 1 and 1 + 2^-7
    mid = lo + 2.0 ** -8
    assert float(O.bf16_round_f64(mid)) == 1.0                       # even
    mid2 = 1.0 + 2.0 ** -7 + 2.0 ** -8                               # between odd and even
    assert float(O.bf16_round_f64(mid2)) == 1.0 + 2.0 ** -6
    above = mid + 2.0 ** -40
    assert np.float32(above) == np.float32(mid)                      # float32 loses it
    assert float(O.bf16_round_f64(above)) == 1.0 + 2.0 ** -7
    assert float(O.bf16_round_f64(-above)) == -(1.0 + 2.0 ** -7)
    # agrees with the float32 rounding wherever the input is a float32
    rng = np.random.default_rng(4)
    f = (rng.standard_normal(3000) * 10.0 ** rng.uniform(-30, 30, 3000)).astype(np.float32)
    np.testing.assert_array_equal(O.bf16_round_f64(f.astype(np.float64)), O.bf16_round(f))
    # subnormal spacing 2^-133, overflow to infinity, NaN kept
    q = 2.0 ** -133
    assert float(O.bf16_round_f64(2.5 * q)) == 2.0 * q
    assert float(O.bf16_round_f64(3.5 * q)) == 4.0 * q
    assert np.isinf(O.bf16_round_f64(np.float64(3.4e38)))
    assert np.isnan(O.bf16_round_f64(np.float64("nan")))


def test_bf16_storage_rounds_the_fp32_storage_step():
    """The same step under bf16 storage gives the bfloat16 rounding of the
    float64 result that fp32 storage rounds to float32 (checked through the
    rounding window of the float32 value), for both groups; states are
    unchanged by the storage."""
    rng = np.random.default_rng(8)
    hp32 = O.HParams(max_grad_norm=0.0)
    hp16 = O.HParams(max_grad_norm=0.0, param_storage="bf16")
    p = O.bf16_round(rng.standard_normal((16, 24)).astype(np.float32) * 0.02)
    g = O.bf16_round(rng.standard_normal((16, 24)).astype(np.float32) * 1e-3)
    z = np.zeros_like(p)
    p32, m32, v32 = O.adamw_update(p, g, z, z, 1, 1.0, hp32)
    p16, m16, v16 = O.adamw_update(p, g, z, z, 1, 1.0, hp16)
    np.testing.assert_array_equal(m16, m32)
    np.testing.assert_array_equal(v16, v32)
    assert np.all(O.bf16_round(p16) == p16)                          # bf16 values
    spacing = np.abs(p16) * 2.0 ** -7
    assert np.all(np.abs(p16.astype(np.float64) - p32) <= 0.5 * spacing + 1e-12)
    # AdamW's first step moves p by about lr = 2.5e-5, under half a bf16
    # spacing at |p| ~ 0.02: most parameters stay where they were
    assert np.mean(p16 == p) > 0.5
    s = O.lr_shape_scale(16, 24)
    q32, b32, d32 = O.muon_matrix_update(p, g, z, 1.0, hp32, s)
    q16, b16, d16 = O.muon_matrix_update(p, g, z, 1.0, hp16, s)
    np.testing.assert_array_equal(b16, b32)
    np.testing.assert_array_equal(d16, d32)
    np.testing.assert_array_equal(q16, O.bf16_round_f64(p.astype(np.float64) - d32))


def test_rank_shares_partition_the_hybrid_table():
    """The per-GPU shares of the owner-compute sharding cover the hybrid
    table exactly once: every Muon matrix on one GPU (LPT loads within 1 %
    of the mean), the AdamW elements cut into equal contiguous ranges."""
    import workloads as W
    world = 8
    full = W.vla_hybrid_bf16()
    muon = [p for p in full.params if p.name.startswith("action_expert.")]
    adam = [p for p in full.params if p.trainable and not p.name.startswith("action_expert.")]
    seen, loads, adam_total = [], [], 0
    for r in range(world):
        w = W.vla_hybrid_share(r, world)
        mats = [p for p in w.params if "[" not in p.name]
        seen += [p.name for p in mats]
        loads.append(sum(W.ns_cost(p.shape) for p in mats))
        n = sum(p.numel for p in w.params if "[" in p.name)
        assert n == sum(p.numel for p in adam) // world
        adam_total += n
    assert sorted(seen) == sorted(p.name for p in muon)
    mean = sum(loads) / world
    assert max(loads) <= 1.01 * mean and min(loads) >= 0.99 * mean
    assert adam_total == sum(p.numel for p in adam)
