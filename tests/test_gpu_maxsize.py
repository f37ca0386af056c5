"""The Muon step at the plan's size limit, against a closed form.

A Muon matrix may hold at most (2^31 - 1) / 4 elements after padding both
sides to the 256-wide GEMM tiles (its fp32 Newton-Schulz operand stays under
2 GiB); 16384 x 32512 is the largest such shape.  No CPU check can run the
iteration on it, so the gradient is built with a known singular value
decomposition (workloads.known_svd: orthonormal DCT factors), and sampled rows
of the update are compared with the oracle's steps applied to that spectrum
(tests/_harness.known_svd_muon_delta_rows, pinned against the oracle's
whole-matrix update in test_known_svd.py).  One case per NS precision, one in
each stored orientation.
"""

import math

import numpy as np
import pytest

import oracle as O
import workloads as W
from tests import _harness as H

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
M = pytest.importorskip("muon_newton_schulz_02_amd")

R_MAX, C_MAX = 16384, 32512


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    M.load_library()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_limit_shape_is_the_largest_accepted():
    assert R_MAX * C_MAX <= ((1 << 31) - 1) // 4
    assert R_MAX * (C_MAX + 256) > ((1 << 31) - 1) // 4
    name = "action_expert.layers.0.mlp.up_proj.weight"
    M.muon_adamw_plan([(name, (R_MAX, C_MAX), True)])
    with pytest.raises(M.MuonAdamWError):
        M.muon_adamw_plan([(name, (R_MAX, C_MAX + 1), True)])


@pytest.mark.parametrize("prec,transposed", [("bf16", False), ("fp32", True)])
def test_max_size_matrix_closed_form(prec, transposed):
    dev = torch.device("cuda", 0)
    ks = W.known_svd(17, R_MAX, C_MAX)
    m, n = (C_MAX, R_MAX) if transposed else (R_MAX, C_MAX)
    name = "action_expert.layers.0.mlp.up_proj.weight"
    plan = M.muon_adamw_plan([(name, (m, n), True)])
    assert M.muon_adamw_plan_entry(plan, 0)["group"] == M.MA_GROUP_MUON
    assert M.muon_adamw_plan_entry(plan, 0)["transposed"] == int(transposed)
    hp = O.HParams()
    lhp = H.lib_hparams(M, hp, prec)

    H.say("max size %s %dx%d: inputs" % (prec, m, n))
    grad = W.torch_known_svd_grad(ks, dev, transposed=transposed)
    torch.cuda.empty_cache()
    gen = torch.Generator(device=dev)
    gen.manual_seed(W.torch_seed(17, W.KIND_PARAM, 0, 0))
    param = torch.empty((m, n), dtype=torch.float32, device=dev).normal_(0.0, 0.02, generator=gen)
    buf = torch.zeros((m, n), dtype=torch.float32, device=dev)
    delta = torch.empty((m, n), dtype=torch.float32, device=dev)
    norm_out = torch.empty(1, dtype=torch.float32, device=dev)
    state = M.State(1)
    state.muon_momentum[0] = buf
    ws = torch.empty(M.muon_adamw_workspace_size(plan, lhp.ns_precision), dtype=torch.uint8,
                     device=dev)

    rng = np.random.default_rng(3)
    rows = sorted({0, R_MAX - 1, *rng.choice(R_MAX, size=6, replace=False).tolist()})
    idx = torch.as_tensor(rows, device=dev)

    def canon_rows(t):
        return H.host(t[:, idx].t() if transposed else t[idx])

    p_old = canon_rows(param).copy()
    g_rows = canon_rows(grad).copy()

    H.say("max size %s %dx%d: step" % (prec, m, n))
    M.muon_adamw_step(plan, [param], [grad], state, lhp, ws, grad_norm_out=norm_out,
                      muon_update_out=[delta])
    torch.cuda.synchronize()
    H.say("max size %s %dx%d: compare" % (prec, m, n))

    norm = float(H.host(norm_out)[0])
    assert math.isclose(norm, 3.0, rel_tol=1e-5)
    got = canon_rows(delta).astype(np.float64)
    want = H.known_svd_muon_delta_rows(ks, rows, hp, m, n, norm)
    err = float(np.linalg.norm(got - want) / np.linalg.norm(want))
    tol = H.BF16_TOL if prec == "bf16" else H.FP32_TOL
    H.say("max size %s: relative Frobenius error over %d rows %.3e (gate %.0e)"
          % (prec, len(rows), err, tol))
    assert err <= tol
    # p = p - delta exactly (Muon decay 0); buf = coef * g, one rounding
    np.testing.assert_array_equal(canon_rows(param), p_old - canon_rows(delta))
    coef = O.clip_coefficient(norm, hp.max_grad_norm)
    np.testing.assert_allclose(canon_rows(buf), coef * g_rows.astype(np.float64), rtol=2e-6)
    del grad, param, buf, delta, ws
    torch.cuda.empty_cache()
