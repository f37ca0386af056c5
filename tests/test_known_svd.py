"""Inputs with a singular value decomposition known by construction.

The maximum-size GPU tests feed the step a gradient G = U diag(sigma) V^T
built from orthonormal DCT-II matrices and compare sampled rows of the Muon
update with the oracle's steps applied to that spectrum.  These CPU tests pin
every piece of that at small sizes: the factors are orthonormal, G has the
stated singular values (LAPACK), rows come out right from one inverse DCT
each, the torch generator builds the same G, and the expected rows equal the
oracle's whole-matrix Muon update.
"""

import math

import numpy as np
import pytest

import oracle as O
import workloads as W
from tests import _harness as H


@pytest.mark.parametrize("n", [1, 2, 5, 16, 37])
def test_dct_matrix_is_orthonormal(n):
    c = W.dct_entries(n, np.arange(n)[:, None], np.arange(n)[None, :])
    np.testing.assert_allclose(c @ c.T, np.eye(n), atol=1e-13)


@pytest.mark.parametrize("r,c", [(1, 1), (3, 8), (12, 40), (16, 16)])
def test_known_svd_has_the_stated_spectrum(r, c):
    ks = W.known_svd(5, r, c)
    g = W.np_known_svd_matrix(ks, ks.sigma)
    s = np.linalg.svd(g, compute_uv=False)
    np.testing.assert_allclose(s, np.sort(ks.sigma)[::-1], rtol=1e-12)
    assert math.isclose(float(np.linalg.norm(g)), 3.0, rel_tol=1e-12)
    assert len(set(ks.rows.tolist())) == r


def test_rows_by_inverse_dct():
    ks = W.known_svd(9, 12, 40)
    w = np.linspace(-1.0, 2.0, 12)
    full = W.np_known_svd_matrix(ks, w)
    for i in range(12):
        np.testing.assert_allclose(W.np_known_svd_row(ks, i, w), full[i], rtol=0, atol=1e-13)


@pytest.mark.parametrize("transposed", [False, True])
def test_torch_generator_builds_the_same_matrix(transposed):
    torch = pytest.importorskip("torch")
    ks = W.known_svd(4, 20, 52)
    want = W.np_known_svd_matrix(ks, ks.sigma)
    if transposed:
        want = want.T
    got = W.torch_known_svd_grad(ks, "cpu", transposed=transposed, block=7).numpy()
    assert got.dtype == np.float32 and got.shape == want.shape
    # float64 sums in another order, then one rounding: equal to within an ulp
    np.testing.assert_allclose(got, want, rtol=0, atol=2e-7 * np.abs(want).max())


@pytest.mark.parametrize("r,c,transposed", [(12, 40, False), (12, 40, True), (16, 16, False)])
@pytest.mark.parametrize("coeffs", [O.DEFAULT_NS_COEFFS, O.PUBLISHED_NS_COEFFS])
def test_expected_rows_equal_oracle_update(r, c, transposed, coeffs):
    """The expected-value helper (clip, momentum, normalisation, NS map,
    rate on the known spectrum) equals the oracle's whole-matrix Muon
    update of the first step, row by row."""
    ks = W.known_svd(2, r, c)
    hp = O.HParams()
    hp.ns_coeffs = coeffs
    g = W.np_known_svd_matrix(ks, ks.sigma).astype(np.float32)
    stored = g.T if transposed else g
    m, n = stored.shape
    norm = O.global_grad_norm([stored])
    coef = O.clip_coefficient(norm, hp.max_grad_norm)
    assert coef < 1.0                       # the clip is active at norm 3
    _, _, delta = O.muon_matrix_update(np.zeros_like(stored), stored, np.zeros_like(stored),
                                       coef, hp, O.lr_shape_scale(m, n))
    canon = delta.T if transposed else delta
    want = H.known_svd_muon_delta_rows(ks, range(r), hp, m, n, norm)
    # G is rounded to float32, so its spectrum is sigma only to ~1e-7
    assert np.linalg.norm(canon - want) <= 1e-6 * np.linalg.norm(want)
