"""Pins of the oracle's Newton-Schulz chain against mathematics that does not
come from the oracle itself.

* closed form through the SVD: each iteration maps every singular value by the
  scalar polynomial p(s) = a s + b s^3 + c s^5 and keeps the singular vectors;
* the cubic (1.5, -0.5, 0) converges to the polar factor (scipy.linalg.polar);
* the quintic output's singular values lie in a stated band;
* invariances (transpose, positive scaling, orthogonal equivariance);
* degenerate inputs with exact answers (1 x 1, one row, zero matrix, K = 0).
"""

import math

import numpy as np
import pytest
import scipy.linalg

from oracle import muon
from synth import random_case

QUINTIC = (3.4445, -4.7750, 2.0315)


def scalar_poly_iterate(s, a, b, c, k):
    s = np.asarray(s, dtype=np.float64)
    for _ in range(k):
        s = a * s + b * s ** 3 + c * s ** 5
    return s


def svd_closed_form(X, a, b, c, k):
    U, S, Vt = np.linalg.svd(X, full_matrices=False)
    return (U * scalar_poly_iterate(S, a, b, c, k)) @ Vt


SHAPES = [(1, 1), (1, 7), (4, 6), (8, 8), (16, 5), (33, 17), (64, 128), (96, 96)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("coeffs,k", [(QUINTIC, 5), (QUINTIC, 3), ((1.5, -0.5, 0.0), 7),
                                      ((2.0, -1.3, 0.4), 4)])
def test_ns_matches_svd_closed_form(shape, coeffs, k):
    r, c = shape
    G = random_case(11 + r * 1000 + c, r, c, std=1.0)
    X0, transposed = muon.normalise_and_orient(G, 1e-7)
    got = muon.newton_schulz(X0, *coeffs, k)
    want = svd_closed_form(X0, *coeffs, k)
    err = np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-300)
    assert err < 1e-11, err


def well_conditioned(seed, r, c, kappa=10.0):
    rng = np.random.default_rng(seed)
    m = min(r, c)
    Q1, _ = np.linalg.qr(rng.standard_normal((r, m)))
    Q2, _ = np.linalg.qr(rng.standard_normal((c, m)))
    s = np.linspace(1.0, kappa, m)
    return (Q1 * s) @ Q2.T


@pytest.mark.parametrize("shape", [(4, 6), (8, 8), (16, 5), (3, 11)])
def test_cubic_converges_to_polar_factor(shape):
    M = well_conditioned(7, *shape)
    cfg = muon.StepConfig(a=1.5, b=-0.5, c=0.0, ns_steps=60, eps=0.0)
    O = muon.orthogonalise(M, cfg)
    Upol, _ = scipy.linalg.polar(M, side="right")
    assert np.max(np.abs(O - Upol)) < 1e-12


@pytest.mark.parametrize("shape,k,thr,lo,hi", [
    ((64, 160), 5, 3e-3, 0.6818, 1.2024),
    ((160, 64), 5, 1e-2, 0.6818, 1.1344),
    ((96, 96), 3, 3e-2, 0.6818, 1.2024),
    ((48, 200), 8, 1e-3, 0.6818, 1.1344),
])
def test_quintic_singular_value_band(shape, k, thr, lo, hi):
    """Default quintic coefficients: every input singular value (after
    normalisation) above ``thr`` leaves the iteration inside [lo, hi]."""
    G = random_case(5, *shape)
    X0, transposed = muon.normalise_and_orient(G, 1e-7)
    s_in = np.linalg.svd(X0, compute_uv=False)
    cfg = muon.StepConfig(ns_steps=k)
    O = muon.orthogonalise(G, cfg)
    U, s_out, Vt = np.linalg.svd(O.T if transposed else O, full_matrices=False)
    # p^k is not monotone on [0, 1], so compare the two spectra as sorted lists
    mapped = scalar_poly_iterate(s_in, *QUINTIC, k)
    assert np.allclose(np.sort(mapped), np.sort(s_out), atol=1e-10)
    sel = s_in >= thr
    assert sel.sum() > 0
    assert np.all(mapped[sel] >= lo - 1e-4) and np.all(mapped[sel] <= hi + 1e-4)


def test_band_edges_from_scalar_polynomial():
    grid = np.linspace(3e-3, 1.0, 200001)
    v = scalar_poly_iterate(grid, *QUINTIC, 5)
    assert abs(v.min() - 0.6818) < 1e-4 and abs(v.max() - 1.2024) < 1e-4
    assert abs(scalar_poly_iterate(1.0, *QUINTIC, 5) - 0.6964) < 1e-4


@pytest.mark.parametrize("shape", [(12, 30), (30, 12), (17, 17)])
def test_transpose_invariance(shape):
    cfg = muon.StepConfig()
    M = random_case(3, *shape)
    assert np.allclose(muon.orthogonalise(M.T, cfg), muon.orthogonalise(M, cfg).T,
                       rtol=0, atol=1e-13)


@pytest.mark.parametrize("alpha", [1e-3, 0.5, 37.0])
def test_positive_scaling_invariance(alpha):
    cfg = muon.StepConfig(eps=0.0)
    M = random_case(4, 20, 33)
    assert np.allclose(muon.orthogonalise(alpha * M.astype(np.float64), cfg),
                       muon.orthogonalise(M, cfg), rtol=0, atol=1e-12)


def test_orthogonal_equivariance():
    cfg = muon.StepConfig()
    rng = np.random.default_rng(9)
    M = random_case(6, 10, 24).astype(np.float64)
    Q1, _ = np.linalg.qr(rng.standard_normal((10, 10)))
    Q2, _ = np.linalg.qr(rng.standard_normal((24, 24)))
    assert np.allclose(muon.orthogonalise(Q1 @ M @ Q2, cfg),
                       Q1 @ muon.orthogonalise(M, cfg) @ Q2, rtol=0, atol=1e-12)


def test_orientation_is_wide():
    X, t = muon.normalise_and_orient(np.ones((9, 4)), 0.0)
    assert t and X.shape == (4, 9)
    X, t = muon.normalise_and_orient(np.ones((4, 9)), 0.0)
    assert (not t) and X.shape == (4, 9)
    X, t = muon.normalise_and_orient(np.ones((5, 5)), 0.0)
    assert (not t) and X.shape == (5, 5)


def test_scalar_case():
    cfg = muon.StepConfig(eps=0.0)
    for v in (-3.0, 0.25, 8.0):
        O = muon.orthogonalise(np.array([[v]]), cfg)
        assert abs(O[0, 0] - math.copysign(scalar_poly_iterate(1.0, *QUINTIC, 5), v)) < 1e-14


def test_single_row_case():
    cfg = muon.StepConfig(eps=1e-7)
    x = random_case(8, 1, 50).astype(np.float64)
    nrm = np.linalg.norm(x)
    s0 = nrm / (nrm + 1e-7)
    want = scalar_poly_iterate(s0, *QUINTIC, 5) * x / nrm
    assert np.allclose(muon.orthogonalise(x, cfg), want, rtol=0, atol=1e-14)
    # a single column is the transpose of a single row
    assert np.allclose(muon.orthogonalise(x.T, cfg), want.T, rtol=0, atol=1e-14)


def test_zero_matrix_gives_zero():
    O = muon.orthogonalise(np.zeros((6, 10)), muon.StepConfig())
    assert np.all(O == 0.0)


def test_zero_steps_is_normalised_input():
    G = random_case(12, 7, 13).astype(np.float64)
    O = muon.orthogonalise(G, muon.StepConfig(ns_steps=0, eps=0.0))
    assert np.allclose(O, G / np.linalg.norm(G), rtol=0, atol=1e-15)
