"""Pins of the oracle's momentum, norm and update arithmetic, and of the whole
one-matrix step, against closed forms and library routines."""

import math

import numpy as np
import pytest

from oracle import muon
from synth import random_case

QUINTIC = (3.4445, -4.7750, 2.0315)


def p_iter(s, k, coeffs=QUINTIC):
    a, b, c = coeffs
    for _ in range(k):
        s = a * s + b * s ** 3 + c * s ** 5
    return s


@pytest.mark.parametrize("mu", [0.0, 0.5, 0.95])
def test_momentum_geometric_series(mu):
    """From M0 = 0 with a constant gradient, t accumulations give
    G (1 - mu^t) / (1 - mu) (or t G when mu = 1)."""
    G = random_case(21, 5, 9).astype(np.float64)
    M = np.zeros_like(G)
    for t in range(1, 8):
        M = muon.momentum_accumulate(M, G, mu)
        want = G * (t if mu == 1.0 else (1 - mu ** t) / (1 - mu))
        assert np.allclose(M, want, rtol=1e-15, atol=0)


def test_momentum_decays_without_gradient():
    M0 = random_case(22, 4, 4).astype(np.float64)
    M = M0
    for t in range(1, 5):
        M = muon.momentum_accumulate(M, np.zeros_like(M0), 0.9)
        assert np.allclose(M, M0 * 0.9 ** t, rtol=1e-15, atol=0)


def test_frobenius_closed_forms_and_library():
    assert muon.frobenius_norm(np.ones((3, 7))) == math.sqrt(21)
    Q, _ = np.linalg.qr(np.random.default_rng(1).standard_normal((12, 5)))
    assert abs(muon.frobenius_norm(Q.T) - math.sqrt(5)) < 1e-14
    X = random_case(23, 31, 47).astype(np.float64)
    assert abs(muon.frobenius_norm(X) - np.linalg.norm(X, "fro")) < 1e-12 * np.linalg.norm(X)
    big = random_case(24, 2100, 2000)            # takes the NumPy-sum branch
    assert abs(muon.frobenius_norm(big) / np.linalg.norm(big.astype(np.float64)) - 1) < 1e-13


def orthonormal(seed, r, c):
    m = min(r, c)
    Q, _ = np.linalg.qr(np.random.default_rng(seed).standard_normal((max(r, c), m)))
    return Q if r >= c else Q.T            # r x c, orthonormal columns or rows


@pytest.mark.parametrize("shape", [(6, 10), (10, 6), (7, 7), (1, 5)])
@pytest.mark.parametrize("nesterov", [False, True])
def test_whole_step_closed_form(shape, nesterov):
    """G = alpha Q with Q having orthonormal rows (wide) or columns (tall):
    every singular value of X0 is alpha'/(alpha' sqrt(m) + eps), so O is
    p^K(that) Q and the step is known in closed form."""
    r, c = shape
    m = min(r, c)
    Q = orthonormal(3, r, c)
    alpha, mu, lr, eps, scale = 0.37, 0.9, 0.02, 1e-7, 1.7
    G = alpha * Q
    P = random_case(25, r, c, std=0.02).astype(np.float64)
    M = np.zeros((r, c))
    cfg = muon.StepConfig(ns_steps=5, lr=lr, momentum=mu, eps=eps, nesterov=nesterov)
    P1, M1, O = muon.muon_step_matrix(P, G, M, scale, cfg)
    assert np.array_equal(M1, G)                       # mu * 0 + G
    eff = alpha * (1 + mu) if nesterov else alpha       # Nesterov input G + mu*M1
    s0 = eff / (eff * math.sqrt(m) + eps)
    O_want = p_iter(s0, 5) * Q
    assert np.allclose(O, O_want, rtol=0, atol=1e-13)
    assert np.allclose(P1, P - lr * scale * O_want, rtol=0, atol=1e-15)


@pytest.mark.parametrize("shape", [(6, 10), (10, 6), (7, 7)])
@pytest.mark.parametrize("nesterov", [False, True])
def test_step_from_nonzero_momentum_closed_form(shape, nesterov):
    """G = alpha Q and M0 = beta Q (Q with orthonormal rows or columns):
    M1 = (mu beta + alpha) Q; the Newton-Schulz input is M1, or with
    Nesterov the look-ahead G + mu M1 = (alpha + mu (mu beta + alpha)) Q.
    eps is of the order of ||U||, so X0's singular value
    u / (u sqrt(m) + eps) depends on the input's scale u and O tells the
    inputs apart: a swapped look-ahead mu G + M1 (equal to the right one
    only when M0 = 0) misses the closed form by far more than the tolerance.
    """
    r, c = shape
    m = min(r, c)
    Q = orthonormal(5, r, c)
    alpha, beta, mu, lr, eps, scale = 0.37, -0.81, 0.9, 0.02, 0.6, 1.3
    P = random_case(28, r, c, std=0.02).astype(np.float64)
    cfg = muon.StepConfig(ns_steps=5, lr=lr, momentum=mu, eps=eps, nesterov=nesterov)
    P1, M1, O = muon.muon_step_matrix(P, alpha * Q, beta * Q, scale, cfg)
    assert np.allclose(M1, (mu * beta + alpha) * Q, rtol=0, atol=1e-15)

    def o_for(u):
        s0 = abs(u) / (abs(u) * math.sqrt(m) + eps)
        return math.copysign(p_iter(s0, 5), u) * Q
    u = alpha + mu * (mu * beta + alpha) if nesterov else mu * beta + alpha
    assert np.allclose(O, o_for(u), rtol=0, atol=1e-13)
    assert np.allclose(P1, P - lr * scale * o_for(u), rtol=0, atol=1e-15)
    if nesterov:
        swapped = mu * alpha + (mu * beta + alpha)
        assert np.max(np.abs(o_for(swapped) - o_for(u))) > 1e-2


def test_momentum_and_update_match_scalar_loops():
    """Element-by-element Python float loops of M <- mu M + G and
    P <- P - lr s O give the oracle's arrays bit for bit (both are one
    correctly rounded fp64 multiply-add sequence per element)."""
    G = random_case(26, 3, 4).astype(np.float64)
    M0 = random_case(27, 3, 4).astype(np.float64)
    P = random_case(29, 3, 4).astype(np.float64)
    O = random_case(31, 3, 4).astype(np.float64)
    mu, lr, s = 0.95, 0.02, 1.7
    M1 = muon.momentum_accumulate(M0, G, mu)
    P1 = muon.scaled_update(P, O, lr, s)
    for i in range(3):
        for j in range(4):
            assert M1[i, j] == float(mu) * float(M0[i, j]) + float(G[i, j])
            assert P1[i, j] == float(P[i, j]) - (lr * s) * float(O[i, j])


def test_muon_step_list_is_per_matrix():
    cfg = muon.StepConfig()
    mats = [(random_case(30 + i, r, c, 0.02), random_case(40 + i, r, c),
             np.zeros((r, c)), 1.0 + i) for i, (r, c) in enumerate([(3, 5), (8, 2), (4, 4)])]
    Ps, Ms, Os = muon.muon_step(*zip(*mats), cfg)
    for (P, G, M, s), P1, M1, O in zip(mats, Ps, Ms, Os):
        p1, m1, o = muon.muon_step_matrix(P, G, M, s, cfg)
        assert np.array_equal(p1, P1) and np.array_equal(m1, M1) and np.array_equal(o, O)
