"""fp64 reference for the owner's Muon update of one matrix.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What the method computes, and where it is stated
------------------------------------------------
DMuon landing page ("DMuon", intro and "LLM Pretraining"): every Muon-target
matrix parameter has a single owner rank; the owner holds the full parameter,
receives the reduced gradient and runs Newton-Schulz on it alone, once per
step.  The optimizer defaults shown there are ``lr=0.02`` and ``ns_steps=5``.
"Z2 vs Z3 Modes", "Byte cost per step": Newton-Schulz runs once, on the owner,
instead of on every rank.

The pages name the iteration ("Newton-Schulz", and a "Gram Newton-Schulz"
kernel in the credits) but print no formula, coefficient, momentum rule,
epsilon or update scale.  This oracle takes the standard Muon update (Jordan
et al., 2024) as the plain reading of those names:

  step 1  momentum accumulation, heavy-ball sum: M <- mu * M + G
  step 2  Frobenius normalisation X0 = U / (||U||_F + eps) of U = M (or of the
          look-ahead G + mu*M when Nesterov is on), turned to wide
          orientation: X0 <- X0^T when rows > cols, so X0 is m x n, m <= n
  step 3  ns_steps iterations  A = X X^T ;  X <- a X + (b A + c A^2) X,
          with the coefficients (a, b, c) passed in
  step 4  back to r x c: O = X^T if step 2 transposed, else X
  step 5  scaled update P <- P - lr * scale * O, with a per-matrix scale
          passed in

Everything is float64; there is no blocking, symmetry shortcut or fusion.
The GPU path stores X, A, B in bf16 (or fp32 in its fp32 mode) and is compared
against these values within tolerances.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

# Public Muon defaults (Jordan et al., 2024).  Not printed on the DMuon pages;
# passed in everywhere, these are only defaults.
QUINTIC = (3.4445, -4.7750, 2.0315)
# Textbook Newton-Schulz polar iteration X <- 1.5 X - 0.5 X X^T X.
CUBIC = (1.5, -0.5, 0.0)


@dataclass(frozen=True)
class StepConfig:
    """Step hyper-parameters.  ``lr`` and ``ns_steps`` defaults follow the
    optimizer call on the DMuon landing page ("LLM Pretraining")."""

    a: float = QUINTIC[0]
    b: float = QUINTIC[1]
    c: float = QUINTIC[2]
    ns_steps: int = 5
    lr: float = 0.02
    momentum: float = 0.95
    eps: float = 1e-7
    nesterov: bool = False


def f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def momentum_accumulate(M, G, mu: float) -> np.ndarray:
    """Step 1: heavy-ball momentum buffer, ``M <- mu*M + G``."""
    return mu * f64(M) + f64(G)


def ns_input(M_new, G, mu: float, nesterov: bool) -> np.ndarray:
    """The matrix handed to Newton-Schulz: the new buffer, or with Nesterov
    on, the look-ahead ``G + mu*M_new``."""
    if nesterov:
        return f64(G) + mu * f64(M_new)
    return f64(M_new)


def frobenius_norm(U) -> float:
    """sqrt of the sum of squares: ``math.fsum`` (exactly rounded) for inputs
    up to 4M elements, NumPy's pairwise float64 sum above that."""
    u = f64(U).ravel()
    return math.sqrt(math.fsum((u * u).tolist())) if u.size < 4_000_000 else \
        float(np.sqrt(np.sum(u * u)))


def normalise_and_orient(U, eps: float):
    """Step 2: ``X0 = U / (||U||_F + eps)``, transposed when rows > cols so that
    X0 is m x n with m = min(rows, cols).

    Returns ``(X0, transposed)``."""
    U = f64(U)
    X = U / (frobenius_norm(U) + eps)
    transposed = U.shape[0] > U.shape[1]
    return (X.T.copy() if transposed else X), transposed


def newton_schulz(X, a: float, b: float, c: float, steps: int) -> np.ndarray:
    """Step 3: ``steps`` iterations of ``X <- a X + (b A + c A A) X`` with
    ``A = X X^T``, all dense float64 products."""
    X = f64(X)
    for _ in range(steps):
        A = X @ X.T
        B = b * A + c * (A @ A)
        X = a * X + B @ X
    return X


def scaled_update(P, O, lr: float, scale: float) -> np.ndarray:
    """Step 5: ``P <- P - lr * scale * O``, scale per matrix."""
    return f64(P) - (lr * scale) * f64(O)


def orthogonalise(U, cfg: StepConfig) -> np.ndarray:
    """Steps 2-4: the Newton-Schulz output O in the r x c orientation of U."""
    X, transposed = normalise_and_orient(U, cfg.eps)
    X = newton_schulz(X, cfg.a, cfg.b, cfg.c, cfg.ns_steps)
    return X.T if transposed else X


def muon_step_matrix(P, G, M, scale: float, cfg: StepConfig):
    """One owner-side Muon step for one matrix.

    Returns ``(P_new, M_new, O)``, all float64 and r x c."""
    M_new = momentum_accumulate(M, G, cfg.momentum)
    U = ns_input(M_new, G, cfg.momentum, cfg.nesterov)
    O = orthogonalise(U, cfg)
    P_new = scaled_update(P, O, cfg.lr, scale)
    return P_new, M_new, O


def muon_step(params, grads, moms, scales, cfg: StepConfig):
    """The owner's step over its matrix list: matrices are independent, so
    this is ``muon_step_matrix`` applied to each one in turn."""
    out = [muon_step_matrix(P, G, M, s, cfg)
           for P, G, M, s in zip(params, grads, moms, scales)]
    return [o[0] for o in out], [o[1] for o in out], [o[2] for o in out]
