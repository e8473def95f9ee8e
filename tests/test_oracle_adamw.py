"""Pins of the AdamW oracle: torch.optim.AdamW in float64 on the CPU (a
library routine), and closed forms."""

import numpy as np
import pytest
import torch

from oracle.adamw import AdamWConfig, adamw_step
from synth import random_case


@pytest.mark.parametrize("wd", [0.0, 0.01, 0.1])
def test_matches_torch_adamw_fp64(wd):
    P0 = random_case(1, 13, 29, 0.02).astype(np.float64)
    grads = [random_case(10 + t, 13, 29, 1e-2).astype(np.float64) for t in range(6)]
    p = torch.nn.Parameter(torch.from_numpy(P0.copy()))
    opt = torch.optim.AdamW([p], lr=3e-3, betas=(0.8, 0.99), eps=1e-6, weight_decay=wd)
    P, M, V = P0, np.zeros_like(P0), np.zeros_like(P0)
    for t, g in enumerate(grads, start=1):
        p.grad = torch.from_numpy(g.copy())
        opt.step()
        P, M, V = adamw_step(P, g, M, V, AdamWConfig(3e-3, 0.8, 0.99, 1e-6, wd, t))
        st = opt.state[p]
        # torch forms the first moment with lerp, m + (1 - beta1)(g - m), which
        # rounds differently where the two terms nearly cancel: absolute
        # tolerance relative to the tensor's scale
        assert np.allclose(P, p.detach().numpy(), rtol=1e-13, atol=1e-16)
        assert np.allclose(M, st["exp_avg"].numpy(), rtol=1e-12, atol=1e-15 * np.abs(M).max())
        assert np.allclose(V, st["exp_avg_sq"].numpy(), rtol=1e-12, atol=1e-15 * np.abs(V).max())


def test_constant_gradient_closed_form():
    """With a constant gradient the bias-corrected moments equal g and g^2 at
    every step, so each update is lr * g / (|g| + eps)."""
    g = random_case(3, 7, 5, 1.0).astype(np.float64)
    P, M, V = np.zeros_like(g), np.zeros_like(g), np.zeros_like(g)
    lr, eps = 1e-2, 1e-8
    for t in range(1, 9):
        P_prev = P
        P, M, V = adamw_step(P, g, M, V, AdamWConfig(lr, 0.9, 0.999, eps, 0.0, t))
        assert np.allclose(P_prev - P, lr * g / (np.abs(g) + eps), rtol=1e-12, atol=0)


def test_zero_gradient_is_pure_decay():
    P0 = random_case(4, 6, 6, 0.5).astype(np.float64)
    P, M, V = P0, np.zeros_like(P0), np.zeros_like(P0)
    for t in range(1, 5):
        P, M, V = adamw_step(P, np.zeros_like(P0), M, V, AdamWConfig(0.1, 0.9, 0.999, 1e-8, 0.2, t))
        assert np.allclose(P, P0 * (1 - 0.1 * 0.2) ** t, rtol=1e-14, atol=0)
        assert not M.any() and not V.any()
