"""Pins the bf16 error model that the K-dependent bf16 tolerance rests on."""

import numpy as np
import pytest

from _bf16_model import ns_bf16_storage, tol_o_bf16
from oracle import muon
from synth import matrix_inputs, workload


@pytest.fixture(scope="module")
def qwen7b_k():
    w = workload(5)
    _, G, _ = matrix_inputs(w, 1)            # layers.0.k_proj, 512 x 3584
    X0, _ = muon.normalise_and_orient(G, 1e-7)
    return X0


@pytest.mark.parametrize("k,lo,hi", [(3, 1e-3, 6e-3), (5, 8e-3, 2e-2), (8, 2e-2, 3e-2)])
def test_bf16_storage_error_grows_with_iterations(qwen7b_k, k, lo, hi):
    ref = muon.newton_schulz(qwen7b_k, *muon.QUINTIC, k)
    emu = ns_bf16_storage(qwen7b_k, *muon.QUINTIC, k)
    err = np.linalg.norm(emu - ref) / np.linalg.norm(ref)
    assert lo < err < hi, err
    assert err < tol_o_bf16(k) / 1.4


def test_quintic_expands_errors_inside_its_band():
    a, b, c = muon.QUINTIC
    s = np.linspace(0.6818, 1.2024, 10001)
    dp = a + 3 * b * s ** 2 + 5 * c * s ** 4
    assert np.max(np.abs(dp)) > 1.0          # some band points amplify errors
