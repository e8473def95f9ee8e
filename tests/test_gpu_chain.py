"""GPU tests of the chained mode (DMUON_FLAG_CHAIN_LAUNCH): every bf16
Newton-Schulz product of a step in one dependency-driven launch, each
matrix's tiles on one XCD, waiting per matrix for its previous stage.

Parity against the fp64 oracle at the bars of the grouped launches, and bit
equality with the grouped launches where those run whole 256-tiles (same
tile code, same K order): any missed wait or stale read shows as a
difference."""

import numpy as np
import pytest

from _gpu_util import Case, check_step, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def nsd():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import newton_schulz_dmuon_amd as m
    m.load()
    return m


@pytest.mark.parametrize("shapes,k,gram", [
    ([(300, 700), (700, 300), (513, 513), (1024, 2048)], 5, True),   # both chains, ragged
    ([(1000, 1500), (129, 640), (17, 33)], 8, False),                 # pairs; an fp32 small matrix beside
    ([(1536, 1536), (256, 1536), (1536, 4608)], 6, True),             # Gram-space pairs (P, T)
    ([(2, 300), (300, 2), (256, 256)], 3, False),                     # fp32 chains, one bf16 matrix
])
def test_chain_launch_matches_oracle(nsd, shapes, k, gram):
    opts = nsd.StepOptions(ns_steps=k, gram_ns=gram, chain_launch=True)
    L = nsd.step_launches(shapes, opts)
    assert "chain" in [kd for kd, _ in L]
    say(f"chained step {shapes}, ns_steps {k}, gram_ns {gram}: {len(L)} launches")
    case = Case(shapes, "bf16", "bf16", seed=90 + k, m_std=1e-3)
    err = check_step(case, opts, case.run_gpu(opts), case.run_oracle(opts))
    say(f"  worst O rel err {err:.3e}")


@pytest.mark.parametrize("gram", [False, True])
def test_chain_launch_equals_grouped_launches(nsd, gram):
    """Shapes whose grouped launches all run whole 256-tiles (at least 256
    tiles each: no split K, no 128-tiles): the chained step gives the same
    bits, twice in a row (the counters start from zero each step)."""
    shapes = [(2048, 4096)] * 4 + [(4096, 4096)] * 2
    grouped = nsd.StepOptions(ns_steps=5, gram_ns=gram)
    L = nsd.step_launches(shapes, grouped, tiles=True)
    assert all(t in (0, 256) for _, _, t in L) and all(f > 0 for kd, f, t in L if t), L
    chained = nsd.StepOptions(ns_steps=5, gram_ns=gram, chain_launch=True)
    case = Case(shapes, "bf16", "bf16", seed=95, m_std=1e-3)
    want = case.run_gpu(grouped)
    for rep in range(2):
        got = case.run_gpu(chained)
        # host copies are float64 images of the bf16 / fp32 values: equal
        # values are equal bits (the step writes no NaN here)
        for name, g, w in zip(("param", "momentum", "orth_out"), got, want):
            for i, (x, y) in enumerate(zip(g, w)):
                assert np.array_equal(x, y), (rep, name, i, shapes[i], int((x != y).sum()))
    say(f"chained step bit-equal to the grouped launches (gram_ns {gram}), twice")
