"""GPU parity of steps over seeded random shape sets that hold both chains
at once: square and near-square matrices (direct chain), wide and tall ones
with m >= 128 (Gram-space chain), and small ones (m < 128, the direct chain
in fp32).  The two bf16 chains share grouped launches, same-kind or a Gram
launch with a Square launch, in positions that vary with the set and with
ns_steps (pairs from 6 iterations on, phases of two); every matrix of every
set is checked against the fp64 oracle at the usual bars."""

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


def random_set(seed):
    """Five to eight shapes: two near-square (direct chain), two to four with
    aspect >= 2 and m >= 128 (Gram-space chain, either orientation), one or
    two small ones (m < 128), at sizes the oracle finishes in seconds."""
    rng = np.random.default_rng(1000 + seed)
    shapes = []
    for _ in range(2):
        m = int(rng.integers(128, 700))
        shapes.append((m, int(m * rng.uniform(0.8, 1.9))))
    for _ in range(int(rng.integers(2, 5))):
        m = int(rng.integers(128, 520))
        n = int(m * rng.uniform(2.0, 8.0))
        shapes.append((m, n) if rng.random() < 0.5 else (n, m))
    for _ in range(int(rng.integers(1, 3))):
        m = int(rng.integers(1, 128))
        shapes.append((m, int(rng.integers(m, 900))))
    return shapes


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("k", [5, 6, 8])
def test_random_sets_with_both_chains(nsd, seed, k):
    shapes = random_set(seed)
    opts = nsd.StepOptions(ns_steps=k, gram_ns=True)
    kinds = [kd for kd, f in nsd.step_launches(shapes, opts)]
    say(f"seed {seed} ns_steps {k}: {shapes}; {len(kinds)} launches, "
        f"{kinds.count('gram_square')} mixed")
    case = Case(shapes, "bf16", "bf16", seed=40 + seed, m_std=1e-3)
    err = check_step(case, opts, case.run_gpu(opts), case.run_oracle(opts))
    say(f"  worst O rel err {err:.3e}")
