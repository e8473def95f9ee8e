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


def _run(nsd, case, opts, noalloc=False):
    from _gpu_util import to_dev
    P = [to_dev(p, case.pdt) for p in case.P]
    G = [to_dev(g, case.gdt) for g in case.G]
    M = [to_dev(m, "f32") for m in case.M]
    O = [torch.empty_like(p) for p in P]
    ws = None
    if noalloc:
        nsd.muon_step_noalloc(P, G, M, case.scales, opts, orth_out=O)
    else:
        ws = nsd.Workspace()
        nsd.muon_step(P, G, M, case.scales, opts, orth_out=O, workspace=ws)
    torch.cuda.synchronize()
    flags = nsd.nonfinite_flags(P, opts, ws).cpu().tolist() if opts.check_finite and ws is not None else None
    return [t.float().cpu() for t in P + M + O], flags


def test_chain_launch_with_nesterov_and_finite_check(nsd):
    """Nesterov look-ahead and the non-finite check in the chained mode: the
    same bits as the grouped launches with the same flags (shapes whose
    grouped launches run whole 256-tiles), and every flag zero."""
    shapes = [(2048, 4096)] * 4 + [(4096, 4096)] * 2
    base = dict(ns_steps=5, gram_ns=True, nesterov=True, check_finite=True)
    grouped = nsd.StepOptions(**base)
    L = nsd.step_launches(shapes, grouped, tiles=True)
    assert all(t in (0, 256) for _, _, t in L) and all(f > 0 for kd, f, t in L if t), L
    case = Case(shapes, "bf16", "bf16", seed=97, m_std=1e-3)
    want, wflags = _run(nsd, case, grouped)
    got, flags = _run(nsd, case, nsd.StepOptions(chain_launch=True, **base))
    for i, (x, y) in enumerate(zip(got, want)):
        assert torch.equal(x, y), i
    assert flags == wflags == [0] * len(shapes)
    say("chained step with Nesterov and the non-finite check: bit-equal to the grouped launches")


def test_chain_status_word_is_cleared_and_stays_zero(nsd):
    """The status word of the chained step (dmuon_chain_status_offset): the
    step clears it (here pre-set to 7) and no wait gives up, so it reads 0
    after the step."""
    from _gpu_util import to_dev
    shapes = [(300, 700), (700, 300), (513, 513), (1024, 2048)]
    opts = nsd.StepOptions(ns_steps=5, gram_ns=True, chain_launch=True)
    case = Case(shapes, "bf16", "bf16", seed=96, m_std=1e-3)
    P = [to_dev(p, case.pdt) for p in case.P]
    G = [to_dev(g, case.gdt) for g in case.G]
    M = [to_dev(m, "f32") for m in case.M]
    ws = nsd.Workspace()
    ws.get(nsd.workspace_bytes(P, opts), P[0].device)
    word = nsd.chain_status(P, opts, ws)
    word.fill_(7)
    torch.cuda.synchronize()
    nsd.muon_step(P, G, M, case.scales, opts, workspace=ws)
    torch.cuda.synchronize()
    assert word.item() == 0
    say("chained step: status word cleared, no wait gave up")


def test_chain_launch_without_allocation(nsd):
    """The chained mode through the entry point that allocates nothing (its
    tickets and counters in the static scratch): the same bits as the
    chained step with a workspace, on two calls in a row (the second
    smaller), and within the bars of the oracle."""
    for k, (shapes, ns) in enumerate([([(300, 700), (700, 300), (513, 513), (1024, 2048)], 5),
                                      ([(200, 600), (17, 33)], 8)]):
        opts = nsd.StepOptions(ns_steps=ns, gram_ns=True, chain_launch=True)
        case = Case(shapes, "bf16", "bf16", seed=98 + k, m_std=1e-3)
        got, _ = _run(nsd, case, opts, noalloc=True)
        want, _ = _run(nsd, case, opts)
        for i, (x, y) in enumerate(zip(got, want)):
            assert torch.equal(x, y), (k, i)
        n = len(shapes)
        err = check_step(case, opts, ([x.double().numpy() for x in got[:n]],
                                      [x.double().numpy() for x in got[n:2 * n]],
                                      [x.double().numpy() for x in got[2 * n:]]), case.run_oracle(opts))
        say(f"chained step without allocation {shapes}: bit-equal; O rel err {err:.3e}")
