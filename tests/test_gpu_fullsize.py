"""Parity at full workload sizes, in the launch configuration bench.py times.

The whole matrix set runs in one ``muon_step`` call with a packed param
buffer (``dmuon_muon_step_packed``, as bench.py times it), with the gradients
read from one packed buffer; every packed slot must equal its updated param
bit for bit.  A sample of matrices (one of every shape, from the
first and the last layer) gets seeded inputs from ``synth`` and is checked
against the fp64 oracle; the other matrices get device-generated values and
only shape the launch.
"""

import numpy as np
import pytest

from _gpu_util import Case, check_step, say, to_dev, to_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def nsd():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import newton_schulz_dmuon_amd as m
    m.load()
    return m


def run_set(nsd, w, shapes, sample, opts):
    """One step over ``shapes`` (list of (global index, name, r, c)); returns
    the GPU outputs of the sampled positions and the oracle's."""
    from synth import matrix_inputs, update_scale
    numels = [r * c for _, _, r, c in shapes]
    offs, total = nsd.pack_offsets(numels, 128)
    dev = torch.device("cuda")
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    gpacked = torch.empty(total, dtype=torch.bfloat16, device=dev)
    P, G, M, O = [], [], [], []
    case = Case([], "bf16", "bf16")
    for pos, ((gi, name, r, c), off) in enumerate(zip(shapes, offs)):
        g = gpacked[off:off + r * c].view(r, c)
        if pos in sample:
            p_h, g_h, m_h = matrix_inputs(w, gi)
            case.shapes.append((r, c)); case.P.append(p_h); case.G.append(g_h)
            case.M.append(m_h); case.scales.append(update_scale(r, c))
            g.copy_(to_dev(g_h, "bf16"))
            P.append(to_dev(p_h, "bf16"))
            O.append(torch.empty_like(P[-1]))
        else:
            g.copy_(torch.randn(r, c, generator=gen, device=dev) * w.grad_std)
            P.append((torch.randn(r, c, generator=gen, device=dev) * w.param_std).to(torch.bfloat16))
            O.append(None)
        G.append(g)
        M.append(torch.zeros(r, c, dtype=torch.float32, device=dev))
    scales = [update_scale(r, c) for _, _, r, c in shapes]
    # orth_out only for the sampled matrices: the binding takes None entries
    # as "no output" (NULL pointer)
    ppacked = torch.empty(total, dtype=torch.bfloat16, device=dev)
    nsd.muon_step(P, G, M, scales, opts, orth_out=O, packed=ppacked, packed_offsets=offs)
    torch.cuda.synchronize()
    for p, off in zip(P, offs):
        slot = ppacked[off:off + p.numel()].view(p.shape)
        assert torch.equal(slot.view(torch.int16), p.view(torch.int16))
    gpu = ([to_host(P[i]) for i in sorted(sample)], [to_host(M[i]) for i in sorted(sample)],
           [to_host(O[i]) for i in sorted(sample)])
    say(f"  gpu step done ({len(shapes)} matrices); oracle on {len(sample)}")
    return case, gpu


def sample_positions(shapes):
    """First occurrence of each distinct shape in the first layer and the
    last one (every shape appears in both)."""
    seen, pos = set(), []
    last_layer = max(int(n.split(".")[1]) for _, n, _, _ in shapes)
    for layer in (0, last_layer):
        for i, (_, n, r, c) in enumerate(shapes):
            if int(n.split(".")[1]) == layer and (layer, r, c) not in seen:
                seen.add((layer, r, c))
                pos.append(i)
    return pos


@pytest.mark.parametrize("gram_ns", [False, True])
def test_llama31_8b_owner0_share(nsd, gram_ns):
    """The benchmark workload: owner 0's 28 matrices of Llama-3.1-8B, with the
    direct chain and with the Gram-space chain (k, gate, up and down take it;
    q keeps the direct one)."""
    from synth import workload
    w = workload(4)
    numels = [r * c for _, r, c in w.shapes]
    owners, _ = nsd.partition_lpt(numels, w.n_owners)
    shapes = [(i, n, r, c) for i, ((n, r, c), o) in enumerate(zip(w.shapes, owners)) if o == 0]
    assert len(shapes) == 28
    seen, sample = set(), set()
    for pos, (_, _, r, c) in enumerate(shapes):
        if (r, c) not in seen:
            seen.add((r, c)); sample.add(pos)
    assert len(sample) == 4   # q, k, gate/up (tall), down (wide)
    say(f"llama-3.1-8b owner 0: 28 matrices, gram_ns {gram_ns}")
    opts = nsd.StepOptions(gram_ns=gram_ns)
    case, gpu = run_set(nsd, w, shapes, sample, opts)
    err = check_step(case, opts, gpu, case.run_oracle(opts))
    say(f"  worst O rel err {err:.3e}")


FULL_SET_CASES = [(3, 5, False), (3, 5, True)] + \
    [(5, k, g) for k in (3, 5, 8) for g in (False, True)]


@pytest.mark.parametrize("wid,k,gram_ns", FULL_SET_CASES)
def test_full_model_sets(nsd, wid, k, gram_ns):
    """All 28 layers of Llama-3.2-3B and Qwen2.5-7B (196 matrices) in one step;
    sampled matrices checked against the oracle.  Llama-3.2-3B: one of every
    shape from the first and the last layer.  Qwen2.5-7B at ns_steps 5: every
    shape of the first layer; at ns_steps 3 and 8: q, k and v of the first
    and the last layer, and gate (18944 x 3584, tall) and down
    (3584 x 18944, wide) of the first layer.  up has gate's shape and takes
    the same code path."""
    from synth import workload
    w = workload(wid)
    shapes = [(i, n, r, c) for i, (n, r, c) in enumerate(w.shapes)]
    pos = sample_positions(shapes)
    layer = lambda p: int(shapes[p][1].split(".")[1])
    big = lambda p: shapes[p][2] * shapes[p][3] > 4096 * 4096
    if wid == 5 and k == 5:
        sample = {p for p in pos if layer(p) == 0}
    elif wid == 5:
        sample = {p for p in pos if not big(p) or layer(p) == 0}
    else:
        sample = set(pos)
    say(f"{w.name}: {len(shapes)} matrices, ns_steps {k}, gram_ns {gram_ns}, {len(sample)} checked")
    opts = nsd.StepOptions(ns_steps=k, gram_ns=gram_ns)
    case, gpu = run_set(nsd, w, shapes, sample, opts)
    err = check_step(case, opts, gpu, case.run_oracle(opts))
    say(f"  worst O rel err {err:.3e}")


@pytest.mark.parametrize("wid", [3, 4])
def test_gram_and_direct_chains_agree_on_every_matrix(nsd, wid):
    """Every matrix of the set, not a sample: the Gram-space step (merged
    launches of both chains) and the direct-chain step, on the same device
    inputs, give O within 3e-2 of each other per matrix (each is within
    about 1.5e-2 of fp64 on these inputs).  A tile or table of a merged
    launch that named the wrong matrix or buffer would show as a gross
    mismatch on the matrices it touched."""
    from synth import update_scale, workload
    w = workload(wid)
    shapes = [(r, c) for _, r, c in w.shapes]
    if w.n_owners > 1:
        owners, _ = nsd.partition_lpt([r * c for r, c in shapes], w.n_owners)
        shapes = [s for s, o in zip(shapes, owners) if o == w.owner]
    dev = torch.device("cuda")
    gen = torch.Generator(device=dev)
    gen.manual_seed(11)
    G = [(torch.randn(r, c, generator=gen, device=dev) * w.grad_std).to(torch.bfloat16)
         for r, c in shapes]
    P0 = [(torch.randn(r, c, generator=gen, device=dev) * w.param_std).to(torch.bfloat16)
          for r, c in shapes]
    scales = [update_scale(r, c) for r, c in shapes]
    out = {}
    for gram in (False, True):
        P = [p.clone() for p in P0]
        M = [torch.zeros(r, c, dtype=torch.float32, device=dev) for r, c in shapes]
        O = [torch.empty_like(p) for p in P]
        nsd.muon_step(P, G, M, scales, nsd.StepOptions(gram_ns=gram), orth_out=O)
        torch.cuda.synchronize()
        out[gram] = O
        del P, M
    worst = 0.0
    for i, (r, c) in enumerate(shapes):
        a, b = out[False][i].float(), out[True][i].float()
        d = float(torch.linalg.norm(a - b) / torch.linalg.norm(a))
        worst = max(worst, d)
        assert d <= 3e-2, (i, (r, c), d)
    say(f"{w.name}: {len(shapes)} matrices, worst direct/gram O difference {worst:.3e}")
