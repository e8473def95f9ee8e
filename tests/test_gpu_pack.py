"""GPU pack / unpack: bit-exact against the oracle's packed buffer."""

import numpy as np
import pytest

from oracle import pack as refpack
from oracle import partition as refp
from synth import random_case

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def nsd():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import newton_schulz_dmuon_amd as m
    m.load()
    return m


def bits(t):
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.view(torch.int32).cpu().numpy().view(np.uint32)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("align", [8, 128])
def test_pack_unpack_bit_exact(nsd, dt, align):
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    shapes = [(300, 700), (1, 1), (17, 33), (1024, 64), (5, 3), (700, 301)]
    host = [random_case(50 + i, r, c, 1.0, dt) for i, (r, c) in enumerate(shapes)]
    mats = [torch.from_numpy(h).to(tdt).cuda() for h in host]
    if dt == "f32" and align == 8:
        align = 4   # 16-byte aligned slots
    offs, total = nsd.pack_offsets([r * c for r, c in shapes], align)
    packed = torch.full((total,), -7.0, dtype=tdt, device="cuda")
    nsd.pack(mats, offs, packed)
    torch.cuda.synchronize()
    want = refpack.pack([bits(m).reshape(m.shape) for m in mats], offs, total,
                        fill=bits(torch.tensor([-7.0], dtype=tdt))[0])
    assert np.array_equal(bits(packed), want)
    outs = [torch.zeros_like(m) for m in mats]
    nsd.unpack(packed, outs, offs)
    torch.cuda.synchronize()
    for m, o in zip(mats, outs):
        assert np.array_equal(bits(m), bits(o))


def test_pack_llama8b_owner_share_offsets(nsd):
    """Offsets of owner 0's Llama-3.1-8B share: host planner vs oracle."""
    from synth import LLAMA31_8B, model_shapes
    shapes = model_shapes(**LLAMA31_8B)
    numels = [r * c for _, r, c in shapes]
    owner, _ = nsd.partition_lpt(numels, 8)
    mine = [numels[i] for i in range(len(numels)) if owner[i] == 0]
    assert nsd.pack_offsets(mine, 128) == refp.pack_offsets(mine, 128)


@pytest.mark.parametrize("pdt,k", [("bf16", 5), ("bf16", 0), ("f32", 2)])
def test_step_packed_equals_step_then_pack(nsd, pdt, k):
    """dmuon_muon_step_packed against dmuon_muon_step followed by dmuon_pack,
    both through the C ABI on the same inputs: params, momenta and the packed
    buffer bit for bit (the gaps between slots keep their fill).  The step's
    own parity with the oracle is checked in test_gpu_step.py."""
    from _gpu_util import Case, to_dev, torch_dtype
    shapes = [(300, 700), (700, 300), (17, 33), (256, 256), (1, 300)]
    case = Case(shapes, pdt, "bf16", seed=11, m_std=1e-3)
    opts = nsd.StepOptions(ns_steps=k)
    offs, total = nsd.pack_offsets([r * c for r, c in shapes], 128)

    def run(fused):
        P = [to_dev(p, pdt) for p in case.P]
        G = [to_dev(g, "bf16") for g in case.G]
        M = [to_dev(m, "f32") for m in case.M]
        packed = torch.full((total,), -3.0, dtype=torch_dtype(pdt), device="cuda")
        if fused:
            nsd.muon_step(P, G, M, case.scales, opts, packed=packed, packed_offsets=offs)
        else:
            nsd.muon_step(P, G, M, case.scales, opts)
            nsd.pack(P, offs, packed)
        torch.cuda.synchronize()
        return P, M, packed

    P1, M1, k1 = run(True)
    P2, M2, k2 = run(False)
    for a, b in zip(P1, P2):
        assert np.array_equal(bits(a), bits(b))
    for a, b in zip(M1, M2):
        assert np.array_equal(bits(a), bits(b))
    assert np.array_equal(bits(k1), bits(k2))
    fill = bits(torch.tensor([-3.0], dtype=torch_dtype(pdt)))[0]
    kb = bits(k1)
    for p, off in zip(P1, offs):
        assert np.array_equal(kb[off:off + p.numel()], bits(p).reshape(-1))
    ends = [off + p.numel() for p, off in zip(P1, offs)]
    gaps = np.ones(total, bool)
    for off, end in zip(offs, ends):
        gaps[off:end] = False
    assert np.all(kb[gaps] == fill)
