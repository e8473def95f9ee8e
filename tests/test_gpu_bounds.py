"""Writes stay inside their buffers: a step with a workspace of exactly
dmuon_workspace_bytes() (and params, momenta, orth_out and the packed buffer
placed inside larger buffers) leaves canary bytes around every one of them
untouched.  Both chains, with and without the non-finite flags, ragged
shapes over several tiles."""

import ctypes

import numpy as np
import pytest

from _gpu_util import Case, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

CANARY = 4096   # bytes on each side
FILL = 0x5A


@pytest.fixture(scope="module")
def nsd():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import newton_schulz_dmuon_amd as m
    m.load()
    return m


def _guarded(nbytes):
    """A uint8 device buffer with CANARY filled bytes on each side; returns
    (whole, inner view)."""
    whole = torch.full((nbytes + 2 * CANARY,), FILL, dtype=torch.uint8, device="cuda")
    return whole, whole[CANARY:CANARY + nbytes]


def _intact(whole, nbytes):
    head = whole[:CANARY]
    tail = whole[CANARY + nbytes:]
    return bool((head == FILL).all()) and bool((tail == FILL).all())


@pytest.mark.parametrize("gram,k,check", [(False, 5, False), (True, 5, True), (True, 8, False),
                                          (True, 6, True), (False, 0, True)])
def test_step_writes_stay_in_bounds(nsd, gram, k, check):
    from newton_schulz_dmuon_amd import _lib
    from newton_schulz_dmuon_amd.api import matrices
    shapes = [(300, 700), (700, 300), (513, 513), (17, 100), (257, 1000)]
    say(f"bounds: gram {gram}, ns_steps {k}, check_finite {check}")
    case = Case(shapes, "bf16", "bf16", seed=50, m_std=1e-3)
    opts = nsd.StepOptions(ns_steps=k, gram_ns=gram, check_finite=check)
    guards = []

    def place(arr, dt):
        t = torch.from_numpy(np.ascontiguousarray(arr, np.float32)).to(dt)
        nb = t.numel() * t.element_size()
        whole, inner = _guarded(nb)
        view = inner.view(dt).view(t.shape)
        view.copy_(t.cuda())
        guards.append((whole, nb))
        return view

    P = [place(p, torch.bfloat16) for p in case.P]
    G = [place(g, torch.bfloat16) for g in case.G]
    M = [place(m, torch.float32) for m in case.M]
    O = [place(np.zeros_like(p), torch.bfloat16) for p in case.P]
    offs, total = nsd.pack_offsets([r * c for r, c in shapes], 128)
    pwhole, pinner = _guarded(total * 2)
    packed = pinner.view(torch.bfloat16)
    guards.append((pwhole, total * 2))
    need = nsd.workspace_bytes(P, opts)
    wwhole, winner = _guarded(need)
    guards.append((wwhole, need))
    arr, n = matrices(P, G, M, case.scales, O, offs)
    cfg = opts.to_c()
    lib = nsd.load()
    stream = torch.cuda.current_stream().cuda_stream
    _lib.check(lib.dmuon_muon_step_packed(arr, n, ctypes.byref(cfg), winner.data_ptr(), need,
                                          packed.data_ptr(), _lib.BF16, total, stream, None, 0))
    torch.cuda.synchronize()
    for i, (whole, nb) in enumerate(guards):
        assert _intact(whole, nb), f"canary overwritten around buffer {i}"
    # the step did run: every O is finite and nonzero
    for o in O:
        assert torch.isfinite(o.float()).all() and o.float().abs().sum() > 0
