"""dmuon_muon_step_noalloc: the step in the library's static per-device
scratch, for callers that cannot allocate.  Through the C ABI, its results
must equal dmuon_muon_step's with a caller workspace bit for bit (same
kernels, same plan, same workspace layout), on consecutive calls whose
second one is smaller than the first (the scratch keeps the first call's
contents), and an input too large for the scratch is refused before any
launch."""

import ctypes

import numpy as np
import pytest

from _gpu_util import Case, check_step, say, to_dev, to_host

torch = pytest.importorskip("torch")


def test_too_large_input_is_refused_without_a_launch():
    """Host-only: fake, never dereferenced pointers; the size check comes
    before the first HIP call."""
    import newton_schulz_dmuon_amd as nsd
    from newton_schulz_dmuon_amd import _lib
    lib = nsd.load()
    base = 1 << 40
    r, c = 4096, 4096           # direct chain: X^T x 2, A, B = 128 MiB of bf16
    n = r * c
    mats = (_lib.Matrix * 1)(_lib.Matrix(base, _lib.BF16, _lib.BF16, base + 4 * n, base + 8 * n,
                                         None, r, c, 1.0, 0, 0))
    cfg = nsd.StepOptions().to_c()
    need = ctypes.c_size_t(0)
    _lib.check(lib.dmuon_workspace_bytes(mats, 1, ctypes.byref(cfg), ctypes.byref(need)))
    assert need.value > _lib.NOALLOC_SCRATCH_BYTES
    rc = lib.dmuon_muon_step_noalloc(mats, 1, ctypes.byref(cfg), None)
    assert rc == _lib.ERR_WORKSPACE_TOO_SMALL
    assert b"static scratch" in lib.dmuon_last_error()


def _step(nsd, case, opts, noalloc):
    P = [to_dev(p, case.pdt) for p in case.P]
    G = [to_dev(g, case.gdt) for g in case.G]
    M = [to_dev(m, "f32") for m in case.M]
    O = [torch.empty_like(p) for p in P]
    if noalloc:
        nsd.muon_step_noalloc(P, G, M, case.scales, opts, orth_out=O)
    else:
        nsd.muon_step(P, G, M, case.scales, opts, orth_out=O)
    torch.cuda.synchronize()
    return P, M, O


@pytest.mark.gpu
def test_noalloc_equals_workspace_step_on_consecutive_calls():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import newton_schulz_dmuon_amd as nsd
    nsd.load()
    calls = [
        # larger first: both chains, ragged tiles; then smaller ones, the
        # last at ns_steps 8 (hi + lo pairs)
        ([(300, 700), (700, 300), (513, 513), (1024, 2048)], 5),
        ([(128, 256), (17, 33)], 5),
        ([(200, 600)], 8),
    ]
    for k, (shapes, ns) in enumerate(calls):
        case = Case(shapes, "bf16", "bf16", seed=30 + k, m_std=1e-3)
        opts = nsd.StepOptions(ns_steps=ns, gram_ns=True)
        say(f"noalloc call {k}: {shapes}, ns_steps {ns}")
        got = _step(nsd, case, opts, noalloc=True)
        want = _step(nsd, case, opts, noalloc=False)
        for name, a, b in zip(("param", "momentum", "orth_out"), got, want):
            for i, (x, y) in enumerate(zip(a, b)):
                assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32),
                                   y.view(torch.int16) if y.dtype == torch.bfloat16 else y.view(torch.int32)), \
                    (k, name, i, shapes[i])
        gpu = ([to_host(p) for p in got[0]], [to_host(m) for m in got[1]], [to_host(o) for o in got[2]])
        err = check_step(case, opts, gpu, case.run_oracle(opts))
        say(f"  bitwise equal to the workspace step; O rel err vs oracle {err:.3e}")
