"""GPU parity of the AdamW step on the non-Muon parameters against the fp64
oracle, over several steps with the state carried on the device."""

import numpy as np
import pytest

from _gpu_util import rel_fro, say, to_dev, to_host, ulp_bf16
from oracle.adamw import AdamWConfig, adamw_step
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


SIZES = [1, 7, 4096, 8193, 100_003, 1_000_000]


@pytest.mark.parametrize("pdt,gdt", [("bf16", "bf16"), ("f32", "f32"), ("f32", "bf16")])
def test_adamw_steps(nsd, pdt, gdt):
    say(f"adamw {pdt}/{gdt} over {len(SIZES)} tensors")
    opts = nsd.AdamWOptions(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)
    P = [random_case(100 + i, 1, n, 0.02, pdt)[0] for i, n in enumerate(SIZES)]
    Pd = [to_dev(p[None], pdt)[0] for p in P]
    Md = [torch.zeros(n, dtype=torch.float32, device="cuda") for n in SIZES]
    Vd = [torch.zeros(n, dtype=torch.float32, device="cuda") for n in SIZES]
    Pw = [p.astype(np.float64) for p in P]
    Mw = [np.zeros(n) for n in SIZES]
    Vw = [np.zeros(n) for n in SIZES]
    acc_ulp = [np.zeros(n) for n in SIZES]   # bf16 rounding allowance so far
    for t in range(1, 4):
        G = [random_case(1000 * t + i, 1, n, 1e-3, gdt)[0] for i, n in enumerate(SIZES)]
        Gd = [to_dev(g[None], gdt)[0] for g in G]
        nsd.adamw_step(Pd, Gd, Md, Vd, t, opts)
        torch.cuda.synchronize()
        cfg = AdamWConfig(opts.lr, opts.beta1, opts.beta2, opts.eps, opts.weight_decay, t)
        for i in range(len(SIZES)):
            Pw[i], Mw[i], Vw[i] = adamw_step(Pw[i], G[i], Mw[i], Vw[i], cfg)
            m, v, p = to_host(Md[i]), to_host(Vd[i]), to_host(Pd[i])
            assert rel_fro(m, Mw[i]) <= 1e-6, (t, i, "exp_avg")
            assert rel_fro(v, Vw[i]) <= 1e-6, (t, i, "exp_avg_sq")
            if pdt == "f32":
                # fp32 arithmetic: a few ulps of the larger of P and the update
                bound = 1e-6 * (np.abs(Pw[i]) + opts.lr) + 1e-12
            else:
                # bf16 storage: the GPU rounds its fp32 result every step while
                # the oracle carries fp64; the moments do not depend on P, so
                # the gap grows by at most one rounding per step, each at the
                # ulp of that step's value (values can shrink across binades)
                acc_ulp[i] = acc_ulp[i] + np.maximum(ulp_bf16(Pw[i]), ulp_bf16(p))
                bound = acc_ulp[i] + 1e-6 * opts.lr * t
            assert np.all(np.abs(p - Pw[i]) <= bound), (t, i, "param",
                                                        float(np.max(np.abs(p - Pw[i]) - bound)))
