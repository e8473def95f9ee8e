"""Helpers for the GPU parity tests: seeded inputs, running the HIP step
through the binding, running the oracle on the same inputs, and the
comparison rules."""

from __future__ import annotations

import math
import sys

import numpy as np

from oracle import muon as ref
from synth import random_case, update_scale

TOL_O_BF16 = 2e-2     # relative Frobenius, bf16 chain up to 5 iterations (see _bf16_model)
TOL_O_FP32 = 1e-4     # relative Frobenius, fp32 checking mode
TOL_ELEMENTWISE = 1e-6


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def rel_fro(got, want) -> float:
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    den = np.linalg.norm(want)
    num = np.linalg.norm(got - want)
    return float(num / den) if den > 0 else float(num)


def torch_dtype(dt: str):
    import torch
    return {"bf16": torch.bfloat16, "f32": torch.float32}[dt]


def to_dev(a: np.ndarray, dt: str):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch_dtype(dt)).cuda()


def to_host(t) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def ulp_bf16(x: np.ndarray) -> np.ndarray:
    _, e = np.frexp(np.abs(x).astype(np.float64))
    u = np.ldexp(1.0, e - 8)
    return np.where(x == 0, 2.0 ** -133, u)


def rne_bf16(x: np.ndarray) -> np.ndarray:
    import torch
    return torch.from_numpy(np.asarray(x, np.float64)).to(torch.bfloat16).double().numpy()


class Case:
    """Inputs of one step: shapes, dtypes, seeded values."""

    def __init__(self, shapes, pdt="bf16", gdt="bf16", seed=0, p_std=0.02, g_std=1e-3,
                 m_std=0.0):
        self.shapes = list(shapes)
        self.pdt, self.gdt = pdt, gdt
        self.P, self.G, self.M, self.scales = [], [], [], []
        for i, (r, c) in enumerate(self.shapes):
            base = 10_000 * seed + 10 * i
            self.P.append(random_case(base + 1, r, c, p_std, pdt))
            self.G.append(random_case(base + 2, r, c, g_std, gdt))
            self.M.append(random_case(base + 3, r, c, m_std, "f32") if m_std
                          else np.zeros((r, c), np.float32))
            self.scales.append(update_scale(r, c))

    def run_gpu(self, opts, with_orth=True, workspace=None):
        import torch
        import newton_schulz_dmuon_amd as nsd
        P = [to_dev(p, self.pdt) for p in self.P]
        G = [to_dev(g, self.gdt) for g in self.G]
        M = [to_dev(m, "f32") for m in self.M]
        O = [torch.empty_like(p) for p in P] if with_orth else None
        nsd.muon_step(P, G, M, self.scales, opts, orth_out=O, workspace=workspace)
        torch.cuda.synchronize()
        return ([to_host(p) for p in P], [to_host(m) for m in M],
                [to_host(o) for o in O] if with_orth else None)

    def run_oracle(self, opts):
        cfg = ref.StepConfig(a=opts.a, b=opts.b, c=opts.c, ns_steps=opts.ns_steps, lr=opts.lr,
                             momentum=opts.momentum, eps=opts.eps, nesterov=opts.nesterov)
        return ref.muon_step(self.P, self.G, self.M, self.scales, cfg)


def check_step(case: Case, opts, gpu, want, tol_o=None):
    """Compares one step's outputs; returns the worst O error."""
    from _bf16_model import tol_o_bf16
    tol_o = tol_o or (TOL_O_FP32 if opts.ns_fp32 else tol_o_bf16(opts.ns_steps))
    Pg, Mg, Og = gpu
    Pw, Mw, Ow = want
    worst = 0.0
    for i, (r, c) in enumerate(case.shapes):
        em = rel_fro(Mg[i], Mw[i])
        assert em <= TOL_ELEMENTWISE, (i, (r, c), "momentum", em)
        if Og is not None:
            eo = rel_fro(Og[i], Ow[i])
            worst = max(worst, eo)
            # orth_out is rounded to the param dtype: RNE to bf16 moves each
            # element by at most 2^-9 of itself, so the relative Frobenius
            # error grows by at most 2^-9
            extra = 2.0 ** -9 if case.pdt == "bf16" else 0.0
            assert eo <= tol_o + extra, (i, (r, c), "O", eo)
        P0 = case.P[i].astype(np.float64)
        step = opts.lr * case.scales[i]
        if case.pdt == "f32":
            ed = rel_fro(Pg[i] - P0, Pw[i] - P0)
            assert ed <= tol_o + 1e-5, (i, (r, c), "update", ed)
        else:
            o_err = np.abs(Og[i] - Ow[i]) + ulp_bf16(Og[i]) if Og is not None else \
                np.full((r, c), 0.1 * np.max(np.abs(Ow[i])))
            # P_gpu = RNE_bf16(y), y = P0 - step*o in fp32 with o the fp32 value
            # orth_out rounds: |P_gpu - y| <= ulp(P_gpu)/2 and
            # |y - P64| <= step*|o - O64| <= step*(|O_gpu - O64| + ulp(O_gpu)/2)
            bound = np.maximum(ulp_bf16(Pw[i]), ulp_bf16(Pg[i])) + step * o_err + 1e-12
            bad = np.abs(Pg[i] - Pw[i]) > bound
            if bad.any():
                idx = np.argwhere(bad)[:5]
                for (a, b) in idx:
                    say(f"  param violation at {(int(a), int(b))}: P0 {P0[a, b]!r} gpu {Pg[i][a, b]!r} "
                        f"oracle {Pw[i][a, b]!r} bound {bound[a, b]!r} O_gpu "
                        f"{(Og[i][a, b] if Og is not None else None)!r} O64 {Ow[i][a, b]!r} "
                        f"step {step!r}")
            assert not bad.any(), (i, (r, c), "param", int(bad.sum()))
    return worst
