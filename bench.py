"""Throughput of the owner-side Muon step on one MI355X.

A step is the owner's whole per-step work on its share of matrices: momentum
accumulation and Frobenius normalisation, ns_steps Newton-Schulz iterations
(bf16 MFMA), the scaled parameter update and the packing of the updated
parameters into the packed buffer the owner broadcasts, all in one
``dmuon_muon_step_packed`` call (the gradients read in place from the owner's
packed gradient buffer; the last Apply writes each updated parameter to its
tensor and to its packed slot).  Inputs are seeded synthetic tensors already
resident in HBM.

The Gram-space chain (DMUON_FLAG_GRAM_NS) runs for the matrices with
max(r,c) >= 2 min(r,c); ``--direct-ns`` runs the direct chain for all.

Prints one JSON line.  ``value`` is the effective Newton-Schulz TFLOP/s:
the direct iteration's algorithmic flops (symmetric products counted as
their upper triangle: m(m+1)n + m^2(m+1) + 2m^2 n per matrix per
iteration) over the whole step time, whichever chain runs, so that it
compares across chains.  The MFMA use is ``pct_bf16_peak``: the flops the
launches execute (``executed_tflops``) over the step time, as a percentage
of the bf16 peak; ``effective_pct_bf16_peak`` is ``value`` over that peak.
"""

from __future__ import annotations

import argparse
import ctypes
import faulthandler
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3    # MI355X dense fp32 MFMA
PEAK_HBM_GBS = 8000.0
METRIC = "Muon step: NS TFLOP/s (% bf16 MFMA peak) + matrices/s on one owner's share"


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def ns_flops(m: int, n: int, k: int) -> dict:
    """Algorithmic flops of k iterations on an m x n (m <= n) matrix."""
    return {"gram": k * m * (m + 1) * n, "square": k * m * m * (m + 1),
            "apply": k * 2 * m * m * n}


def dense_ns_flops(m: int, n: int, k: int) -> int:
    """Flops of k iterations computed densely, as the oracle does: X X^T,
    A A and B X as full products."""
    return k * (2 * m * m * n + 2 * m ** 3 + 2 * m * m * n)


class TraceEvents:
    """One step's worth of timing events (torch's HIP events, created by a
    first record) whose raw handles the traced step re-records."""

    def __init__(self, n: int, stream):
        import torch
        self.ev = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        for e in self.ev:
            e.record(stream)
        self.handles = (ctypes.c_void_p * n)(*[e.cuda_event for e in self.ev])

    def elapsed_ms(self, j: int) -> float:
        return self.ev[j].elapsed_time(self.ev[j + 1])


def measured_traffic(workload_name: str, fp32: bool, kind: str, gram_ns: bool):
    """HBM bytes per launch of the dominant kernel from the committed
    rocprofv3 counter summary (FETCH_SIZE and WRITE_SIZE scaled by a copy
    kernel of known size), or None when the summary is for another workload,
    kernel or chain, or the GEMM source has changed since the counters were
    taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "dominant_kernel_traffic_llama31_8b_owner0.json")
    csrc = os.path.join(ROOT, "newton_schulz_dmuon_amd", "csrc")
    try:
        rec = json.load(open(path))
        # the kernel source, and the host planner that decides each launch's tiles
        sha = {k: hashlib.sha256(open(os.path.join(csrc, f), "rb").read()).hexdigest()
               for k, f in (("gemm", "gemm.hip"), ("host", "host_api.cpp"))}
    except OSError:
        return None
    if fp32 or rec.get("workload") != workload_name or rec.get("gemm_source_sha256") != sha["gemm"] \
            or rec.get("host_source_sha256") != sha["host"] \
            or rec.get("kind") != kind or rec.get("gram_ns") != gram_ns:
        return None
    return rec["traffic_bytes_per_launch"]


def adamw_measure(nsd, torch, dev, stream, steps: int):
    """AdamW on one rank's 1/8 shard of Llama-3.1-8B's non-Muon parameters
    (embeddings, lm_head, norms), bf16 params and grads, fp32 moments."""
    from synth import LLAMA31_8B, LLAMA31_8B_VOCAB, non_muon_sizes
    sizes = [(n, (c + 7) // 8) for n, c in
             non_muon_sizes(LLAMA31_8B["d_model"], LLAMA31_8B["n_layers"], LLAMA31_8B_VOCAB)]
    gen = torch.Generator(device=dev)
    gen.manual_seed(99)
    P = [(torch.randn(c, generator=gen, device=dev) * 0.02).to(torch.bfloat16) for _, c in sizes]
    G = [(torch.randn(c, generator=gen, device=dev) * 1e-3).to(torch.bfloat16) for _, c in sizes]
    M = [torch.zeros(c, dtype=torch.float32, device=dev) for _, c in sizes]
    V = [torch.zeros(c, dtype=torch.float32, device=dev) for _, c in sizes]
    opts = nsd.AdamWOptions()
    for t in range(1, 3):
        nsd.adamw_step(P, G, M, V, t, opts, stream=stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for t in range(3, 3 + steps):
        nsd.adamw_step(P, G, M, V, t, opts, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    elems = sum(c for _, c in sizes)
    nbytes = elems * (2 + 2 + 4 + 4 + 2 + 4 + 4)   # P, G, M, V read; P, M, V written
    return {"tensors": [n for n, _ in sizes], "elements": elems, "ms": round(ms, 4),
            "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1), "bytes_per_elem": 22,
            "peak_gbs": PEAK_HBM_GBS}


def owner_share(w, nsd):
    shapes = w.shapes
    if w.n_owners > 1:
        owners, _ = nsd.partition_lpt([r * c for _, r, c in shapes], w.n_owners)
        shapes = [s for s, o in zip(shapes, owners) if o == w.owner]
    return shapes


def cpu_baseline(w, shapes, ns_steps, budget_s: float):
    """Times the fp64 oracle on a bounded sample of the workload's matrices
    (one matrix per distinct shape, smallest first, while the budget lasts)."""
    import numpy as np
    from oracle import muon as ref
    from synth import normal, update_scale
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    seen, sample = set(), []
    for idx, (name, r, c) in enumerate(shapes):
        if (r, c) not in seen:
            seen.add((r, c))
            sample.append((idx, name, r, c))
    sample.sort(key=lambda s: s[2] * s[3])
    cfg = ref.StepConfig(ns_steps=ns_steps)
    flops, dense, done, t_total = 0, 0, [], 0.0
    per_shape = {}
    for idx, name, r, c in sample:
        P = normal(w.wid, idx, 1, r, c, w.param_std, w.param_dtype)
        G = normal(w.wid, idx, 0, r, c, w.grad_std, w.grad_dtype)
        M = np.zeros((r, c), np.float32)
        t0 = time.perf_counter()
        ref.muon_step_matrix(P, G, M, update_scale(r, c), cfg)
        dt = time.perf_counter() - t0
        t_total += dt
        flops += sum(ns_flops(min(r, c), max(r, c), ns_steps).values())
        dense += dense_ns_flops(min(r, c), max(r, c), ns_steps)
        per_shape[(r, c)] = dt
        done.append(f"{name.split('.')[-1]} {r}x{c}")
        log(f"cpu oracle {r}x{c}: {dt:.2f} s")
        if t_total > budget_s:
            break
    # the smallest sampled matrix again on one BLAS thread
    one_thread = None
    try:
        from threadpoolctl import threadpool_limits
        idx, name, r, c = sample[0]
        P = normal(w.wid, idx, 1, r, c, w.param_std, w.param_dtype)
        G = normal(w.wid, idx, 0, r, c, w.grad_std, w.grad_dtype)
        M = np.zeros((r, c), np.float32)
        with threadpool_limits(limits=1):
            t0 = time.perf_counter()
            ref.muon_step_matrix(P, G, M, update_scale(r, c), cfg)
            dt1 = time.perf_counter() - t0
        f1 = sum(ns_flops(min(r, c), max(r, c), ns_steps).values())
        one_thread = {"value": round(f1 / dt1 / 1e12, 6), "unit": "TFLOP/s", "cores": 1,
                      "sample": f"{name.split('.')[-1]} {r}x{c}", "seconds": round(dt1, 3)}
        log(f"cpu oracle {r}x{c} on one thread: {dt1:.2f} s")
    except Exception:  # pragma: no cover
        pass
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    # the whole share's oracle step, from the sampled per-shape times and
    # each shape's count (only when every shape was sampled)
    full = None
    if all((r, c) in per_shape for _, r, c in shapes):
        full = sum(per_shape[(r, c)] for _, r, c in shapes)
    return {"value": round(flops / t_total / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle", "cpu_model": cpu_model, "host_cpus": os.cpu_count(),
            "one_thread": one_thread,
            "matrices_per_s": round(len(done) / t_total, 4),
            "seconds": round(t_total, 3),
            "dense_fp64_gflops": round(dense / t_total / 1e9, 2),
            "full_step_seconds_extrapolated": round(full, 2) if full is not None else None,
            "full_step_note": f"extrapolated: sampled time of each distinct shape x its count "
                              f"in the {len(shapes)}-matrix share",
            "sample": f"fp64 NumPy oracle, one step of {len(done)} matrices "
                      f"({', '.join(done)}), the direct iteration's algorithmic NS flops "
                      f"(upper-triangle count) / wall time; dense_fp64_gflops counts the "
                      f"oracle's dense products"}


def main(argv=None) -> int:
    faulthandler.enable()
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="4", help="workload id or name (synth.workloads)")
    ap.add_argument("--shape", action="append", default=None,
                    help="RxC: run a custom bf16 set of these shapes instead (repeatable)")
    ap.add_argument("--repeat", type=int, default=1, help="copies of each --shape")
    ap.add_argument("--ns-steps", type=int, default=None)
    ap.add_argument("--fp32-ns", action="store_true", help="fp32 checking mode")
    ap.add_argument("--chain-launch", action="store_true",
                    help="every bf16 product of the step in one dependency-driven launch")
    ap.add_argument("--direct-ns", action="store_true",
                    help="direct chain for every matrix (default: Gram-space chain where n >= 2m, ns_steps >= 5)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle time")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(json.dumps({"error": "bench.py measures one owner's step on one GPU (each owner "
                                   "runs its share independently); --gpus above 1 is not supported"}))
        return 2

    import torch

    import newton_schulz_dmuon_amd as nsd
    from synth import update_scale, workload

    key = int(args.workload) if args.workload.isdigit() else args.workload
    w = workload(key)
    if args.shape:
        from synth import Workload
        shp = []
        for s in args.shape:
            r, c = (int(x) for x in s.lower().split("x"))
            shp += [(f"custom.{r}x{c}.{i}", r, c) for i in range(args.repeat)]
        w = Workload(0, "custom:" + ",".join(args.shape) + f"x{args.repeat}", shp,
                     "bf16", "bf16", 0.02, 1e-3)
    K = args.ns_steps if args.ns_steps is not None else w.ns_steps
    nsd.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    shapes = owner_share(w, nsd)
    numels = [r * c for _, r, c in shapes]
    offsets, total = nsd.pack_offsets(numels, 128)
    pdt = torch.bfloat16 if w.param_dtype == "bf16" else torch.float32
    gdt = torch.bfloat16 if w.grad_dtype == "bf16" else torch.float32
    log(f"workload {w.name}: {len(shapes)} matrices, {sum(numels):,} elements, ns_steps {K}")

    gen = torch.Generator(device=dev)
    gen.manual_seed(1234 + w.wid)
    grad_packed = torch.empty(total, dtype=gdt, device=dev)
    param_packed = torch.empty(total, dtype=pdt, device=dev)
    P, G, M = [], [], []
    for (name, r, c), off in zip(shapes, offsets):
        g = grad_packed[off:off + r * c].view(r, c)
        g.copy_(torch.randn(r, c, generator=gen, device=dev) * w.grad_std)
        G.append(g)
        P.append((torch.randn(r, c, generator=gen, device=dev) * w.param_std).to(pdt))
        M.append(torch.zeros(r, c, dtype=torch.float32, device=dev))
    scales = [update_scale(r, c) for _, r, c in shapes]
    opts = nsd.StepOptions(ns_steps=K, ns_fp32=args.fp32_ns, gram_ns=not args.direct_ns,
                           chain_launch=args.chain_launch)
    ws = nsd.Workspace()
    ws_bytes = nsd.workspace_bytes(P, opts)
    wsbuf = ws.get(ws_bytes, dev)
    log(f"workspace {ws_bytes / 2**30:.2f} GiB")

    lib = nsd.load()
    arr, n = nsd.api.matrices(P, G, M, scales, packed_offsets=offsets)
    cfg = opts.to_c()
    stream = torch.cuda.current_stream(dev)
    # the step's launches in order, with the algorithmic flops of each
    launches = nsd.step_launches([(r, c) for _, r, c in shapes], opts)
    n_launch = len(launches)
    log("launches: " + " ".join(k for k, _ in launches))

    pk_dtype = nsd._lib.BF16 if pdt == torch.bfloat16 else nsd._lib.F32

    def step(ev=None):
        # the step writes the updated params into the packed buffer too (the
        # last Apply stores both), which is the owner's dmuon_pack of them
        rc = lib.dmuon_muon_step_packed(arr, n, ctypes.byref(cfg), wsbuf.data_ptr(), wsbuf.numel(),
                                        param_packed.data_ptr(), pk_dtype, param_packed.numel(),
                                        stream.cuda_stream, ev.handles if ev else None,
                                        len(ev.handles) if ev else 0)
        nsd._lib.check(rc)

    for i in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} done")

    evs = [TraceEvents(n_launch + 1, stream) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms = dt * 1e3 / args.steps
    log(f"timed {args.steps} steps: {ms:.3f} ms/step")
    # Outside the timed region: one plain copy of known size (the updated
    # params into the packed buffer, 2 x elements x param bytes), which a
    # counter profile of this run uses to scale FETCH_SIZE / WRITE_SIZE.
    nsd.pack(P, offsets, param_packed, stream=stream)
    torch.cuda.synchronize()

    # per-launch durations from the traced events, grouped by launch kind
    names = [k for k, _ in launches]
    per = {nm: [] for nm in set(names)}
    for ev in evs:
        for j, nm in enumerate(names):
            per[nm].append(ev.elapsed_ms(j))
    avg = {nm: sum(v) / len(v) for nm, v in per.items()}
    kind_flops = {nm: sum(f for k, f in launches if k == nm) for nm in set(names)}

    # the metric's count: the direct chain's algorithmic flops, whichever
    # chain runs, so that the rate compares across chains
    flops = {"gram": 0, "square": 0, "apply": 0}
    for _, r, c in shapes:
        for kk, v in ns_flops(min(r, c), max(r, c), K).items():
            flops[kk] += v
    ns_total = sum(flops.values())
    executed = sum(f for _, f in launches)
    gemm_kinds = ("gram", "square", "gram_square", "apply", "final", "chain")
    ns_ms = sum(sum(v) for nm, v in per.items() if nm in gemm_kinds) / args.steps
    peak = PEAK_FP32_TFLOPS if args.fp32_ns else PEAK_BF16_TFLOPS
    value = ns_total / (ms * 1e-3) / 1e12

    stages = {}
    for nm in gemm_kinds:
        if nm in per:
            t = sum(per[nm]) / args.steps   # ms per step in this kind
            stages[nm] = {"ms": avg[nm], "ms_per_step": t, "launches_per_step": names.count(nm),
                          "tflops": kind_flops[nm] / (t * 1e-3) / 1e12}
    elem = sum(numels)
    gsz = 2 if w.grad_dtype == "bf16" else 4
    gbytes = {"momentum_sumsq": elem * (4 + 4 + gsz),
              # G read, M read + write, U written once (as X^T)
              "momentum_orient": elem * (gsz + 4 + 4 + (4 if args.fp32_ns else 2))}
    for nm, b in gbytes.items():
        if nm in avg:
            stages[nm] = {"ms": avg[nm], "gbs": b / (avg[nm] * 1e-3) / 1e9}
    stages["norm"] = {"ms": avg["norm"]}
    # median launch duration of each stage over all its launches in the timed steps
    for nm, v in stages.items():
        src = per.get(nm)
        if src:
            srt = sorted(src)
            v["median_ms"] = srt[len(srt) // 2] if len(srt) % 2 else 0.5 * (srt[len(srt) // 2 - 1] + srt[len(srt) // 2])
            v["launches"] = len(srt)
    for v in stages.values():
        for kk in list(v):
            v[kk] = round(v[kk], 4)

    roofline = None
    if K > 0:
        # the dominant kernel: the GEMM stage with the most time per step;
        # achieved = its algorithmic flops over its launches' summed durations
        dom = max((nm for nm in gemm_kinds if nm in per), key=lambda nm: sum(per[nm]))
        ach = kind_flops[dom] / (sum(per[dom]) / args.steps * 1e-3) / 1e12
        kernel = {"gram": "ns_gemm_kernel<Gram> (A = X X^T)",
                  "square": "ns_gemm_kernel<Square> (symmetric m x m products)",
                  "gram_square": "ns_gemm_kernel<GramSquare> (Gram and Square tiles of different matrices)",
                  "apply": "ns_gemm_kernel<Apply> (X <- aX + BX / X <- QX)",
                  "final": "ns_gemm_kernel<Final> (last apply + update)",
                  "chain": "ns_gemm_chain_kernel (every bf16 stage, one launch)"}[dom]
        roofline = {"bound": "mfma", "kernel": kernel,
                    "achieved": round(ach, 2), "peak": peak, "unit": "TFLOP/s",
                    "frac": round(ach / peak, 4),
                    "traffic": measured_traffic(w.name, args.fp32_ns, dom, opts.gram_ns),
                    "algorithmic_flops_per_launch": kind_flops[dom] / names.count(dom),
                    "launches_per_step": names.count(dom)}

    out = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32" if args.fp32_ns else "bf16", "data": "synthetic",
        "config": {"workload": w.name, "matrices": len(shapes), "elements": elem,
                   "ns_steps": K, "gram_ns": opts.gram_ns, "chain_launch": opts.chain_launch,
                   "param_dtype": w.param_dtype, "grad_dtype": w.grad_dtype,
                   "parallelism": "one owner's share on 1 GPU"},
        # MFMA use: the executed flops over the step, as a share of the
        # peak; value (effective, direct-chain count) over the peak beside it
        "value_is": "effective NS TFLOP/s: the direct iteration's algorithmic flops per step "
                    "/ step time, whichever chain runs",
        "pct_bf16_peak": round(100 * executed / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
        "effective_pct_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "matrices_per_s": round(len(shapes) / (ms * 1e-3), 2),
        "steps_per_s": round(1e3 / ms, 3),
        "ns_chain": "gram-space where max(r,c) >= 2 min(r,c), direct otherwise" if opts.gram_ns
                    else "direct",
        "flop_count": "direct-chain algorithmic count m(m+1)n + m^2(m+1) + 2m^2 n per matrix "
                      "per iteration, whichever chain runs",
        "executed_tflop_per_step": round(executed / 1e12, 3),
        "executed_tflops": round(executed / (ms * 1e-3) / 1e12, 3),
        "ns_kernels_ms": round(ns_ms, 4),
        "ns_kernels_executed_tflops": round(executed / (ns_ms * 1e-3) / 1e12, 3) if ns_ms else None,
        "stages": stages,
        "roofline": roofline,
        "cpu_baseline": None,
    }
    if w.wid == 4 and not args.shape:
        out["adamw"] = adamw_measure(nsd, torch, dev, stream, args.steps)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, shapes, K, args.cpu_budget)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
