"""Seeded synthetic inputs and workload shape tables.

This is the only module that both the oracle side (tests, the CPU baseline)
and the HIP side (binding tests, bench) read.  It holds no arithmetic of the
method: it draws Gaussian values, rounds them to the storage dtype with the
library conversion, and lists matrix shapes.

The DMuon landing page ("Benchmarks") runs on random initialisation and
synthetic data; so does everything here.  Shapes are the attention and MLP
projection matrices (the ones the landing page's predicate ``"proj" in name``
selects) of the model families named on that page, in PyTorch ``[out, in]``
order, in model order within a layer: q, k, v, o, gate, up, down.

Recipe
------
* a matrix is identified by ``(workload_id, matrix_index, kind)`` with kind
  0 = gradient, 1 = parameter, 2 = momentum;
* values are ``std * standard_normal`` drawn in float32 from NumPy's
  Philox counter-based generator seeded with that triple;
* bf16 inputs are rounded to bf16 (round-to-nearest-even, torch's
  conversion) and returned as float32 arrays holding exactly those values.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

# ----------------------------------------------------------------- shapes ---

PROJ_ORDER = ("q", "k", "v", "o", "gate", "up", "down")


def layer_shapes(d_model: int, kv_dim: int, d_ff: int):
    """Projection shapes of one transformer layer, ``[out, in]``."""
    return [("q", d_model, d_model), ("k", kv_dim, d_model), ("v", kv_dim, d_model),
            ("o", d_model, d_model), ("gate", d_ff, d_model), ("up", d_ff, d_model),
            ("down", d_model, d_ff)]


def model_shapes(d_model: int, kv_dim: int, d_ff: int, n_layers: int):
    out = []
    for layer in range(n_layers):
        for name, r, c in layer_shapes(d_model, kv_dim, d_ff):
            out.append((f"layers.{layer}.{name}_proj", r, c))
    return out


QWEN25_1P5B = dict(d_model=1536, kv_dim=256, d_ff=8960, n_layers=28)
LLAMA32_3B = dict(d_model=3072, kv_dim=1024, d_ff=8192, n_layers=28)
LLAMA31_8B = dict(d_model=4096, kv_dim=1024, d_ff=14336, n_layers=32)
QWEN25_7B = dict(d_model=3584, kv_dim=512, d_ff=18944, n_layers=28)


def non_muon_sizes(d_model: int, n_layers: int, vocab: int, tied: bool = False):
    """Element counts of a decoder's parameters the Muon predicate leaves out:
    token embedding, output head (unless tied), and the RMSNorm weights (two
    per layer plus the final one)."""
    sizes = [("embed_tokens", vocab * d_model)]
    if not tied:
        sizes.append(("lm_head", vocab * d_model))
    sizes.append(("norms", (2 * n_layers + 1) * d_model))
    return sizes


LLAMA31_8B_VOCAB = 128256   # public Llama-3.1-8B configuration


@dataclass
class Workload:
    """A named set of matrices with its value distributions."""

    wid: int
    name: str
    shapes: list                    # [(name, rows, cols)]
    param_dtype: str                # "bf16" | "f32"
    grad_dtype: str
    param_std: float
    grad_std: float
    ns_steps: int = 5
    n_owners: int = 1               # >1: shapes are the whole model, one owner's share is taken
    owner: int = 0
    notes: str = ""
    extra: dict = field(default_factory=dict)


def workloads():
    """The five workloads, smallest first."""
    return [
        Workload(1, "single-128x256-f32", [("w", 128, 256)], "f32", "f32", 0.02, 1.0,
                 notes="one fp32 128x256 matrix, grad N(0,1), param N(0,0.02)"),
        Workload(2, "qwen2.5-1.5b-1layer",
                 [(f"layers.0.{n}_proj", r, c) for n, r, c in layer_shapes(1536, 256, 8960)],
                 "bf16", "bf16", 0.02, 1e-3),
        Workload(3, "llama3.2-3b-28layers", model_shapes(**LLAMA32_3B), "bf16", "bf16", 0.02, 1e-3),
        Workload(4, "llama3.1-8b-owner0-of-8", model_shapes(**LLAMA31_8B), "bf16", "bf16", 0.02, 1e-3,
                 n_owners=8, owner=0,
                 notes="whole 32-layer projection set; the step runs on owner 0's share"),
        Workload(5, "qwen2.5-7b-28layers", model_shapes(**QWEN25_7B), "bf16", "bf16", 0.02, 1e-3,
                 extra={"ns_steps_sweep": (3, 5, 8)}),
    ]


def workload(key):
    for w in workloads():
        if w.wid == key or w.name == key:
            return w
    raise KeyError(key)


def update_scale(rows: int, cols: int) -> float:
    """Per-shape update scale handed to the step: ``sqrt(max(1, rows/cols))``
    (the public Muon convention; the DMuon pages give no rule)."""
    return math.sqrt(max(1.0, rows / cols))


# ----------------------------------------------------------------- values ---

KIND_GRAD, KIND_PARAM, KIND_MOMENTUM = 0, 1, 2


def _rng(wid: int, index: int, kind: int) -> np.random.Generator:
    return np.random.Generator(np.random.Philox(np.random.SeedSequence([wid, index, kind])))


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to the storage dtype; float32 array out."""
    if dtype == "f32":
        return x.astype(np.float32, copy=False)
    if dtype == "bf16":
        import torch
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(
            torch.bfloat16).to(torch.float32).numpy()
    raise ValueError(dtype)


def normal(wid: int, index: int, kind: int, rows: int, cols: int, std: float,
           dtype: str) -> np.ndarray:
    """Seeded ``std * N(0,1)`` matrix, rounded to ``dtype``, as float32."""
    x = _rng(wid, index, kind).standard_normal((rows, cols), dtype=np.float32)
    x *= np.float32(std)
    return round_to(x, dtype)


def matrix_inputs(w: Workload, index: int, momentum_std: float = 0.0):
    """(param, grad, momentum) float32 arrays for matrix ``index`` of ``w``.
    The momentum buffer is zero unless ``momentum_std`` is given."""
    _, r, c = w.shapes[index]
    P = normal(w.wid, index, KIND_PARAM, r, c, w.param_std, w.param_dtype)
    G = normal(w.wid, index, KIND_GRAD, r, c, w.grad_std, w.grad_dtype)
    if momentum_std:
        M = normal(w.wid, index, KIND_MOMENTUM, r, c, momentum_std, "f32")
    else:
        M = np.zeros((r, c), np.float32)
    return P, G, M


def random_case(seed: int, rows: int, cols: int, std: float = 1.0, dtype: str = "f32",
                kind: int = 0) -> np.ndarray:
    """Free-standing seeded matrix for tests (workload id 0)."""
    return normal(0, seed, kind, rows, cols, std, dtype)
