"""fp64 reference for the AdamW step on the parameters Muon does not own.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

DMuon landing page, "LLM Pretraining": the optimizer takes an ``adamw_lr``
(1e-3 in the example) next to Muon's ``lr``; "VLA and VLM": parameters the
predicate does not select (embeddings, norms, task heads) stay under the usual
sharded setup.  Those parameters get AdamW.  The pages give no betas, epsilon
or weight decay; the reading taken is decoupled weight decay AdamW (Loshchilov
and Hutter) with bias correction, all hyper-parameters passed in:

  P <- P - lr * wd * P
  M <- beta1 * M + (1 - beta1) * G
  V <- beta2 * V + (1 - beta2) * G^2
  P <- P - lr * (M / (1 - beta1^t)) / (sqrt(V / (1 - beta2^t)) + eps)

with t the 1-based step count.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class AdamWConfig:
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.01
    step: int = 1


def adamw_step(P, G, M, V, cfg: AdamWConfig):
    """One AdamW step on one tensor; returns ``(P, M, V)`` in float64."""
    P = np.asarray(P, np.float64)
    G = np.asarray(G, np.float64)
    M = np.asarray(M, np.float64)
    V = np.asarray(V, np.float64)
    t = cfg.step
    P = P - cfg.lr * cfg.weight_decay * P
    M = cfg.beta1 * M + (1.0 - cfg.beta1) * G
    V = cfg.beta2 * V + (1.0 - cfg.beta2) * G * G
    m_hat = M / (1.0 - cfg.beta1 ** t)
    v_hat = V / (1.0 - cfg.beta2 ** t)
    P = P - cfg.lr * m_hat / (np.sqrt(v_hat) + cfg.eps)
    return P, M, V
