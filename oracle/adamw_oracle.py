"""Plain fp64 CPU oracle of the AdamW step for the parameters outside the
MuonH group.

TEST INFRASTRUCTURE ONLY, like muonh_oracle: only the test suite and the
benchmark's CPU-baseline leg use it; it shares no code with the HIP path.

Source: model card page "Puro", section "Training": the parameters that are
not updated by MuonH use AdamW with weight decay 0.1. The page prints nothing
else. Reading: AdamW as defined with decoupled weight decay (the decay scales
the parameter by 1 - lr*wd, separately from the adaptive step), first and
second moments with bias correction, and eps added to the square root of the
corrected second moment. beta1, beta2 and eps are arguments.

One step t >= 1, per element:
    p <- p * (1 - lr*wd)
    m <- beta1*m + (1 - beta1)*g
    v <- beta2*v + (1 - beta2)*g^2
    p <- p - lr * (m / (1 - beta1^t)) / (sqrt(v / (1 - beta2^t)) + eps)
Everything in float64 with numpy elementwise operations.
"""
from __future__ import annotations

import numpy as np


def adamw_step(p, g, m, v, lr: float, beta1: float, beta2: float, eps: float,
               weight_decay: float, step: int):
    """One AdamW step at step number `step` (1-based). Returns (p, m, v) in float64."""
    if step < 1:
        raise ValueError("step is 1-based")
    p = np.asarray(p, dtype=np.float64) * (1.0 - lr * weight_decay)
    g = np.asarray(g, dtype=np.float64)
    m = beta1 * np.asarray(m, dtype=np.float64) + (1.0 - beta1) * g
    v = beta2 * np.asarray(v, dtype=np.float64) + (1.0 - beta2) * g * g
    m_hat = m / (1.0 - beta1 ** step)
    v_hat = v / (1.0 - beta2 ** step)
    p = p - lr * m_hat / (np.sqrt(v_hat) + eps)
    return p, m, v
