"""Plain fp64 CPU oracle of the MuonH optimizer step.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module. The product path (the HIP
library and its Python binding) never calls it, and it imports nothing from the
product path: the two share no code.

What it computes, and where each step comes from
------------------------------------------------
Sources are the web pages this project is built from, cited by page title and
section:

* Page "Puro-2B trains for $6.9K, attention sinks hit 99%, LoopArena tops at
  24.69%" (a research digest), section "The load-bearing tricks aren't in the
  abstract", and its footnote 3: MuonH extends Muon; it keeps the Frobenius
  norm of every weight matrix equal to the norm the matrix had at
  initialization, by putting each update back on that fixed sphere. Footnote 4
  of the same page: Muon's cost is its Newton-Schulz iterations.
* Page "Puro" (model card), section "Training": the matrix group is updated by
  MuonH with hyperball projection and no weight decay; master weights and
  optimizer state are kept in FP32 (or BF16).
* Page "Puro" (model card), section "Why Puro-2B?", and the arXiv abstract page
  "Puro-2B: Poor Lab's Qwen2-1.5B Trained on RTX 5090 within $5090": the
  method is called hyperball optimization.

The pages print neither the momentum rule, nor the Newton-Schulz polynomial,
its coefficients or its input normalisation, nor the projection formula. The
readings taken here (each one is listed with its reason in the design notes):

1. Momentum is heavy-ball without dampening: M <- beta*M + G.
2. Newton-Schulz input: X0 = M / (||M||_F + eps), eps = 1e-7, run on the
   transpose when rows > cols (square matrices are not transposed).
3. Each iteration applies the odd quintic p(s) = a*s + b*s^3 + c*s^5 to every
   singular value: A = X X^T, B = b*A + c*A*A, X <- a*X + B X, with
   (a, b, c) = (3.4445, -4.7750, 2.0315), the usual Muon coefficients.
4. Update without extra scale or weight decay: W' = W - lr*O.
5. Projection onto the sphere of radius R = ||W0||_F: W <- (R/||W'||_F) W',
   and W <- W' when ||W'||_F = 0 (only possible when R = 0).

Everything is computed in float64 with numpy; matrix products use numpy's
matmul as a library primitive. There is no blocking, fusion or reordering.
"""
from __future__ import annotations

import math
from typing import Tuple

import numpy as np

from .bf16_state_oracle import momentum_update_bf16_state

NS_COEFFS: Tuple[float, float, float] = (3.4445, -4.7750, 2.0315)
NS_EPS: float = 1e-7


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def frobenius_norm(x) -> float:
    """sqrt of the sum of squares of all entries, in float64."""
    x = _f64(x)
    return math.sqrt(float(np.sum(x * x)))


def init_radius(w0) -> float:
    """R = ||W0||_F, the radius the matrix keeps for the whole run.

    Digest page, section "The load-bearing tricks aren't in the abstract":
    the norm is fixed at its value at initialization.
    """
    return frobenius_norm(w0)


def momentum_update(m, g, beta: float, mom_bf16: bool = False) -> np.ndarray:
    """M <- beta*M + G (reading 1: heavy-ball, no dampening, no Nesterov).

    Muon's first stage; the digest page (same section) calls MuonH an
    extension of Muon. With mom_bf16 the momentum is stored in bf16 (model
    card, section "Training": state in FP32 or BF16): the new value is
    rounded as bf16_state_oracle.momentum_update_bf16_state states.
    """
    if mom_bf16:
        return momentum_update_bf16_state(m, g, beta)
    return float(beta) * _f64(m) + _f64(g)


def newton_schulz(m, ns_iters: int, coeffs=NS_COEFFS, eps: float = NS_EPS) -> np.ndarray:
    """Orthogonalized update O of a momentum matrix M (readings 2 and 3).

    The digest page (footnote 4) names these iterations as the cost of Muon.
    Steps, in order:
      transpose when rows > cols; X = X / (||X||_F + eps);
      repeat ns_iters times: A = X X^T; B = b A + c A A; X = a X + B X;
      transpose back.
    """
    a, b, c = (float(v) for v in coeffs)
    x = _f64(m)
    transposed = x.shape[0] > x.shape[1]
    if transposed:
        x = x.T
    x = x / (frobenius_norm(x) + eps)
    for _ in range(int(ns_iters)):
        gram = x @ x.T
        poly = b * gram + c * (gram @ gram)
        x = a * x + poly @ x
    return x.T if transposed else x


def hyperball_project(w, o, radius: float, lr: float) -> np.ndarray:
    """W <- R * (W - lr*O) / ||W - lr*O||_F (readings 4 and 5).

    Digest page, section "The load-bearing tricks aren't in the abstract":
    the update is projected back onto the fixed sphere of the matrix's
    initial norm. Model card, section "Training": no weight decay term.
    """
    w_trial = _f64(w) - float(lr) * _f64(o)
    n = frobenius_norm(w_trial)
    if n > 0.0:
        return (float(radius) / n) * w_trial
    return w_trial


def muonh_step(w, g, m, radius: float, lr: float, beta: float, ns_iters: int,
               coeffs=NS_COEFFS, eps: float = NS_EPS, mom_bf16: bool = False):
    """One MuonH step for one matrix. Returns (W_new, M_new, O) in float64.
    With mom_bf16, M holds bf16 values and so does M_new (see
    momentum_update); a bf16 gradient needs nothing special: its values are
    the bf16 numbers given."""
    m_new = momentum_update(m, g, beta, mom_bf16)
    o = newton_schulz(m_new, ns_iters, coeffs=coeffs, eps=eps)
    w_new = hyperball_project(w, o, radius, lr)
    return w_new, m_new, o


def muon_wd_step(w, g, m, lr: float, beta: float, weight_decay: float, ns_iters: int,
                 coeffs=NS_COEFFS, eps: float = NS_EPS, mom_bf16: bool = False):
    """Muon with decoupled weight decay: the baseline MuonH is measured against.

    The digest page ("The load-bearing tricks aren't in the abstract" and its
    footnote 3) quotes MuonH's speedup against standard weight decay, and the
    report page (part 6/7, section 4.3 "Cost Estimation") its compute
    multiplier relative to Muon. Neither prints the baseline's update. Reading:
    the same momentum and Newton-Schulz orthogonalisation as MuonH, then weight
    decay decoupled from the update, W <- (1 - lr*wd) W - lr O, and no
    projection. Returns (W_new, M_new, O) in float64. mom_bf16 as in
    muonh_step.
    """
    m_new = momentum_update(m, g, beta, mom_bf16)
    o = newton_schulz(m_new, ns_iters, coeffs, eps)
    w_new = (1.0 - lr * weight_decay) * _f64(w) - lr * o
    return w_new, m_new, o
