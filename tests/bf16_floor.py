"""bf16 emulation of the Newton-Schulz iteration (test tooling, not the oracle).

Rounds every operand that the bf16 path stores (X0, A, B and each new X) to
bf16 with round-to-nearest-even, and accumulates products in float64. The
relative Frobenius distance between this and the fp64 oracle is the error
floor that bf16 storage alone imposes on the iteration for a given input; a
bf16 GPU result cannot be expected to beat it. For most shapes the floor is
well under the 2e-2 parity bound; for tiny matrices (a handful of singular
values, so no averaging) it can exceed it.
"""
from __future__ import annotations

import numpy as np

A_, B_, C_ = 3.4445, -4.7750, 2.0315
EPS = 1e-7


def round_bf16(x) -> np.ndarray:
    """float -> nearest bf16 (ties to even), returned as float64. NaN stays NaN."""
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000).astype(np.uint32)
    out = r.view(np.float32).astype(np.float64)
    return np.where(np.isnan(f), np.nan, out)


def ns_bf16(m, k: int) -> np.ndarray:
    x = np.asarray(m, dtype=np.float64)
    t = x.shape[0] > x.shape[1]
    if t:
        x = x.T
    x = round_bf16(x / (np.linalg.norm(x) + EPS))
    for _ in range(int(k)):
        a = round_bf16(x @ x.T)
        b = round_bf16(B_ * a + C_ * (a @ a))
        x = round_bf16(A_ * x + b @ x)
    return x.T if t else x


def floor(m, k: int, reference) -> float:
    """Relative Frobenius error of the bf16-emulated iteration vs `reference`."""
    e = ns_bf16(m, k)
    nr = np.linalg.norm(reference)
    return float(np.linalg.norm(e - reference) / (nr if nr > 0 else 1.0))
