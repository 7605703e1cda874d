"""bf16 emulation of the Newton-Schulz iteration (test tooling, not the oracle).

Rounds every operand that the bf16 path stores (X0, A, B and each new X) to
bf16 with round-to-nearest-even, and accumulates products in float64. The
relative Frobenius distance between this and the fp64 oracle is the error
floor that bf16 storage alone imposes on the iteration for a given input; a
bf16 GPU result cannot be expected to beat it. For most shapes the floor is
well under the 2e-2 parity bound; for tiny matrices (a handful of singular
values, so no averaging) it can exceed it.

fmt="split_bf16" emulates the split storage instead: a stored value v is
hi + lo with hi = bf16(v) and lo = bf16(v - hi) (the difference taken in
fp32), and a product of two split operands omits lo*lo.

By default the emulation follows the definition's order: X0 = M/(||M|| + eps)
is rounded after the normalisation. deferred=True instead stores M itself
rounded and folds 1/(||M|| + eps) into the first Gram (squared) and the
first apply, for norms in [2^-40, 2^40] (or 0), and fold=True stores
B' = a*I + b*A + c*A*A and computes X <- B' X (the library's order for
matrices of more than 65536 entries); with fmt="exact" these check that the
rescheduled algebra equals the definition. The parity bars never use them.
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


def split_bf16(x):
    """float -> (hi, lo) bf16 pair as float64 arrays, lo = bf16(fp32(x) - hi)."""
    f = np.asarray(x, dtype=np.float32)
    hi = round_bf16(f)
    lo = round_bf16((f - hi.astype(np.float32)).astype(np.float32))
    return hi, lo


def _deferred(n: float) -> bool:
    """Norms for which X0's normalisation is folded into the first GEMMs."""
    return n == 0.0 or 2.0 ** -40 <= n <= 2.0 ** 40


def _ns_emulated(m, k: int, fmt: str, deferred: bool = False, fold: bool = False) -> np.ndarray:
    if fmt == "bf16":
        def store(v):
            r = round_bf16(v)
            return r, r, None

        def mul(p, q):
            return p[0] @ q[0]
    elif fmt == "exact":  # no rounding: checks the arithmetic of the scheme itself
        def store(v):
            v = np.asarray(v, dtype=np.float64)
            return v, v, None

        def mul(p, q):
            return p[0] @ q[0]
    elif fmt == "split_bf16":
        def store(v):
            hi, lo = split_bf16(v)
            return hi + lo, hi, lo

        def mul(p, q):
            return p[1] @ q[1] + p[1] @ q[2] + p[2] @ q[1]
    else:
        raise ValueError(fmt)
    x = np.asarray(m, dtype=np.float64)
    t = x.shape[0] > x.shape[1]
    if t:
        x = x.T
    nrm = float(np.linalg.norm(x))
    eye = np.eye(x.shape[0])

    def poly(a):
        # B = b*A + c*A*A, or B' = a*I + B when folded
        return store(B_ * a[0] + C_ * mul(a, a) + (A_ * eye if fold else 0.0))

    def apply(b, y):
        return mul(b, y) if fold else A_ * y[0] + mul(b, y)
    first = 0
    if deferred and int(k) >= 1 and _deferred(nrm):
        # the stored operand is M itself; the first Gram takes sigma^2 and
        # the first apply sigma
        sigma = 1.0 / (nrm + EPS)
        y = store(x)
        yt = tuple(None if v is None else v.T for v in y)
        a = store(sigma * sigma * mul(y, yt))
        x = store(sigma * apply(poly(a), y))
        first = 1
    else:
        x = store(x / (nrm + EPS))
    for _ in range(first, int(k)):
        xt = tuple(None if v is None else v.T for v in x)
        a = store(mul(x, xt))
        x = store(apply(poly(a), x))
    return x[0].T if t else x[0]


def ns_bf16(m, k: int) -> np.ndarray:
    return _ns_emulated(m, k, "bf16")


def ns_split_bf16(m, k: int) -> np.ndarray:
    return _ns_emulated(m, k, "split_bf16")


def floor(m, k: int, reference, fmt: str = "bf16", deferred: bool = False) -> float:
    """Relative Frobenius error of the emulated iteration vs `reference`."""
    e = _ns_emulated(m, k, fmt, deferred)
    nr = np.linalg.norm(reference)
    return float(np.linalg.norm(e - reference) / (nr if nr > 0 else 1.0))
