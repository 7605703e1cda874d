"""bf16 storage of the gradient and the momentum: the oracle's side.

TEST INFRASTRUCTURE ONLY (as the rest of this package): imported by the
test suite, the smoke check and the benchmark's CPU-baseline leg, never by
the product path, and sharing no code with it.

Model card page "Puro", section "Training": master weights and optimizer
state are kept in FP32 or BF16. The page does not say which tensors take
bf16 or how values are rounded. Readings taken here:

* A bf16 gradient is an input: its values are exactly the bf16 numbers
  given (bf16 is the upper half of an IEEE binary32), nothing is rounded.
* A bf16 momentum is storage: the new momentum is beta*M + G evaluated in
  binary32 with a single rounding (what a fused multiply-add gives, with
  beta the binary32 value the kernel receives), then rounded to the nearest
  bf16, ties to even, and stored. The stored (rounded) value is the momentum
  that Newton-Schulz normalises and orthogonalises. Both roundings decide
  bits, so this side takes them in the kernel's precision, exactly.

Everything here is numpy: conversions to float32 (IEEE round to nearest
even) and float64 arithmetic are the library primitives; the rest is
written out from the definitions.
"""
from __future__ import annotations

import numpy as np


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Values of bf16 bit patterns: the 16 bits are the upper half of a binary32."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):   # NaN payloads convert as NaN
        return u.view(np.float32).astype(np.float64)


def f32_to_bf16_bits(x) -> np.ndarray:
    """Round binary32 values to bf16: nearest of the two bf16 numbers that
    bracket x, ties to the one with an even last significand bit; values at
    or past the midpoint above the largest finite bf16 go to infinity. NaN
    maps to a quiet NaN, infinities to themselves. Returns uint16 bits."""
    x = np.asarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    down = (u >> np.uint32(16)).astype(np.uint32)   # drop 16 bits: toward zero
    up = down + np.uint32(1)                         # next bf16 away from zero
    xd = x.astype(np.float64)
    v_down = bf16_bits_to_f64(down.astype(np.uint16))
    # magnitude of the bf16 above; past the largest finite value that is
    # infinity, which sits at 2^128 for the purpose of the distance
    up_inf = (up & np.uint32(0x7FFF)) == np.uint32(0x7F80)
    v_up = np.where(up_inf, np.copysign(2.0 ** 128, xd),
                    bf16_bits_to_f64((up & np.uint32(0xFFFF)).astype(np.uint16)))
    finite = np.isfinite(xd)
    with np.errstate(invalid="ignore"):
        d_down = np.abs(xd - v_down)
        d_up = np.abs(v_up - xd)
    odd = (down & np.uint32(1)) == np.uint32(1)
    pick_up = finite & ((d_up < d_down) | ((d_up == d_down) & odd))
    out = np.where(pick_up, up, down)
    out = np.where(np.isnan(xd), down | np.uint32(0x0040), out)   # quiet NaN
    return out.astype(np.uint16)


def round_to_bf16(x) -> np.ndarray:
    """Binary32 values rounded to bf16 (nearest, ties to even), as float64."""
    return bf16_bits_to_f64(f32_to_bf16_bits(x))


def fma_f32(a, b, c) -> np.ndarray:
    """a*b + c for binary32 a, b, c, computed exactly and rounded once to
    binary32 (nearest, ties to even).

    The product of two 24-bit significands fits a float64 exactly. The sum s
    is rounded to float64, and its rounding error e is recovered exactly
    (Knuth's two-sum), so s + e is the exact result. Rounding s to binary32
    gives the right answer unless s falls exactly on the midpoint between
    two binary32 neighbours while e is not zero: then the exact value lies on
    the side of the midpoint that e points to.
    """
    a = np.asarray(a, dtype=np.float32).astype(np.float64)
    b = np.asarray(b, dtype=np.float32).astype(np.float64)
    c = np.asarray(c, dtype=np.float32).astype(np.float64)
    p = a * b                      # exact
    s = p + c
    bv = s - p
    e = (p - (s - bv)) + (c - bv)  # s + e == p + c exactly
    r = s.astype(np.float32)
    rd = r.astype(np.float64)
    # binary32 neighbours below and above s (when s is not itself binary32)
    lo = np.where(rd <= s, r, np.nextafter(r, np.float32(-np.inf)))
    hi = np.nextafter(lo, np.float32(np.inf))
    with np.errstate(invalid="ignore", over="ignore"):
        mid = (lo.astype(np.float64) + hi.astype(np.float64)) / 2.0
    on_mid = (s == mid) & (rd != s) & np.isfinite(s)
    out = np.where(on_mid & (e > 0), hi, np.where(on_mid & (e < 0), lo, r))
    return out.astype(np.float32)


def momentum_update_bf16_state(m, g, beta: float) -> np.ndarray:
    """New momentum kept in bf16: round_to_bf16(fl32(beta32*M + G)).

    m: the stored momentum (bf16 values, given as any float array); g: the
    gradient (binary32 or bf16 values). Returns float64 values that are all
    exactly bf16.
    """
    m32 = np.asarray(m, dtype=np.float64).astype(np.float32)
    if not np.array_equal(round_to_bf16(m32), np.asarray(m, dtype=np.float64), equal_nan=True):
        raise ValueError("a bf16 momentum must hold bf16 values")
    g32 = np.asarray(g, dtype=np.float64).astype(np.float32)
    beta32 = np.float32(beta)
    return round_to_bf16(fma_f32(np.full_like(m32, beta32), m32, g32))
