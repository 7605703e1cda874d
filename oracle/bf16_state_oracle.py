"""bf16 storage of the gradient and the momentum: the oracle's side.

TEST INFRASTRUCTURE ONLY (as the rest of this package): imported by the
test suite, the smoke check and the benchmark's CPU-baseline leg, never by
the product path, and sharing no code with it.

Model card page "Puro", section "Training": master weights and optimizer
state are kept in FP32 or BF16. The page does not say which tensors take
bf16 or how values are rounded. Readings taken here:

* A bf16 gradient is an input: its values are exactly the bf16 numbers
  given (bf16 is the upper half of an IEEE binary32), nothing is rounded.
* A bf16 momentum is storage: the new momentum is the exact real number
  beta*M + G (beta taken as the binary32 value a caller passes), rounded
  once to the nearest bf16, ties to even, and stored. The stored (rounded)
  value is the momentum that Newton-Schulz normalises and orthogonalises.
  This is the plain definition of storing a result in bf16: no intermediate
  binary32 rounding is assumed, since the page prints none.

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


def round_real_to_bf16(hi, lo) -> np.ndarray:
    """The bf16 number nearest to the real number hi + lo, ties to the one
    with an even last significand bit, as float64.

    hi is float64 and lo is what float64 could not hold of the real number
    (hi = fl64(hi + lo), so |lo| is at most half a float64 ulp of hi). bf16
    keeps 8 significant bits; below 2^-126 its spacing stays 2^-133
    (subnormals). Magnitudes at or past the midpoint above the largest finite
    bf16 go to infinity; infinities and NaN stay what they are.

    Written out from the definition: the spacing of the bf16 numbers around
    |hi| is a power of two, so |hi| / spacing is exact and its fractional
    part says on which side of the midpoint |hi| lies; exactly on it, lo
    decides, and with lo = 0 it is a tie.
    """
    hi = np.asarray(hi, dtype=np.float64)
    lo = np.asarray(lo, dtype=np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        a = np.abs(hi)
        sgn = np.where(np.signbit(hi), -1.0, 1.0)
        lo_out = lo * sgn                   # > 0: the real magnitude is above a
        _, ex = np.frexp(np.where(np.isfinite(a), a, 0.0))   # a = f * 2^ex, f in [0.5, 1)
        e = np.maximum(ex - 1, -126)        # exponent of the leading bit
        spacing = np.ldexp(1.0, e - 7)
        q = np.where(np.isfinite(a), a, 0.0) / spacing        # exact
        n = np.floor(q)
        frac = q - n
        odd = np.fmod(n, 2.0) == 1.0
        up = (frac > 0.5) | ((frac == 0.5) & ((lo_out > 0) | ((lo_out == 0) & odd)))
        mag = (n + up) * spacing
        mag = np.where(mag >= 2.0 ** 128, np.inf, mag)
        out = sgn * mag
    return np.where(np.isfinite(hi), out, hi)


def momentum_update_bf16_state(m, g, beta: float) -> np.ndarray:
    """New momentum kept in bf16: the bf16 number nearest to the exact real
    beta32*M + G (one rounding, ties to even).

    m: the stored momentum (bf16 values, given as any float array); g: the
    gradient (binary32 or bf16 values); beta32: beta as a binary32 number.
    beta32*M has at most 24 + 8 significant bits, so float64 holds it
    exactly; the float64 sum s of it and G is rounded, and its rounding
    error e is recovered exactly (Knuth's two-sum: s + e = beta32*M + G), so
    round_real_to_bf16(s, e) rounds the exact value once. Returns float64
    values that are all exactly bf16.
    """
    m32 = np.asarray(m, dtype=np.float64).astype(np.float32)
    if not np.array_equal(round_to_bf16(m32), np.asarray(m, dtype=np.float64), equal_nan=True):
        raise ValueError("a bf16 momentum must hold bf16 values")
    g64 = np.asarray(g, dtype=np.float64).astype(np.float32).astype(np.float64)
    beta64 = float(np.float32(beta))
    p = beta64 * m32.astype(np.float64)     # exact
    with np.errstate(invalid="ignore"):
        s = p + g64
        bv = s - p
        e = (p - (s - bv)) + (g64 - bv)     # s + e == p + g exactly
    return round_real_to_bf16(s, np.where(np.isfinite(s), e, 0.0))
