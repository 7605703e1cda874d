"""Pins of the oracle's bf16 storage of the gradient and the momentum.

The oracle (oracle/bf16_state_oracle.py) keeps a bf16 momentum as the bf16
number nearest to the exact real beta32*M + G (one rounding, ties to even).
Checked here against torch's CPU bf16 conversion (a library routine), hand
values, and a brute force in exact rational arithmetic with its own
rounding, on random and on constructed near-tie inputs; planted mistakes
(among them the two-step reading that rounds to binary32 first) must fail.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")


# ---------------------------------------------------------------------------
# exact reference: rational arithmetic, rounding written out independently
# ---------------------------------------------------------------------------
def rne_fraction(q: Fraction, sig_bits: int, min_exp: int = -126) -> Fraction:
    """q rounded to the nearest binary number with sig_bits significant bits
    (exponents below min_exp keep the spacing of min_exp: subnormals), ties
    to an even last bit. No overflow handling: test values stay small."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, min_exp)
    ulp = Fraction(2) ** (e - (sig_bits - 1))
    n = a / ulp
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * ulp


def exact_momentum(beta32: np.float32, m: float, g: float) -> float:
    q = Fraction(float(beta32)) * Fraction(float(m)) + Fraction(float(g))
    return float(rne_fraction(q, 8))


def bf16_midpoint_above(v: Fraction) -> Fraction:
    """The midpoint between the bf16 number v and its neighbour away from zero."""
    if v == 0:
        return Fraction(2) ** -134
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    half = Fraction(2) ** (max(e, -126) - 8)
    return v + (half if v > 0 else -half)


def fma_f32(a, b, c) -> np.ndarray:
    """a*b + c for binary32 a, b, c rounded once to binary32 (a test helper:
    the planted two-step reading below rounds through it).

    The product of two 24-bit significands fits a float64 exactly; the sum's
    float64 rounding error e is recovered with two-sum, and a float64 sum
    that lands exactly on a binary32 midpoint is moved to the side e points
    to."""
    a = np.asarray(a, dtype=np.float32).astype(np.float64)
    b = np.asarray(b, dtype=np.float32).astype(np.float64)
    c = np.asarray(c, dtype=np.float32).astype(np.float64)
    p = a * b
    s = p + c
    bv = s - p
    e = (p - (s - bv)) + (c - bv)
    r = s.astype(np.float32)
    rd = r.astype(np.float64)
    lo = np.where(rd <= s, r, np.nextafter(r, np.float32(-np.inf)))
    hi = np.nextafter(lo, np.float32(np.inf))
    with np.errstate(invalid="ignore", over="ignore"):
        mid = (lo.astype(np.float64) + hi.astype(np.float64)) / 2.0
    on_mid = (s == mid) & (rd != s) & np.isfinite(s)
    out = np.where(on_mid & (e > 0), hi, np.where(on_mid & (e < 0), lo, r))
    return out.astype(np.float32)


def bf16_values(rng, n, lo_exp=-20, hi_exp=4):
    """Random bf16 numbers: binary32 values whose low 16 bits are zero."""
    x = (rng.standard_normal(n) * 2.0 ** rng.integers(lo_exp, hi_exp, n)).astype(np.float32)
    return (x.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)


def near_tie_cases(rng, beta32, n):
    """(m, g) with beta32*m + g within two binary32 ulps of a bf16 midpoint,
    and cases where it is exactly on one (m = 0)."""
    ms, gs = [], []
    h = bf16_values(rng, n, -6, 3)
    for i in range(n):
        hf = Fraction(float(h[i]))
        e = abs(hf).numerator.bit_length() - abs(hf).denominator.bit_length()
        while Fraction(2) ** e > abs(hf):
            e -= 1
        while Fraction(2) ** (e + 1) <= abs(hf):
            e += 1
        mid = hf + (1 if hf > 0 else -1) * Fraction(2) ** (e - 8)      # half a bf16 ulp
        m = float(bf16_values(rng, 1, e - 30, e - 24)[0]) if i % 4 else 0.0
        p = Fraction(float(beta32)) * Fraction(m)
        k = int(rng.integers(-2, 3))
        g = float(rne_fraction(mid - p + k * Fraction(2) ** (e - 23), 24))
        ms.append(m)
        gs.append(g)
    return np.array(ms, np.float32), np.array(gs, np.float32)


def exact_tie_cases(rng, beta32, n):
    """Two families that only the exact value decides:
    even i: beta32*m + g is exactly a bf16 midpoint, with beta32*m of about
      the midpoint's size (g = midpoint - beta32*m is a binary32 number), so
      the result is the tie's even neighbour, and an error in beta32*m moves it;
    odd i: g is a bf16 midpoint and beta32*m is below half a float64 ulp of
      it, so the float64 sum is the midpoint itself and only its rounding
      error says on which side the exact value lies."""
    ms, gs = [], []
    for i in range(n):
        if i % 2 == 0:
            while True:
                m = float(bf16_values(rng, 1, -6, 3)[0])
                p = Fraction(float(beta32)) * Fraction(m)
                mid = bf16_midpoint_above(Fraction(float(rne_fraction(p, 8))))
                g = mid - p
                if Fraction(float(np.float32(float(g)))) == g:
                    break
            ms.append(m)
            gs.append(float(g))
        else:
            h = float(bf16_values(rng, 1, -6, 3)[0])
            mid = bf16_midpoint_above(Fraction(h))
            e = abs(h).hex().split("p")[1]
            m = float(bf16_values(rng, 1, int(e) - 70, int(e) - 60)[0])
            ms.append(m)
            gs.append(float(mid))
    return np.array(ms, np.float32), np.array(gs, np.float32)


# the binary32 beta and inputs of a double-rounding trap: beta*m = 2^-24 + 2^-54,
# so beta*m + g = 1 + 2^-8 + 2^-24 + 2^-54 lies just above a binary32
# midpoint; rounding the float64 sum (1 + 2^-8 + 2^-24) ties to even instead
TRAP_BETA = np.float32(16519105 * 2.0 ** -24)   # 16519105 * 65 = 2^30 + 1
TRAP_M, TRAP_G = np.float32(65 * 2.0 ** -30), np.float32(1 + 2.0 ** -8)
# a double-rounding case of the two-step reading: beta*m + g = 1 + 2^-8 + 2^-30
# lies above the bf16 midpoint 1 + 2^-8 (so it rounds up to 1 + 2^-7), but
# within half a binary32 ulp of it, so a binary32 rounding first lands on the
# midpoint and the tie then goes to the even 1.0
DR_BETA, DR_M, DR_G = np.float32(0.5), np.float32(2.0 ** -29), np.float32(1 + 2.0 ** -8)


# ---------------------------------------------------------------------------
# the rounding and decoding primitives
# ---------------------------------------------------------------------------
def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(91)
    x = (rng.standard_normal(200000) * 2.0 ** rng.integers(-140, 120, 200000)).astype(np.float32)
    ties = x.view(np.uint32).copy()
    ties[:50000] = (ties[:50000] & np.uint32(0xFFFF0000)) | np.uint32(0x8000)   # exact ties
    x = ties.view(np.float32)
    x = np.concatenate([x, np.float32([0.0, -0.0, np.inf, -np.inf, 3.3895314e38, -3.3895314e38,
                                      1e-45, -1e-45, 1.1754942e-38])])
    ours = oracle.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    nan = oracle.f32_to_bf16_bits(np.float32([np.nan]))
    assert np.isnan(oracle.bf16_bits_to_f64(nan)[0])


def test_bf16_rounding_hand_values():
    r = oracle.round_to_bf16(np.float32([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 1 + 2 ** -8 + 2 ** -20,
                                         2.0 ** -133]))
    assert list(r) == [1.0, 1 + 2 ** -6, -1.0, 1 + 2 ** -7, 2.0 ** -133]
    # the midpoint above the largest finite bf16 rounds to infinity
    top = np.uint32(0x7F7F8000).view(np.float32)
    assert oracle.f32_to_bf16_bits(np.float32([top]))[0] == 0x7F80


def test_bf16_decoding_known_bits():
    v = oracle.bf16_bits_to_f64(np.uint16([0x3F80, 0xC000, 0x7F80, 0x0001, 0x3E80, 0x8000]))
    assert list(v[:2]) == [1.0, -2.0] and np.isposinf(v[2])
    assert v[3] == 2.0 ** -133 and v[4] == 0.25 and v[5] == 0.0 and np.signbit(v[5])


def test_fma_f32_against_exact_rationals():
    rng = np.random.default_rng(92)
    n = 3000
    a = (rng.standard_normal(n) * 2.0 ** rng.integers(-10, 10, n)).astype(np.float32)
    b = (rng.standard_normal(n) * 2.0 ** rng.integers(-30, 5, n)).astype(np.float32)
    c = (rng.standard_normal(n) * 2.0 ** rng.integers(-10, 10, n)).astype(np.float32)
    # exact cancellation and the double-rounding trap
    a = np.concatenate([a, [np.float32(0.75), TRAP_BETA]]).astype(np.float32)
    b = np.concatenate([b, [np.float32(2.0), TRAP_M]]).astype(np.float32)
    c = np.concatenate([c, [np.float32(-1.5), TRAP_G]]).astype(np.float32)
    got = fma_f32(a, b, c)
    for i in range(len(a)):
        q = Fraction(float(a[i])) * Fraction(float(b[i])) + Fraction(float(c[i]))
        assert Fraction(float(got[i])) == rne_fraction(q, 24), i
    assert got[-1] == np.float32(1 + 2 ** -8 + 2 ** -23)


def test_round_real_to_bf16_against_exact_rationals():
    rng = np.random.default_rng(95)
    n = 4000
    hi = rng.standard_normal(n) * 2.0 ** rng.integers(-140, 126, n)
    # exact bf16 midpoints and bf16 numbers, each with a small lo on either side
    mid = np.array([float(bf16_midpoint_above(Fraction(float(v))))
                    for v in oracle.round_to_bf16(hi.astype(np.float32))])
    hi = np.concatenate([hi, mid, mid, mid, oracle.round_to_bf16(hi[:500].astype(np.float32))])
    ulp64 = np.abs(np.spacing(hi))
    lo = np.concatenate([np.zeros(n), 0.25 * ulp64[n:2 * n], -0.25 * ulp64[2 * n:3 * n],
                         np.zeros(n), -0.5 * ulp64[4 * n:]])
    got = oracle.round_real_to_bf16(hi, lo)
    for i in range(len(hi)):
        q = Fraction(float(hi[i])) + Fraction(float(lo[i]))
        assert Fraction(float(got[i])) == rne_fraction(q, 8, -126), i
    # overflow: the midpoint above the largest finite bf16 and beyond
    big = float(np.uint32(0x7F7F0000).view(np.float32))
    top_mid = big + 2.0 ** 119
    out = oracle.round_real_to_bf16([big, top_mid, -top_mid, top_mid], [0.0, 0.0, 0.0, -2.0 ** 60])
    assert out[0] == big and np.isposinf(out[1]) and np.isneginf(out[2]) and out[3] == big
    assert np.isnan(oracle.round_real_to_bf16([np.nan], [0.0])[0])
    assert np.isposinf(oracle.round_real_to_bf16([np.inf], [0.0])[0])


# ---------------------------------------------------------------------------
# the momentum kept in bf16
# ---------------------------------------------------------------------------
def _momentum_cases():
    rng = np.random.default_rng(93)
    cases = []
    for beta in (0.95, 0.9, float(TRAP_BETA)):
        b32 = np.float32(beta)
        m = bf16_values(rng, 600)
        g = (rng.standard_normal(600) * 2.0 ** rng.integers(-12, 2, 600)).astype(np.float32)
        mt, gt = near_tie_cases(rng, b32, 400)
        cases.append((beta, np.concatenate([m, mt]), np.concatenate([g, gt])))
        mx, gx = exact_tie_cases(rng, b32, 200)
        cases.append((beta, mx, gx))
    cases.append((float(TRAP_BETA), np.float32([TRAP_M]), np.float32([TRAP_G])))
    cases.append((float(DR_BETA), np.float32([DR_M]), np.float32([DR_G])))
    return cases


def check_momentum_exact(fn):
    for beta, m, g in _momentum_cases():
        got = fn(m.astype(np.float64), g.astype(np.float64), beta)
        b32 = np.float32(beta)
        exp = np.array([exact_momentum(b32, m[i], g[i]) for i in range(len(m))])
        if not np.array_equal(got, exp):
            return False
    return True


def test_bf16_momentum_against_exact_rationals():
    assert check_momentum_exact(oracle.momentum_update_bf16_state)


def test_bf16_momentum_special_cases():
    rng = np.random.default_rng(94)
    g = bf16_values(rng, 500).astype(np.float64)
    m = bf16_values(rng, 500).astype(np.float64)
    # beta = 0: the new momentum is G, exactly, when G is bf16
    assert np.array_equal(oracle.momentum_update_bf16_state(m, g, 0.0), g)
    # G = 0 and beta = 1/2: halving is exact
    assert np.array_equal(oracle.momentum_update_bf16_state(m, np.zeros(500), 0.5), m / 2)
    # both traps lie above the bf16 midpoint 1 + 2^-8: one rounding goes up
    r = oracle.momentum_update_bf16_state(np.array([float(TRAP_M)]), np.array([float(TRAP_G)]),
                                          float(TRAP_BETA))
    assert r[0] == 1 + 2 ** -7
    r = oracle.momentum_update_bf16_state(np.array([float(DR_M)]), np.array([float(DR_G)]),
                                          float(DR_BETA))
    assert r[0] == 1 + 2 ** -7
    with pytest.raises(ValueError):
        oracle.momentum_update_bf16_state(np.array([1 + 2 ** -10]), np.zeros(1), 0.9)
    # through the step entry points: M_new is bf16 and NS sees that value
    w = rng.standard_normal((6, 10)) * 0.02
    m0 = oracle.round_to_bf16(rng.standard_normal((6, 10)).astype(np.float32) * 0.01)
    g0 = rng.standard_normal((6, 10)) * 0.01
    _, m1, o = oracle.muonh_step(w, g0, m0, 1.0, 0.02, 0.95, 5, mom_bf16=True)
    assert np.array_equal(m1, oracle.momentum_update_bf16_state(m0, g0, 0.95))
    assert np.allclose(o, oracle.newton_schulz(m1, 5), rtol=0, atol=1e-15)
    _, m2, _ = oracle.muon_wd_step(w, g0, m0, 0.02, 0.95, 0.1, 5, mom_bf16=True)
    assert np.array_equal(m2, m1)


def _mutant(kind):
    def fn(m, g, beta):
        m = np.asarray(m, np.float64)
        g = np.asarray(g, np.float64)
        b = float(np.float32(beta)) if kind != "fp64_beta" else float(beta)
        if kind == "fp64_beta":     # beta not taken as its binary32 value
            return oracle.round_real_to_bf16(b * m + g, np.zeros(m.shape))
        if kind == "no_sticky":     # the float64 sum rounded, its error dropped
            return oracle.round_real_to_bf16(b * m + g, np.zeros(m.shape))
        t = fma_f32(np.full(m.shape, np.float32(b)), m.astype(np.float32), g.astype(np.float32))
        if kind == "truncate":
            u = t.view(np.uint32) & np.uint32(0xFFFF0000)
            return u.view(np.float32).astype(np.float64)
        if kind == "ties_away":
            u = (t.view(np.uint32) + np.uint32(0x8000)) & np.uint32(0xFFFF0000)
            return u.view(np.float32).astype(np.float64)
        if kind == "no_bf16_store":
            return t.astype(np.float64)
        return oracle.round_to_bf16(t)  # "through_binary32": two roundings
    return fn


@pytest.mark.parametrize("kind", ["through_binary32", "no_sticky", "fp64_beta", "truncate",
                                  "ties_away", "no_bf16_store"])
def test_planted_bf16_momentum_mistake_is_caught(kind):
    assert not check_momentum_exact(_mutant(kind))
