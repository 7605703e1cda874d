"""Pins of the fp64 oracle against facts fixed outside the oracle itself.

Nothing here compares the oracle with a retyped copy of its own formulas. The
pins are: the singular-value closed form (SVD brute force on tiny matrices),
exact-rational orbits of the scalar quintic (tests/golden), hand-checkable
projection values (tests/golden), invariants of the Newton-Schulz map
(transpose, scale and orthogonal equivariance), the band the quintic maps
singular values into, and the special cases the method reduces to (zero
gradient, zero learning rate, beta = 0, zero iterations). The last section
plants plausible mistakes in copies of the oracle's Newton-Schulz and
projection steps and checks that at least one pin fails for each.
"""
from __future__ import annotations

import math
from fractions import Fraction
from pathlib import Path

import numpy as np
import pytest

import oracle
import workloads

GOLDEN = Path(__file__).resolve().parent / "golden"

# The quintic coefficients, written here independently of the oracle's copy.
A_, B_, C_ = 3.4445, -4.7750, 2.0315


def p_scalar(s, k):
    s = np.asarray(s, dtype=np.float64)
    for _ in range(k):
        s = A_ * s + B_ * s ** 3 + C_ * s ** 5
    return s


def load_orbit():
    rows = {}
    for line in (GOLDEN / "quintic_orbit.txt").read_text().splitlines():
        if not line or line.startswith("#"):
            continue
        s0, k, v = line.split()
        rows[(float(Fraction(s0)), int(k))] = float(v)
    return rows


def rand(shape, key, std=1.0):
    return workloads.host_custom(shape, std, key).astype(np.float64)


def random_orthogonal(n, key):
    q, r = np.linalg.qr(rand((n, n), key))
    return q * np.sign(np.diag(r))


# ----------------------------------------------------------------------------
# Pin checks, written against an arbitrary Newton-Schulz callable so the
# mutation tests at the bottom can reuse them.
# ----------------------------------------------------------------------------

def svd_closed_form_error(ns, m, k, eps=oracle.NS_EPS):
    """Max abs error of ns(m, k) vs U diag(p^k(sigma/(||M||+eps))) V^T."""
    u, s, vt = np.linalg.svd(m, full_matrices=False)
    scale = np.linalg.norm(m) + eps
    expected = (u * p_scalar(s / scale, k)) @ vt
    return float(np.max(np.abs(ns(m, k) - expected)))


def check_svd_closed_form(ns):
    for idx, (r, c) in enumerate([(24, 40), (40, 24), (17, 17), (64, 96), (5, 3)]):
        m = rand((r, c), (1, idx))
        for k in (0, 1, 2, 5, 8):
            if svd_closed_form_error(ns, m, k) > 1e-11:
                return False
    return True


def check_rank_one_orbit(ns):
    orbit = load_orbit()
    u = rand((12, 1), (2, 0))
    v = rand((1, 20), (2, 1))
    m = 3.7 * (u / np.linalg.norm(u)) @ (v / np.linalg.norm(v))
    uv = m / 3.7
    for k in range(9):
        o = ns(m, k, eps=0.0)
        # rounding grows about 3.5x per iteration (|p'| along the orbit)
        if np.max(np.abs(o - orbit[(1.0, k)] * uv)) > 1e-11:
            return False
    return True


def check_orthonormal_rows(ns):
    q = random_orthogonal(96, (3, 0))
    for mrows in (8, 32):
        m = q[:mrows, :]                      # M M^T = I, ||M||_F = sqrt(mrows)
        for k in (1, 5):
            expected = p_scalar(1.0 / (math.sqrt(mrows) + oracle.NS_EPS), k) * m
            if np.max(np.abs(ns(m, k) - expected)) > 1e-12:
                return False
            if np.max(np.abs(ns(m.T, k) - expected.T)) > 1e-12:
                return False
    return True


def check_diagonal(ns):
    d = np.array([3.0, -1.0, 0.5, 2.0, -0.25])
    m = np.zeros((5, 7))
    m[np.arange(5), np.arange(5)] = d
    for k in (1, 3, 5):
        expected = np.zeros_like(m)
        expected[np.arange(5), np.arange(5)] = p_scalar(d / (np.linalg.norm(d) + oracle.NS_EPS), k)
        if np.max(np.abs(ns(m, k) - expected)) > 1e-12:
            return False
    return True


def check_equivariance(ns):
    m = rand((20, 36), (4, 0))
    o = ns(m, 5)
    if np.max(np.abs(ns(m.T, 5) - o.T)) > 1e-12:
        return False
    q1, q2 = random_orthogonal(20, (4, 1)), random_orthogonal(36, (4, 2))
    if np.max(np.abs(ns(q1 @ m @ q2, 5) - q1 @ o @ q2)) > 1e-11:
        return False
    if np.max(np.abs(ns(7.5 * m, 5, eps=0.0) - ns(m, 5, eps=0.0))) > 1e-12:
        return False
    return True


def check_projection_golden(project):
    lines = [l for l in (GOLDEN / "projection_2x3.txt").read_text().splitlines()
             if l and not l.startswith("#")]
    expected = np.array([float(v) for v in lines[0].split()]).reshape(2, 3)
    w = np.array([[3.0, 4.0, 0.0], [0.0, 0.0, 0.0]])
    o = np.array([[1.0, 0.0, 0.0], [0.0, 0.0, 2.0]])
    got = project(w, o, 5.0, 1.0)
    return bool(np.max(np.abs(got - expected)) <= 1e-15 * 8)


def check_projection_sphere(project):
    for idx, (r, c) in enumerate([(16, 48), (48, 16), (33, 33)]):
        w = rand((r, c), (5, idx), 0.02)
        o = oracle.newton_schulz(rand((r, c), (5, 10 + idx)), 5)
        radius = 0.7
        wn = project(w, o, radius, 0.02)
        if abs(np.linalg.norm(wn) - radius) > 1e-13:
            return False
        trial = w - 0.02 * o
        cos = np.sum(wn * trial) / (np.linalg.norm(wn) * np.linalg.norm(trial))
        if abs(cos - 1.0) > 1e-13:
            return False
    return True


# ----------------------------------------------------------------------------
# The pins applied to the oracle.
# ----------------------------------------------------------------------------

def test_coefficients_are_the_quintic():
    assert oracle.NS_COEFFS == (A_, B_, C_)
    assert oracle.NS_EPS == 1e-7
    # p(1) = a + b + c
    assert abs(p_scalar(1.0, 1) - 0.701) < 1e-15


def test_golden_orbit_matches_float_iteration():
    orbit = load_orbit()
    for (s0, k), v in orbit.items():
        assert abs(float(p_scalar(s0, k)) - v) < 1e-14


def test_ns_svd_closed_form():
    assert check_svd_closed_form(oracle.newton_schulz)


def test_ns_svd_closed_form_large_rectangular():
    m = rand((64, 160), (6, 0), 0.01)
    assert svd_closed_form_error(oracle.newton_schulz, m, 5) < 1e-12
    assert svd_closed_form_error(oracle.newton_schulz, m.T, 8) < 1e-12


def test_ns_rank_one_golden():
    assert check_rank_one_orbit(oracle.newton_schulz)


def test_ns_orthonormal_rows():
    assert check_orthonormal_rows(oracle.newton_schulz)


def test_ns_diagonal_entrywise():
    assert check_diagonal(oracle.newton_schulz)


def test_ns_equivariances():
    assert check_equivariance(oracle.newton_schulz)


@pytest.mark.parametrize("k", [5, 8])
def test_ns_band(k):
    # Normalised singular values >= 1e-2 land in [0.6818, 1.1344] after 5 or 8
    # iterations: the quintic maps that interval into itself (next test) and
    # lifts every value >= 1e-2 into it within 5 steps.
    n = 48
    u = random_orthogonal(n, (7, 0))
    v = random_orthogonal(80, (7, 1))[:n, :]
    sig = np.geomspace(1.0, 0.05, n)
    m = (u * sig) @ v
    sig_hat = sig / (np.linalg.norm(sig) + oracle.NS_EPS)
    assert sig_hat.min() >= 1e-2
    o = oracle.newton_schulz(m, k)
    s = np.linalg.svd(o, compute_uv=False)
    assert s.min() >= 0.6818 - 1e-9 and s.max() <= 1.1344 + 1e-9
    # every output singular value is the scalar map of an input one
    np.testing.assert_allclose(np.sort(s), np.sort(np.abs(p_scalar(sig_hat, k))), rtol=0, atol=1e-12)


def test_quintic_band_is_invariant():
    grid = np.linspace(0.6818, 1.1344, 200001)
    img = p_scalar(grid, 1)
    assert img.min() >= 0.6818 - 1e-6 and img.max() <= 1.1344 + 1e-6
    # fixed points 0.8680 (repelling within the band) and 1.2637
    for fp in (0.8680, 1.2637):
        assert abs(float(p_scalar(fp, 1)) - fp) < 2e-4


def test_ns_zero_iterations_is_normalised_momentum():
    m = rand((9, 13), (8, 0))
    o = oracle.newton_schulz(m, 0)
    np.testing.assert_allclose(o, m / (np.linalg.norm(m) + 1e-7), rtol=0, atol=1e-15)


def test_ns_zero_input():
    o = oracle.newton_schulz(np.zeros((6, 10)), 5)
    assert np.all(o == 0.0)


def test_projection_golden():
    assert check_projection_golden(oracle.hyperball_project)


def test_projection_sphere_and_direction():
    assert check_projection_sphere(oracle.hyperball_project)


def test_projection_degenerate_zero_radius():
    w = np.zeros((3, 4))
    o = np.zeros((3, 4))
    assert np.all(oracle.hyperball_project(w, o, 0.0, 0.02) == 0.0)


def test_momentum_hand_values():
    m = np.array([[1.0, -2.0], [0.5, 0.0]])
    g = np.array([[2.0, 1.0], [-1.0, 3.0]])
    np.testing.assert_array_equal(oracle.momentum_update(m, g, 0.5),
                                  np.array([[2.5, 0.0], [-0.75, 3.0]]))
    np.testing.assert_array_equal(oracle.momentum_update(m, g, 0.0), g)


def test_step_zero_gradient_zero_momentum_keeps_w():
    w = rand((12, 20), (9, 0), 0.02)
    r = oracle.init_radius(w)
    w1, m1, o = oracle.muonh_step(w, np.zeros_like(w), np.zeros_like(w), r, 0.02, 0.95, 5)
    assert np.all(m1 == 0.0) and np.all(o == 0.0)
    np.testing.assert_allclose(w1, w, rtol=1e-14, atol=0)


def test_step_zero_gradient_momentum_only():
    # G = 0, M != 0: the update is NS(beta*M) = NS(M) (scale invariance), and
    # W moves by that momentum term, then returns to the sphere.
    w = rand((12, 20), (10, 0), 0.02)
    m = rand((12, 20), (10, 1), 0.01)
    r = oracle.init_radius(w)
    # eps = 0 makes the scale invariance exact (eps only enters as eps/||M||)
    w1, m1, o = oracle.muonh_step(w, np.zeros_like(w), m, r, 0.02, 0.9, 5, eps=0.0)
    np.testing.assert_allclose(m1, 0.9 * m, rtol=1e-15)
    np.testing.assert_allclose(o, oracle.newton_schulz(m, 5, eps=0.0), rtol=0, atol=1e-12)
    assert abs(np.linalg.norm(w1) - r) < 1e-13


def test_step_zero_lr_keeps_w_on_sphere():
    w = rand((16, 8), (11, 0), 0.02)
    r = oracle.init_radius(w)
    w1, _, _ = oracle.muonh_step(w, rand((16, 8), (11, 1), 0.01), np.zeros_like(w), r, 0.0, 0.95, 5)
    np.testing.assert_allclose(w1, w, rtol=1e-14, atol=0)


def test_step_beta_zero_momentum_is_gradient():
    w = rand((8, 8), (12, 0), 0.02)
    g = rand((8, 8), (12, 1), 0.01)
    m = rand((8, 8), (12, 2), 0.01)
    _, m1, _ = oracle.muonh_step(w, g, m, oracle.init_radius(w), 0.02, 0.0, 5)
    np.testing.assert_array_equal(m1, g)


def test_trajectory_stays_on_sphere_small_workload():
    wl = workloads.WORKLOADS["single_128x256"]
    w = workloads.host_weight(wl, 0).astype(np.float64)
    r = oracle.init_radius(w)
    m = np.zeros_like(w)
    for step in range(wl.steps):
        g = workloads.host_grad(wl, 0, step)
        w, m, o = oracle.muonh_step(w, g, m, r, wl.lr, wl.beta, wl.ns_iters[0])
        assert abs(np.linalg.norm(w) / r - 1.0) < 1e-12
        s = np.linalg.svd(o, compute_uv=False)
        assert s.max() < 1.2025 and s.min() > 0.0


# ----------------------------------------------------------------------------
# Planted mistakes: each mutant differs from the oracle by one plausible bug
# and must be caught by at least one pin.
# ----------------------------------------------------------------------------

def _ns_mutant(kind):
    a, b, c = oracle.NS_COEFFS

    def ns(m, k, eps=oracle.NS_EPS):
        x = np.asarray(m, dtype=np.float64)
        t = x.shape[0] > x.shape[1]
        if t and kind != "no_transpose_back":
            x = x.T
        elif t:
            x = x.T
        nrm = np.linalg.norm(x)
        if kind == "eps_inside_sqrt":
            x = x / math.sqrt(nrm * nrm + eps)
        elif kind == "no_normalise":
            pass
        elif kind == "max_norm":
            x = x / (np.abs(x).max() + eps)
        else:
            x = x / (nrm + eps)
        for _ in range(k):
            g = x @ x.T
            if kind == "swap_bc":
                poly = c * g + b * (g @ g)
            elif kind == "drop_quintic":
                poly = b * g
            elif kind == "minus_b":
                poly = -b * g + c * (g @ g)
            else:
                poly = b * g + c * (g @ g)
            if kind == "a_times_poly":
                x = a * (x + poly @ x)
            elif kind == "extra_iteration":
                x = a * x + poly @ x
                g = x @ x.T
                x = a * x + (b * g + c * (g @ g)) @ x
            else:
                x = a * x + poly @ x
        if t and kind == "no_transpose_back":
            return x.reshape(m.shape)
        return x.T if t else x

    return ns


NS_MUTANTS = ["no_transpose_back", "eps_inside_sqrt", "no_normalise", "max_norm", "swap_bc",
              "drop_quintic", "minus_b", "a_times_poly", "extra_iteration"]


@pytest.mark.parametrize("kind", NS_MUTANTS)
def test_planted_ns_mistake_is_caught(kind):
    ns = _ns_mutant(kind)
    caught = (not check_svd_closed_form(ns) or not check_rank_one_orbit(ns)
              or not check_orthonormal_rows(ns) or not check_diagonal(ns)
              or not check_equivariance(ns))
    assert caught, f"mutant {kind} passed every pin"


def test_unmutated_copy_passes_every_pin():
    ns = _ns_mutant("none")
    assert check_svd_closed_form(ns) and check_rank_one_orbit(ns)
    assert check_orthonormal_rows(ns) and check_diagonal(ns) and check_equivariance(ns)


def _project_mutant(kind):
    def project(w, o, radius, lr):
        w = np.asarray(w, dtype=np.float64)
        o = np.asarray(o, dtype=np.float64)
        trial = w + lr * o if kind == "plus_lr" else w - lr * o
        if kind == "norm_of_w":
            n = np.linalg.norm(w)
        elif kind == "squared_norm":
            n = np.sum(trial * trial)
        else:
            n = np.linalg.norm(trial)
        if kind == "no_radius":
            return trial / n
        if kind == "scale_w_only":
            return (radius / n) * w - lr * o
        return (radius / n) * trial

    return project


@pytest.mark.parametrize("kind", ["plus_lr", "norm_of_w", "squared_norm", "no_radius", "scale_w_only"])
def test_planted_projection_mistake_is_caught(kind):
    pr = _project_mutant(kind)
    assert not (check_projection_golden(pr) and check_projection_sphere(pr))


# ----------------------------------------------------------------------------
# The bf16 emulation used as the error floor of tiny matrices in GPU parity.
# ----------------------------------------------------------------------------

def test_bf16_rounding_is_nearest_even():
    from bf16_floor import round_bf16
    one = 1.0
    ulp = 2.0 ** -7                      # bf16 spacing at 1.0
    assert round_bf16(one + ulp / 2) == one            # tie -> even (1.0)
    assert round_bf16(one + 3 * ulp / 2) == one + 2 * ulp  # tie -> even
    assert round_bf16(one + ulp / 2 + 2 ** -20) == one + ulp
    assert round_bf16(-(one + ulp / 4)) == -one
    assert np.isnan(round_bf16(np.float32("nan")))


@pytest.mark.parametrize("scale", [1e-9, 1.0, 1e6])
@pytest.mark.parametrize("shape", [(48, 80), (80, 48)])
def test_deferred_normalisation_is_exact_algebra(scale, shape):
    # The GPU path stores M unscaled and applies sigma = 1/(||M|| + eps) as
    # sigma^2 on the first Gram and sigma on the first apply (both terms).
    # Without rounding that must be the oracle's iteration on M/(||M|| + eps),
    # eps included (at ||M|| ~ 1e-7 it changes the result).
    # sigma is far from 1 at scales 1e-9 and 1e6, so a wrong power of sigma
    # on either GEMM would not match.
    from bf16_floor import _ns_emulated
    m = rand(shape, (23, shape[0]), 0.01 * scale)
    for k in (1, 2, 5):
        ref = oracle.newton_schulz(m, k)
        got = _ns_emulated(m, k, "exact", deferred=True)
        assert np.linalg.norm(got - ref) <= 1e-11 * max(np.linalg.norm(ref), 1e-300)
    if scale == 1e-9:
        # ||M|| ~ 6e-10 << eps: eps is honoured, the eps-free iteration differs
        no_eps = oracle.newton_schulz(m, 1, eps=0.0)
        assert np.linalg.norm(_ns_emulated(m, 1, "exact") - no_eps) > 1e-3 * np.linalg.norm(no_eps)


@pytest.mark.parametrize("shape", [(48, 80), (80, 48), (64, 64)])
def test_folded_polynomial_is_exact_algebra(shape):
    # Matrices of more than 65536 entries take B' = a*I + b*A + c*A*A and
    # X <- B' X (no a*X term): without rounding, the oracle's iteration, also
    # combined with the deferred normalisation. A missing or misplaced a*I
    # (off the diagonal, or also kept as a*X) would not match.
    from bf16_floor import _ns_emulated
    m = rand(shape, (24, shape[0]), 0.01)
    for k in (1, 2, 5):
        ref = oracle.newton_schulz(m, k)
        for deferred in (False, True):
            got = _ns_emulated(m, k, "exact", deferred=deferred, fold=True)
            assert np.linalg.norm(got - ref) <= 1e-11 * np.linalg.norm(ref)


def test_split_bf16_pair_carries_sixteen_bits():
    # hi + lo represents an fp32 value to within about 2^-17 of its magnitude
    # (hi has 8 significant bits, lo the next 8 and a rounding bit), and lo is
    # exactly the rounded remainder of hi.
    from bf16_floor import round_bf16, split_bf16
    x = rand((4096,), (21, 0), 1.0).astype(np.float32).astype(np.float64)
    hi, lo = split_bf16(x)
    np.testing.assert_array_equal(hi, round_bf16(x))
    assert np.all(np.abs(x - (hi + lo)) <= 2.0 ** -16 * np.abs(x))
    assert np.max(np.abs(x - (hi + lo)) / np.abs(x)) > 2.0 ** -20   # not exact: 8 more bits only
    v = np.float64(1.0 + 2.0 ** -7 + 2.0 ** -15)   # hi = 1 + 2^-7, lo = 2^-15 exactly
    h, l = split_bf16(v)
    assert h == 1.0 + 2.0 ** -7 and l == 2.0 ** -15


@pytest.mark.parametrize("shape,k", [((128, 256), 5), ((384, 640), 8)])
def test_split_bf16_floor_is_far_below_bf16(shape, k):
    # The split emulation (hi + lo operands, lo*lo omitted) lands near
    # 2^-8 of the bf16 floor: 2e-5 to 6e-5 on these shapes.
    from bf16_floor import floor
    m = rand(shape, (22, shape[0]), 0.01)
    ref = oracle.newton_schulz(m, k)
    f16 = floor(m, k, ref)
    fsp = floor(m, k, ref, "split_bf16")
    assert fsp < 1e-4
    assert fsp < f16 / 100


@pytest.mark.parametrize("shape,k,limit", [((128, 256), 5, 1.4e-2), ((512, 1536), 5, 1.4e-2),
                                           ((384, 640), 8, 2.3e-2), ((1024, 3072), 8, 2.0e-2)])
def test_bf16_floor_by_shape(shape, k, limit):
    # Records the error that bf16 storage alone costs: about 1.1e-2 at 5
    # iterations, and 1.8e-2 to 2.2e-2 at 8 (the quintic's repelling fixed
    # point amplifies rounding by about 1.6x per iteration), so the 2e-2 bound
    # is only marginally reachable with bf16 operands at 8 iterations.
    from bf16_floor import floor
    m = rand(shape, (20, shape[0]), 0.01)
    assert floor(m, k, oracle.newton_schulz(m, k)) < limit


# ----------------------------------------------------------------------------
# Muon with decoupled weight decay (the baseline MuonH is measured against)
# ----------------------------------------------------------------------------

def _muon_golden_inputs():
    u = np.array([3 / 5, 4 / 5])
    v = np.array([2 / 3, 1 / 3, 2 / 3])
    w = np.array([[1.0, -2.0, 3.0], [0.0, 5.0, -1.0]])
    return w, np.outer(u, v)


def _golden_muon_wd():
    rows = [l for l in (GOLDEN / "muon_wd_2x3.txt").read_text().splitlines() if not l.startswith("#")]
    return np.array([float(x) for x in rows[0].split()]).reshape(2, 3)


def check_muon_golden(step):
    w, g = _muon_golden_inputs()
    w_new, m_new, o = step(w, g, np.zeros_like(g), 0.02, 0.95, 0.1, 5)
    return np.allclose(w_new, _golden_muon_wd(), rtol=0, atol=1e-13)


def check_muon_decay_only(step):
    w = rand((6, 9), (24, 0), 0.02)
    z = np.zeros_like(w)
    w_new, m_new, o = step(w, z, z, 0.02, 0.9, 0.1, 5)
    return np.array_equal(w_new, (1.0 - 0.02 * 0.1) * w) and not np.any(o)


def test_muon_wd_golden():
    # exact-rational expected values (tests/golden/make_golden.py)
    assert check_muon_golden(oracle.muon_wd_step)


def test_muon_wd_decay_only():
    assert check_muon_decay_only(oracle.muon_wd_step)


def test_muon_wd_without_decay_is_the_muonh_trial_update():
    # wd = 0: W - lr*O, i.e. MuonH's W' before the projection; projecting it
    # gives MuonH's result.
    w = rand((24, 40), (25, 0), 0.02)
    g = rand((24, 40), (25, 1), 0.01)
    m = rand((24, 40), (25, 2), 0.01)
    w_new, m_new, o = oracle.muon_wd_step(w, g, m, 0.02, 0.95, 0.0, 5)
    np.testing.assert_allclose(w_new, w - 0.02 * o, rtol=0, atol=1e-15)
    r = oracle.init_radius(w)
    w_h, m_h, o_h = oracle.muonh_step(w, g, m, r, 0.02, 0.95, 5)
    np.testing.assert_array_equal(o, o_h)
    np.testing.assert_allclose(w_h, r * w_new / np.linalg.norm(w_new), rtol=1e-14, atol=0)


def _muon_mutant(kind):
    def step(w, g, m, lr, beta, wd, k):
        m_new = oracle.momentum_update(m, g, beta)
        o = oracle.newton_schulz(m_new, k)
        w = np.asarray(w, dtype=np.float64)
        if kind == "coupled":
            w_new = (1.0 - lr * wd) * (w - lr * o)
        elif kind == "plus_decay":
            w_new = (1.0 + lr * wd) * w - lr * o
        elif kind == "decay_on_update":
            w_new = w - lr * (o + wd * o)
        else:  # "no_decay"
            w_new = w - lr * o
        return w_new, m_new, o
    return step


@pytest.mark.parametrize("kind", ["coupled", "plus_decay", "decay_on_update", "no_decay"])
def test_planted_muon_wd_mistake_is_caught(kind):
    step = _muon_mutant(kind)
    assert not (check_muon_golden(step) and check_muon_decay_only(step))


# ----------------------------------------------------------------------------
# AdamW for the parameters outside the MuonH group
# ----------------------------------------------------------------------------
ADAMW_HP = dict(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)


def check_adamw_first_step(step_fn):
    # zero state, step 1: m_hat = g and v_hat = g^2 exactly, so every element
    # moves by lr * g / (|g| + eps) after the decay
    p = rand((300,), (26, 0), 1.0)
    g = rand((300,), (26, 1), 0.01)
    z = np.zeros_like(p)
    h = ADAMW_HP
    p1, m1, v1 = step_fn(p, g, z, z, h["lr"], h["beta1"], h["beta2"], h["eps"], h["weight_decay"], 1)
    exp = p * (1 - h["lr"] * h["weight_decay"]) - h["lr"] * g / (np.abs(g) + h["eps"])
    return np.allclose(p1, exp, rtol=1e-14, atol=1e-17) and np.allclose(m1, 0.1 * g, rtol=1e-14)


def check_adamw_constant_gradient(step_fn, steps=7):
    # constant g from zero state: m_hat = g and v_hat = g^2 at every step, so
    # p_t = p0 c^t - lr s (1 + c + ... + c^(t-1)), c = 1 - lr wd, s = g/(|g|+eps)
    h = ADAMW_HP
    p0 = rand((200,), (27, 0), 1.0)
    g = rand((200,), (27, 1), 0.01)
    p, m, v = p0, np.zeros_like(p0), np.zeros_like(p0)
    for t in range(1, steps + 1):
        p, m, v = step_fn(p, g, m, v, h["lr"], h["beta1"], h["beta2"], h["eps"], h["weight_decay"], t)
    c = 1 - h["lr"] * h["weight_decay"]
    s = g / (np.abs(g) + h["eps"])
    exp = p0 * c ** steps - h["lr"] * s * sum(c ** i for i in range(steps))
    return np.allclose(p, exp, rtol=1e-12, atol=1e-15)


def check_adamw_decay_only(step_fn):
    h = ADAMW_HP
    p = rand((64,), (28, 0), 1.0)
    z = np.zeros_like(p)
    p1, m1, v1 = step_fn(p, z, z, z, h["lr"], h["beta1"], h["beta2"], h["eps"], h["weight_decay"], 3)
    return np.array_equal(p1, p * (1 - h["lr"] * h["weight_decay"])) and not np.any(m1) and not np.any(v1)


def check_adamw_golden(step_fn):
    rows = [l for l in (GOLDEN / "adamw_2step.txt").read_text().splitlines() if not l.startswith("#")]
    p2e, m2e, v2e = (np.array([float(x) for x in r.split()]) for r in rows)
    p = np.array([0.5, -1.25, 0.0, 2.0])
    m = v = np.zeros(4)
    for t, g in enumerate([np.array([0.3, -0.2, 0.0, 1e-3]), np.array([-0.1, -0.4, 0.05, 2e-3])], 1):
        p, m, v = step_fn(p, g, m, v, 1e-3, 0.9, 0.95, 1e-8, 0.1, t)
    return (np.allclose(p, p2e, rtol=1e-14, atol=1e-16) and np.allclose(m, m2e, rtol=1e-14)
            and np.allclose(v, v2e, rtol=1e-14))


def test_adamw_first_step_closed_form():
    assert check_adamw_first_step(oracle.adamw_step)


def test_adamw_constant_gradient_closed_form():
    assert check_adamw_constant_gradient(oracle.adamw_step)


def test_adamw_decay_only():
    assert check_adamw_decay_only(oracle.adamw_step)


def test_adamw_two_step_golden():
    # 50-digit decimal evaluation of the definition (tests/golden/make_golden.py)
    assert check_adamw_golden(oracle.adamw_step)


def _adamw_mutant(kind):
    def step(p, g, m, v, lr, b1, b2, eps, wd, t):
        p = np.asarray(p, dtype=np.float64)
        g = np.asarray(g, dtype=np.float64)
        if kind == "coupled_l2":
            g = g + wd * p
        else:
            p = p * (1 - lr * wd)
        m = (b2 if kind == "swapped_betas" else b1) * m + (1 - (b2 if kind == "swapped_betas" else b1)) * g
        v = (b1 if kind == "swapped_betas" else b2) * v + (1 - (b1 if kind == "swapped_betas" else b2)) * g * g
        if kind == "no_bias_correction":
            mh, vh = m, v
        else:
            mh, vh = m / (1 - b1 ** t), v / (1 - b2 ** t)
        if kind == "eps_inside_sqrt":
            den = np.sqrt(vh + eps)
        else:
            den = np.sqrt(vh) + eps
        return p - lr * mh / den, m, v
    return step


@pytest.mark.parametrize("kind", ["coupled_l2", "no_bias_correction", "eps_inside_sqrt", "swapped_betas"])
def test_planted_adamw_mistake_is_caught(kind):
    s = _adamw_mutant(kind)
    assert not (check_adamw_first_step(s) and check_adamw_constant_gradient(s)
                and check_adamw_decay_only(s) and check_adamw_golden(s))
