"""Writes the closed-form fixtures in this folder. Run: python tests/golden/make_golden.py

The values are computed in exact rational arithmetic (Python's fractions), from
the definition of the odd quintic p(s) = a*s + b*s^3 + c*s^5 with
(a, b, c) = (3.4445, -4.7750, 2.0315). Nothing here calls the GPU path or the
oracle's matrix code; the fixtures pin the oracle from the outside.
"""
from fractions import Fraction
from pathlib import Path

A, B, C = Fraction("3.4445"), Fraction("-4.7750"), Fraction("2.0315")


def p(s: Fraction) -> Fraction:
    return A * s + B * s ** 3 + C * s ** 5


def orbit(s0: Fraction, n: int):
    out, s = [s0], s0
    for _ in range(n):
        s = p(s)
        out.append(s)
    return out


def main() -> None:
    here = Path(__file__).resolve().parent
    lines = [
        "# p^k(s0) for the Newton-Schulz quintic p(s) = a s + b s^3 + c s^5,",
        "# (a, b, c) = (3.4445, -4.7750, 2.0315); exact rationals rounded to 17 digits.",
        "# Citation: closed form of the per-singular-value map of the iteration",
        "# X <- aX + b(XX^T)X + c(XX^T)^2 X (the odd-quintic reading of the",
        "# Newton-Schulz step the digest page names in its footnote 4).",
        "# columns: s0 k value",
    ]
    for s0 in (Fraction(1), Fraction(1, 2), Fraction(1, 10), Fraction(1, 100)):
        for k, v in enumerate(orbit(s0, 8)):
            lines.append(f"{s0} {k} {float(v):.17g}")
    (here / "quintic_orbit.txt").write_text("\n".join(lines) + "\n")

    # A 2x3 worked projection example, exact: W = [[3,4,0],[0,0,0]], O = [[1,0,0],[0,0,2]],
    # lr = 1, R = 5: W' = [[2,4,0],[0,0,-2]], ||W'||^2 = 24, W_new = (5/sqrt(24)) W'.
    lines = [
        "# Hand-checkable hyperball projection: W <- R (W - lr O) / ||W - lr O||_F",
        "# (digest page, section \"The load-bearing tricks aren't in the abstract\").",
        "# W = [[3,4,0],[0,0,0]], O = [[1,0,0],[0,0,2]], lr = 1, R = 5",
        "# W' = [[2,4,0],[0,0,-2]], ||W'||_F^2 = 24; expected = 5/sqrt(24) * W'",
        "# row-major expected values:",
    ]
    import math
    s = 5.0 / math.sqrt(24.0)
    vals = [2 * s, 4 * s, 0.0, 0.0, 0.0, -2 * s]
    lines.append(" ".join(f"{v:.17g}" for v in vals))
    (here / "projection_2x3.txt").write_text("\n".join(lines) + "\n")

    # Muon with decoupled weight decay on a rank-one momentum, exact: with
    # M = u v^T, ||u|| = ||v|| = 1, X0 = M / (1 + eps) has the single singular
    # value s0 = 1/(1 + eps), so O = p^5(s0) u v^T, and
    # W_new = (1 - lr wd) W - lr O.
    eps = Fraction(1, 10 ** 7)
    u = [Fraction(3, 5), Fraction(4, 5)]
    v = [Fraction(2, 3), Fraction(1, 3), Fraction(2, 3)]
    w = [[1, -2, 3], [0, 5, -1]]
    lr, wd = Fraction(1, 50), Fraction(1, 10)
    s5 = orbit(1 / (1 + eps), 5)[5]
    wn = [[(1 - lr * wd) * w[i][j] - lr * s5 * u[i] * v[j] for j in range(3)] for i in range(2)]
    lines = [
        "# Muon with decoupled weight decay, W <- (1 - lr wd) W - lr O, O = NS_5(M)",
        "# (the baseline MuonH is measured against: digest page, section \"The",
        "# load-bearing tricks aren't in the abstract\"; report part 6/7, 4.3).",
        "# W = [[1,-2,3],[0,5,-1]], M0 = 0, G = u v^T with u = (3/5, 4/5),",
        "# v = (2/3, 1/3, 2/3), lr = 1/50, wd = 1/10, 5 iterations, eps = 1e-7:",
        "# O = p^5(1/(1+eps)) u v^T exactly. Row-major expected W_new:",
        " ".join(f"{float(x):.17g}" for row in wn for x in row),
    ]
    (here / "muon_wd_2x3.txt").write_text("\n".join(lines) + "\n")

    # Two AdamW steps with different gradients, computed from the definition
    # in 50-digit decimal arithmetic (decoupled decay, bias-corrected moments,
    # eps outside the square root).
    from decimal import Decimal, getcontext
    getcontext().prec = 50
    D = Decimal
    lr, b1, b2, ep, wd = D("0.001"), D("0.9"), D("0.95"), D("1e-8"), D("0.1")
    p0 = [D("0.5"), D("-1.25"), D("0.0"), D("2.0")]
    gs = [[D("0.3"), D("-0.2"), D("0.0"), D("1e-3")], [D("-0.1"), D("-0.4"), D("0.05"), D("2e-3")]]
    pv, mv, vv = list(p0), [D(0)] * 4, [D(0)] * 4
    for t, g in enumerate(gs, start=1):
        for i in range(4):
            pv[i] = pv[i] * (1 - lr * wd)
            mv[i] = b1 * mv[i] + (1 - b1) * g[i]
            vv[i] = b2 * vv[i] + (1 - b2) * g[i] * g[i]
            mh = mv[i] / (1 - b1 ** t)
            vh = vv[i] / (1 - b2 ** t)
            pv[i] = pv[i] - lr * mh / (vh.sqrt() + ep)
    lines = [
        "# Two AdamW steps (model card page \"Puro\", section \"Training\": AdamW,",
        "# weight decay 0.1), from the definition in 50-digit decimal arithmetic:",
        "# lr = 1e-3, beta1 = 0.9, beta2 = 0.95, eps = 1e-8, wd = 0.1,",
        "# p0 = (0.5, -1.25, 0, 2), m0 = v0 = 0,",
        "# g1 = (0.3, -0.2, 0, 1e-3), g2 = (-0.1, -0.4, 0.05, 2e-3).",
        "# lines: p2, m2, v2",
    ]
    for vec in (pv, mv, vv):
        lines.append(" ".join(f"{float(x):.17g}" for x in vec))
    (here / "adamw_2step.txt").write_text("\n".join(lines) + "\n")


if __name__ == "__main__":
    main()
