"""Per-step coefficient tables for the quintic Newton-Schulz iteration.

Each step applies p(x) = a x + b x^3 + c x^5 to every singular value of the
(Frobenius-normalised) momentum. Two tables are provided:

* ``keller_jordan(steps)``: the single triple (3.4445, -4.7750, 2.0315)
  repeated ("Chapter 4: The MuonAdamW Optimizer", section "Polar Express:
  Newton-Schulz Orthogonalization"; "3.9 Optimizers: SGD, Adam, Adafactor,
  Lion, Muon & Shampoo", section "Muon: Orthogonalizing the Update").
* ``polar_express(steps, ...)``: a different polynomial at every step, the
  "hard-coded quintic Polar Express steps" of the nanochat discussion ("Stuck
  at the optimizer after figuring out backward()"). The pages name the method
  but print no numbers, so the table is derived here from its construction:
  at step t the singular values are known to lie in [l_t, u_t]; p_t is the
  odd quintic closest to 1 in the uniform norm on that interval, and the next
  interval is its image, [1 - E_t, 1 + E_t] with E_t the minimax error.

The minimax polynomial is found by the Remez exchange: {x, x^3, x^5} is a
Chebyshev system on x > 0, so the best approximation of 1 equioscillates at
four points, here the two ends of the interval and the two interior critical
points of p.

Two options guard the table for low-precision arithmetic:

* ``safety`` > 1 evaluates each polynomial at x / safety, so that values a
  little above u (after bf16 rounding) are still mapped below the next
  interval's top;
* ``cushion`` raises each lower end to at least cushion * u. Early steps
  then target a wider image than the exact minimax would, with milder
  coefficients. 0 keeps the plain greedy construction.

This module is host-side arithmetic on a handful of floats; it runs once per
table and nothing in it touches the GPU.
"""
from __future__ import annotations

import math
from typing import List, Sequence, Tuple

KJ_TRIPLE = (3.4445, -4.7750, 2.0315)

Triple = Tuple[float, float, float]


def keller_jordan(steps: int = 5) -> List[Triple]:
    return [KJ_TRIPLE] * steps


def _poly(abc: Triple, x: float) -> float:
    a, b, c = abc
    x2 = x * x
    return x * (a + x2 * (b + c * x2))


def _critical_points(abc: Triple, lo: float, hi: float) -> List[float]:
    """Interior points of (lo, hi) where p'(x) = a + 3 b x^2 + 5 c x^4 = 0."""
    a, b, c = abc
    ys = []
    if abs(c) > 0.0:
        disc = 9.0 * b * b - 20.0 * a * c
        if disc >= 0.0:
            r = math.sqrt(disc)
            ys = [(-3.0 * b - r) / (10.0 * c), (-3.0 * b + r) / (10.0 * c)]
    elif abs(b) > 0.0:
        ys = [-a / (3.0 * b)]
    xs = sorted(math.sqrt(y) for y in ys if y > 0.0)
    return [x for x in xs if lo < x < hi]


def _solve4(rows: Sequence[Sequence[float]], rhs: Sequence[float]) -> List[float]:
    """Gaussian elimination with partial pivoting on a 4 x 4 system."""
    m = [list(r) + [v] for r, v in zip(rows, rhs)]
    n = 4
    for col in range(n):
        piv = max(range(col, n), key=lambda r: abs(m[r][col]))
        m[col], m[piv] = m[piv], m[col]
        for r in range(col + 1, n):
            f = m[r][col] / m[col][col]
            for k in range(col, n + 1):
                m[r][k] -= f * m[col][k]
    out = [0.0] * n
    for r in range(n - 1, -1, -1):
        out[r] = (m[r][n] - sum(m[r][k] * out[k] for k in range(r + 1, n))) / m[r][r]
    return out


def minimax_odd_quintic(lo: float, hi: float, max_iter: int = 200, tol: float = 1e-15) -> Tuple[Triple, float]:
    """The odd quintic p minimising max_{x in [lo, hi]} |1 - p(x)|, and that
    maximum E. Requires 0 < lo < hi."""
    if not (0.0 < lo < hi):
        raise ValueError("need 0 < lo < hi")
    # initial reference: the interval's ends and two Chebyshev-spaced points
    ref = [lo + (hi - lo) * (1.0 - math.cos(math.pi * k / 3.0)) / 2.0 for k in range(4)]
    abc: Triple = (1.0, 0.0, 0.0)
    err = 1.0
    for _ in range(max_iter):
        # p(x_k) + (-1)^k E = 1: the error 1 - p alternates +E, -E, +E, -E
        rows = [[x, x ** 3, x ** 5, (-1.0) ** k] for k, x in enumerate(ref)]
        a, b, c, e = _solve4(rows, [1.0] * 4)
        abc, err = (a, b, c), abs(e)
        crit = _critical_points(abc, lo, hi)
        if len(crit) != 2:
            break
        new_ref = [lo, crit[0], crit[1], hi]
        moved = max(abs(p - q) for p, q in zip(new_ref, ref))
        ref = new_ref
        if moved <= tol * hi:
            break
    # the levelled error at the reference is the minimax error once the
    # interior critical points are the reference points; report the true max
    pts = [lo, hi] + _critical_points(abc, lo, hi)
    err = max(abs(1.0 - _poly(abc, x)) for x in pts)
    return abc, err


def polar_express(steps: int = 5, lower: float = 1e-3, safety: float = 1.0, cushion: float = 0.0) -> List[Triple]:
    """Greedy per-step minimax table for ``steps`` steps, starting from
    singular values in [lower, 1] (Frobenius normalisation puts them in (0, 1])."""
    if steps < 0 or not (0.0 < lower < 1.0) or safety < 1.0 or not (0.0 <= cushion < 1.0):
        raise ValueError("need steps >= 0, 0 < lower < 1, safety >= 1, 0 <= cushion < 1")
    lo, hi = lower, 1.0
    table: List[Triple] = []
    for _ in range(steps):
        lo_eff = max(lo, cushion * hi)
        (a, b, c), _ = minimax_odd_quintic(lo_eff, hi)
        # p(x / s): coefficients a/s, b/s^3, c/s^5
        s = safety
        abc = (a / s, b / s ** 3, c / s ** 5)
        table.append(abc)
        # image of [lo, hi] under the polynomial actually used
        pts = [lo, hi] + _critical_points(abc, lo, hi)
        vals = [_poly(abc, x) for x in pts]
        lo, hi = min(vals), max(vals)
        if lo <= 0.0:
            raise ValueError("a step maps part of the interval to <= 0; raise `lower` or `cushion`")
    return table


def flat(table: Sequence[Triple]) -> List[float]:
    """The 3 x steps floats the C ABI takes (a_1, b_1, c_1, a_2, ...)."""
    return [float(v) for abc in table for v in abc]
