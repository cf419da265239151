"""CPU oracle of the per-step Newton-Schulz coefficient schedule.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or runs
this module: only ``tests/`` may.  It shares no code with the library and
imports nothing from the ``matrix_optimizer_amd`` package.

Source.  The DMuon-2 page (App. C.3) runs Newton-Schulz with per-step
coefficients from the Polar Express method (Amsel et al., 2025, cited there);
the HyperParallel-FSDP evaluation names an "asym5" set.  Neither page prints
the values.  This oracle follows the greedy construction of that method:

* every singular value of X_0 lies in [l_0, u_0] = [lower, 1] (Frobenius
  normalisation leaves none above 1; ``lower`` is an assumed bound);
* an odd polynomial p of X maps each singular value s to p(s), so step k
  takes the odd quintic p_k(x) = a x + b x^3 + c x^5 closest to 1 in the
  uniform norm on [l_k, u_k], and [l_{k+1}, u_{k+1}] is p_k's range there.

The best approximation is its definition written out: a linear program over
(a, b, c, E) that minimises E subject to |1 - p(x)| <= E at every point of a
fine grid of the interval (scipy's linprog is the library step), followed by
the same program on a grid refined around the points where the first
solution's error peaks.

Readings (the pages are silent on all of them):

* ``safety`` s >= 1: the step uses p(x / s), i.e. (a/s, b/s^3, c/s^5).
* ``cushion``: the design interval is [max(l, cushion u, 1e-4 u), u]; the
  1e-4 floor keeps the levelled minimum 1 - E well above the float rounding
  of the coefficients.  The next interval is still the range over [l, u].
* The coefficients are rounded to float32 (the precision the step takes them
  in) before the next interval is computed.
* When the design interval is shorter than 1e-3 u the problem degenerates and
  the step takes its limit, the quintic with p(m) = 1, p'(m) = p''(m) = 0 at
  the midpoint m.

Parity status: pinned by tests/test_schedule.py against the Chebyshev
alternation theorem (four alternation points with equal error), brute-force
optimality under random perturbations, the classical quintic
x (15 - 10 x^2 + 3 x^4) / 8 as the short-interval limit, and dense-grid
evaluation of the composed polynomials.
"""
from __future__ import annotations

import numpy as np
from scipy.optimize import linprog

FLOOR = 1e-4
SHORT = 1e-3


def poly(coeffs, x):
    """p(x) = a x + b x^3 + c x^5."""
    a, b, c = (float(v) for v in coeffs)
    return a * x + b * x ** 3 + c * x ** 5


def critical_points(coeffs, lo, hi):
    """Real x in (lo, hi) with p'(x) = a + 3 b x^2 + 5 c x^4 = 0."""
    a, b, c = (float(v) for v in coeffs)
    roots = np.roots([5 * c, 0.0, 3 * b, 0.0, a]) if c != 0 else np.roots([3 * b, 0.0, a])
    xs = [r.real for r in roots if abs(r.imag) <= 1e-12 * max(1.0, abs(r.real))]
    return sorted(x for x in xs if lo < x < hi)


def range_on(coeffs, lo, hi):
    """(min, max) of p over [lo, hi]: endpoints and interior critical points."""
    vals = [poly(coeffs, lo), poly(coeffs, hi)] + [poly(coeffs, x) for x in critical_points(coeffs, lo, hi)]
    return min(vals), max(vals)


def _lp(xs):
    """min E s.t. -E <= 1 - p(x) <= E on the points xs; returns (a, b, c), E."""
    V = np.stack([xs, xs ** 3, xs ** 5], axis=1)
    one = np.ones((len(xs), 1))
    A = np.vstack([np.hstack([-V, -one]), np.hstack([V, -one])])
    rhs = np.concatenate([-np.ones(len(xs)), np.ones(len(xs))])
    res = linprog([0, 0, 0, 1], A_ub=A, b_ub=rhs, bounds=[(None, None)] * 4, method="highs")
    if res.status != 0:
        raise RuntimeError(f"linprog: {res.message}")
    return tuple(res.x[:3]), res.x[3]


def best_quintic(lo, hi, n=4001):
    """The odd quintic closest to 1 in the uniform norm on [lo, hi]."""
    xs = np.unique(np.concatenate([np.linspace(lo, hi, n), np.geomspace(lo, hi, n)]))
    coeffs, _ = _lp(xs)
    # refine around the extremal points of the first solution's error
    ext = [lo, hi] + critical_points(coeffs, lo, hi)
    h = (hi - lo) / (n - 1)
    fine = [np.linspace(max(lo, x - 2 * h), min(hi, x + 2 * h), 801) for x in ext]
    xs2 = np.unique(np.concatenate([xs] + fine))
    return _lp(xs2)


def limit_quintic(m):
    """p(m) = 1, p'(m) = 0, p''(m) = 0, solved as a 3 x 3 linear system."""
    A = np.array([[m, m ** 3, m ** 5],
                  [1.0, 3 * m ** 2, 5 * m ** 4],
                  [0.0, 6 * m, 20 * m ** 3]])
    return tuple(np.linalg.solve(A, [1.0, 0.0, 0.0]))


def schedule(steps, lower=1e-3, safety=1.0, cushion=0.0):
    """Greedy per-step coefficients: a list of float32 (a, b, c) triples and the
    list of (l_{k+1}, u_{k+1}) intervals after each step."""
    lo, hi = float(lower), 1.0
    coeffs, bounds = [], []
    for _ in range(steps):
        dlo = max(lo, cushion * hi, FLOOR * hi)
        if hi - dlo <= SHORT * hi:
            p = limit_quintic(0.5 * (dlo + hi))
        else:
            p, _ = best_quintic(dlo, hi)
        a, b, c = p
        f = tuple(np.float32(v) for v in (a / safety, b / safety ** 3, c / safety ** 5))
        lo, hi = range_on(f, lo, hi)
        coeffs.append(f)
        bounds.append((lo, hi))
    return coeffs, bounds
