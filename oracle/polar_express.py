"""Newton-Schulz coefficient table for Muon (test infrastructure only).

The nanochat article (dev.to, section "2. Muon Optimize Edici", and the same
section of its Arabic translation) names the five-step "Polar Express" table
but prints only its first two (a, b, c) tuples before an ellipsis.  The
remaining three are derived here by the principle the name refers to: each
step is the odd quintic p(x) = a x + b x^3 + c x^5 that minimises
max |1 - p(x)| over the interval the singular values occupy after the previous
steps, starting from [1e-3, 1] (singular values of a Frobenius-normalised
matrix lie in [0, 1]).  The minimax problem is solved as a linear programme
on a dense grid; the image interval is then evaluated on the same grid plus
the interval ends and the quintic's critical points.

This is a reading of a gap in the pages, not a reproduction of nanochat's
table; it is unpinned against that table.
"""
from __future__ import annotations

import numpy as np
from scipy.optimize import linprog

# the two tuples the article prints
PRINTED = [(8.156, -22.483, 15.879), (4.043, -2.809, 0.500)]


def quintic(x, abc):
    a, b, c = abc
    return a * x + b * x ** 3 + c * x ** 5


def image(lo, hi, abc, n=20001):
    """[min p, max p] over [lo, hi] (grid + exact critical points)."""
    xs = list(np.geomspace(lo, hi, n))
    a, b, c = abc
    # p'(x) = a + 3b x^2 + 5c x^4 = 0  ->  quadratic in y = x^2
    if c != 0:
        disc = 9 * b * b - 20 * a * c
        if disc >= 0:
            for sgn in (-1, 1):
                y = (-3 * b + sgn * np.sqrt(disc)) / (10 * c)
                if y > 0 and lo <= np.sqrt(y) <= hi:
                    xs.append(np.sqrt(y))
    v = quintic(np.asarray(xs), abc)
    return float(v.min()), float(v.max())


def minimax_step(lo, hi, n=4000):
    """(a, b, c) minimising max_{x in [lo,hi]} |1 - p(x)| (LP on a geometric grid)."""
    x = np.geomspace(lo, hi, n)
    Phi = np.stack([x, x ** 3, x ** 5], axis=1)
    # variables (a, b, c, t): minimise t  s.t.  -t <= 1 - Phi w <= t
    cost = np.array([0, 0, 0, 1.0])
    A = np.vstack([np.hstack([-Phi, -np.ones((n, 1))]),
                   np.hstack([Phi, -np.ones((n, 1))])])
    bvec = np.concatenate([-np.ones(n), np.ones(n)])
    res = linprog(cost, A_ub=A, b_ub=bvec, bounds=[(None, None)] * 3 + [(0, None)],
                  method="highs")
    if not res.success:
        raise RuntimeError(res.message)
    return tuple(float(v) for v in res.x[:3])


def coefficients(steps=5, lo=1e-3, hi=1.0):
    """Printed tuples first, minimax-derived tuples after; returns (table, intervals)."""
    table = []
    intervals = [(lo, hi)]
    for k in range(steps):
        if k < len(PRINTED):
            abc = PRINTED[k]
        else:
            abc = minimax_step(lo, hi)
        table.append(abc)
        lo, hi = image(lo, hi, abc)
        intervals.append((lo, hi))
    return table, intervals


if __name__ == "__main__":
    t, iv = coefficients()
    for abc, (l0, h0) in zip(t, iv[1:]):
        print("(%.6f, %.6f, %.6f) -> [%.4f, %.4f]" % (*abc, l0, h0))
