"""Exhaustive high-precision solve of eq. (2) for tiny rows (n <= 8).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "Fast LapSum: Exact Differentiable Top-k at Million Scale", section
2.1: p_i = F((r_i - b)/t) with F the Laplace CDF, and sum_i p_i = k.

Method (independent of sorting, scanning and of the oracle's bisection): for
every subset U of indices taken to lie at or above b, the budget is
    sum_{i not in U} exp((r_i - b)/t)/2 + sum_{i in U} (1 - exp(-(r_i - b)/t)/2) = k.
With y = exp(b/t), P = sum_{i not in U} exp(r_i/t) and Q = sum_{i in U} exp(-r_i/t)
this is the quadratic Q y^2 - 2(|U| - k) y - P = 0.  Its positive root is the
threshold if the resulting b is consistent with U (r_i >= b on U, r_i <= b off
it).  All arithmetic is mpmath at 50 significant digits.
"""
from __future__ import annotations

import itertools

import mpmath


def solve(r, k, t, dps: int = 50):
    """Return b (mpmath mpf) for the row r (n <= 8)."""
    n = len(r)
    if n > 8:
        raise ValueError("brute force is for n <= 8")
    with mpmath.workdps(dps):
        rr = [mpmath.mpf(float(x)) for x in r]
        kk = mpmath.mpf(k)
        tt = mpmath.mpf(t)
        found = []
        for size in range(n + 1):
            for U in itertools.combinations(range(n), size):
                Us = set(U)
                P = mpmath.fsum(mpmath.exp(rr[i] / tt) for i in range(n) if i not in Us)
                Q = mpmath.fsum(mpmath.exp(-rr[i] / tt) for i in Us)
                e = mpmath.mpf(len(Us)) - kk
                if Q == 0:
                    if e >= 0:
                        continue
                    y = P / (-2 * e)
                elif P == 0:
                    if e <= 0:
                        continue
                    y = 2 * e / Q
                elif e >= 0:
                    y = (e + mpmath.sqrt(e * e + P * Q)) / Q
                else:
                    # same root, written without the cancellation of e + sqrt(.)
                    y = P / (mpmath.sqrt(e * e + P * Q) - e)
                if y <= 0:
                    continue
                b = tt * mpmath.log(y)
                tol = mpmath.mpf(10) ** (-(dps - 10)) * (1 + abs(b))
                ok = all(rr[i] >= b - tol for i in Us) and all(rr[i] <= b + tol for i in range(n) if i not in Us)
                if ok:
                    found.append(b)
        if not found:
            raise RuntimeError("no consistent root found")
        # every consistent subset yields the same root (f is continuous)
        return found[0], found


def budget(r, b, t, dps: int = 50):
    """f(b) in mpmath precision."""
    with mpmath.workdps(dps):
        tot = mpmath.mpf(0)
        for x in r:
            z = (mpmath.mpf(float(x)) - b) / mpmath.mpf(t)
            tot += mpmath.exp(z) / 2 if z < 0 else 1 - mpmath.exp(-z) / 2
        return tot
