"""Pins of the oracle's forward (b and p) to facts that do not come from it.

Source: "Fast LapSum: Exact Differentiable Top-k at Million Scale",
section 2.1 (eq. (1): p_i = F((r_i - b)/t), F the Laplace CDF; eq. (2):
sum p_i = k fixes b uniquely), section 2.2 (full-sort solver), section 2.3
(DFTopK is LapSum's zero-temperature limit: the threshold sits at the
midpoint of the k-th and (k+1)-th order statistics).
"""
import math

import mpmath
import numpy as np
import pytest
import scipy.stats

from oracle import brute


def rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


# ---------------------------------------------------------------- F itself
def test_laplace_cdf_matches_scipy(oracle_mod):
    zs = np.concatenate([np.linspace(-40, 40, 2001), [-1e-300, 0.0, 1e-300, -700, 700]])
    for z in zs:
        assert oracle_mod.laplace_cdf(z) == pytest.approx(scipy.stats.laplace.cdf(z), rel=1e-14, abs=1e-300)
    for u in [1e-12, 1e-6, 0.01, 0.25, 0.5, 0.75, 0.99, 1 - 1e-9]:
        assert oracle_mod.laplace_quantile(u) == pytest.approx(scipy.stats.laplace.ppf(u), rel=1e-12, abs=1e-14)


# ------------------------------------------------------------ brute force
def _brute_cases():
    cases = []
    g = rng(7)
    for n in range(1, 9):
        ks = sorted({x for x in (0.5, 1.0, n / 2, n - 0.5) if 0 < x < n})
        for t in (1e-3, 0.1, 1.0, 10.0):
            for ties in (False, True):
                if ties and n < 2:
                    continue
                r = g.standard_normal(n).astype(np.float32)
                if ties:
                    r[: max(2, n // 2)] = r[0]
                for k in ks:
                    cases.append((r.copy(), float(k), t))
    return cases


@pytest.mark.parametrize("case", range(len(_brute_cases())))
def test_forward_matches_brute_force(oracle_mod, case):
    r, k, t = _brute_cases()[case]
    p, b = oracle_mod.forward(r, k, t, threads=1)
    b_ex, _ = brute.solve(r, k, t)
    with mpmath.workdps(50):
        # eq. (2) holds at the oracle's b to fp64 resolution
        resid = brute.budget(r, mpmath.mpf(b), t) - k
        assert abs(float(resid)) <= 1e-12 * len(r)
        # p agrees elementwise with p at the exact root
        for i, x in enumerate(r):
            z = (mpmath.mpf(float(x)) - b_ex) / t
            pe = mpmath.exp(z) / 2 if z < 0 else 1 - mpmath.exp(-z) / 2
            assert abs(p[i] - float(pe)) <= 1e-12
        # and b itself matches to fp64 resolution, flat budgets (tiny t) included
        assert abs(b - float(b_ex)) <= 1e-14 * max(abs(b), t)


# ------------------------------------------------------------ closed forms
@pytest.mark.parametrize("k", [1e-6, 0.1, 0.5, 0.9, 1 - 1e-6])
@pytest.mark.parametrize("t", [1e-3, 0.7, 50.0])
def test_single_element_closed_form(oracle_mod, k, t):
    r = np.array([0.375], np.float32)
    p, b = oracle_mod.forward(r, k, t, threads=1)
    assert p[0] == pytest.approx(k, rel=1e-12)
    assert b == pytest.approx(0.375 - t * scipy.stats.laplace.ppf(k), rel=1e-12, abs=1e-12 * t)


@pytest.mark.parametrize("n,k", [(2, 1.0), (7, 0.25), (256, 8), (1000, 999.5), (5000, 2500)])
def test_constant_row_closed_form(oracle_mod, n, k):
    c, t = -1.25, 0.05
    r = np.full(n, c, np.float32)
    p, b = oracle_mod.forward(r, k, t, threads=2)
    np.testing.assert_allclose(p, k / n, rtol=1e-12)
    assert b == pytest.approx(c - t * scipy.stats.laplace.ppf(k / n), rel=1e-13, abs=1e-13)


# -------------------------------------------------------------- symmetries
def _row(seed, n):
    return rng(seed).standard_normal(n).astype(np.float32)


def test_shift_equivariance(oracle_mod):
    r = _row(11, 300).astype(np.float64)
    _, b0 = oracle_mod.forward(r, 17.0, 0.2)
    p1, b1 = oracle_mod.forward(r + 3.5, 17.0, 0.2)
    p0, _ = oracle_mod.forward(r, 17.0, 0.2)
    assert b1 == pytest.approx(b0 + 3.5, abs=1e-12)
    np.testing.assert_allclose(p1, p0, atol=1e-12)


def test_scale_equivariance(oracle_mod):
    r = _row(12, 300).astype(np.float64)
    p0, b0 = oracle_mod.forward(r, 9.0, 0.1)
    p1, b1 = oracle_mod.forward(4.0 * r, 9.0, 0.4)
    assert b1 == pytest.approx(4.0 * b0, abs=1e-11)
    np.testing.assert_allclose(p1, p0, atol=1e-12)


def test_complement_symmetry(oracle_mod):
    r = _row(13, 257).astype(np.float64)
    n, k, t = 257, 40.0, 0.3
    p0, b0 = oracle_mod.forward(r, k, t)
    p1, b1 = oracle_mod.forward(-r, n - k, t)
    assert b1 == pytest.approx(-b0, abs=1e-12)
    np.testing.assert_allclose(p1, 1.0 - p0, atol=1e-12)


def test_permutation_equivariance_and_ties(oracle_mod):
    r = _row(14, 200)
    r[50:60] = r[3]                      # a block of exact ties
    perm = rng(15).permutation(200)
    p0, b0 = oracle_mod.forward(r, 12.0, 0.05)
    p1, b1 = oracle_mod.forward(r[perm], 12.0, 0.05)
    assert b1 == b0
    np.testing.assert_array_equal(p1, p0[perm])
    assert np.all(p0[50:60] == p0[3])


# ------------------------------------------------------------ budget
@pytest.mark.parametrize("seed,n,k,t", [(21, 1000, 32, 0.1), (22, 4096, 1, 0.01), (23, 513, 512.5, 1.0),
                                        (24, 20000, 3000, 0.003)])
def test_budget_holds(oracle_mod, seed, n, k, t):
    r = _row(seed, n)
    p, _ = oracle_mod.forward(r, k, t)
    assert math.fsum(p) == pytest.approx(k, abs=1e-12 * n)
    assert np.all((p >= 0) & (p <= 1))


# ---------------------------------------------------- zero-temperature limit
@pytest.mark.parametrize("seed", [31, 32, 33])
@pytest.mark.parametrize("k", [1, 5, 17])
@pytest.mark.parametrize("t", [1e-3, 1e-4])
def test_zero_temperature_limit_is_midpoint(oracle_mod, seed, k, t):
    """Section 2.3: as t -> 0 the threshold tends to the midpoint of the k-th
    and (k+1)-th largest scores and p tends to the hard top-k mask.  Near the
    limit b = mid + (t/2) ln(B/A), where A and B (between 1 and n) weigh the
    scores nearest above and below, so |b - mid| <= (t/2) ln n."""
    r = np.round(_row(seed, 50).astype(np.float64), 2)     # gaps >= 0.01 or exact ties
    n = r.size
    order = np.sort(r)[::-1]
    if order[k - 1] - order[k] < 0.02:
        pytest.skip("k-th and (k+1)-th scores too close for a clean limit")
    p, b = oracle_mod.forward(r, float(k), t)
    mid = 0.5 * (order[k - 1] + order[k])
    assert abs(b - mid) <= 0.5 * t * math.log(n) + 1e-12
    hard = (r >= order[k - 1]).astype(np.float64)
    np.testing.assert_allclose(p, hard, atol=1e-3)
    if t <= 1e-4:
        np.testing.assert_allclose(p, hard, atol=1e-20)


# -------------------------------------------------- full-sort solver route
@pytest.mark.parametrize("seed", range(40, 52))
def test_sorted_solver_matches_bisection(oracle_mod, seed):
    g = rng(seed)
    n = int(g.integers(1, 3000))
    k = float(g.uniform(0.01, n - 0.01)) if g.random() < 0.5 else float(g.integers(1, n)) if n > 1 else 0.5
    t = float(10 ** g.uniform(-3, 1))
    r = g.standard_normal(n).astype(np.float32)
    if g.random() < 0.5 and n > 4:
        r[g.integers(0, n, n // 3)] = r[0]     # ties, some at the threshold
    p, b = oracle_mod.forward(r, k, t)
    bs, j = oracle_mod.solve_sorted(r, k, t)
    d = np.exp(-np.abs(r.astype(np.float64) - b) / t).sum() / 2
    assert abs(bs - b) <= 1e-9 * t / max(d, 1e-300) + 1e-14 * (1 + abs(b))
    s = np.sort(r.astype(np.float64))
    if j < 0:
        assert bs <= s[0]
    elif j == n - 1:
        assert bs >= s[-1]
    else:
        assert s[j] <= bs <= s[j + 1]


def test_sorted_solver_end_cases(oracle_mod):
    r = np.array([0.0, 0.01, 0.02], np.float32)
    # k close to n: b well below every score (left end)
    b, j = oracle_mod.solve_sorted(r, 2.999, 0.5)
    assert j == -1 and b < 0.0
    _, bb = oracle_mod.forward(r, 2.999, 0.5)
    assert b == pytest.approx(bb, abs=1e-12)
    # k close to 0: b above every score (right end)
    b, j = oracle_mod.solve_sorted(r, 0.001, 0.5)
    assert j == 2 and b > 0.02
    _, bb = oracle_mod.forward(r, 0.001, 0.5)
    assert b == pytest.approx(bb, abs=1e-12)


def test_invalid_arguments_raise(oracle_mod):
    r = np.zeros(4, np.float32)
    for k, t in [(0.0, 1.0), (4.0, 1.0), (-1.0, 1.0), (1.0, 0.0), (1.0, -1.0)]:
        with pytest.raises(ValueError):
            oracle_mod.forward(r, k, t)


def test_forward_matches_golden_brute_fixtures(oracle_mod):
    """tests/golden/brute_small.json: 50-digit exhaustive solutions (no sort,
    scan or bisection) for rows of n <= 8."""
    import json
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "brute_small.json")
    with open(path) as f:
        cases = json.load(f)["cases"]
    assert len(cases) > 200
    for c in cases:
        r = np.array(c["r"], np.float32)
        _, b = oracle_mod.forward(r, c["k"], c["t"], threads=1)
        be = float(mpmath.mpf(c["b"]))
        assert abs(b - be) <= 1e-14 * max(abs(be), c["t"]), c
