"""Pins of oracle.midpoint_mass: the DFTopK threshold and the mass the
Laplace kernel assigns at it ("Fast LapSum: Exact Differentiable Top-k at
Million Scale", section 2.3: DFTopK fixes the threshold at the midpoint of
the k-th and (k+1)-th largest scores, and is LapSum's zero-temperature
limit; section 4.1 reports the budget error this causes).

Each check comes from outside the oracle: a closed form on equally spaced
scores, brute-force order statistics by rank counting, the zero-temperature
limit, the monotone link to the LapSum threshold, and symmetries.
"""
import math

import numpy as np
import pytest

import oracle


def closed_form_mass(n, k, h, t):
    """Scores r_i = i h, i = 0..n-1: b_mid = (n - k - 1/2) h, and with
    a = h/t the Laplace-CDF terms are two geometric series,
        mass = k + e^{-a/2} (e^{-k a} - e^{-(n-k) a}) / (2 (1 - e^{-a}))."""
    a = h / t
    return (n - k - 0.5) * h, k + math.exp(-a / 2) * (math.exp(-k * a) - math.exp(-(n - k) * a)) / (2 * (1 - math.exp(-a)))


@pytest.mark.parametrize("n,k,h,t", [(10, 3, 0.5, 0.1), (10, 3, 0.5, 2.0), (257, 1, 0.01, 0.05), (257, 256, 0.01, 0.05),
                                     (1000, 500, 0.001, 0.01), (1000, 17, 0.3, 0.25), (64, 40, 1.0, 5.0)])
def test_equally_spaced_closed_form(n, k, h, t):
    r = np.arange(n, dtype=np.float64) * h
    bm, m = oracle.midpoint_mass(r, k, t)
    bcf, mcf = closed_form_mass(n, k, h, t)
    assert abs(bm - bcf) <= 1e-12 * max(1.0, abs(bcf))
    assert abs(m - mcf) <= 1e-11 * max(1.0, mcf)
    # the permutation of the same scores changes nothing
    perm = np.random.Generator(np.random.PCG64(n + k)).permutation(n)
    bm2, m2 = oracle.midpoint_mass(r[perm], k, t)
    assert bm2 == bm and abs(m2 - m) <= 1e-12 * max(1.0, m)


def brute(r, k, t):
    """Order statistics by counting ranks (no sort): x is the j-th largest
    when fewer than j scores exceed it and at least j are >= it."""
    def kth_largest(j):
        for x in r:
            gt = sum(1 for y in r if y > x)
            ge = sum(1 for y in r if y >= x)
            if gt < j <= ge:
                return x
        raise AssertionError
    bm = 0.5 * (kth_largest(k) + kth_largest(k + 1))
    m = math.fsum(0.5 * math.exp((x - bm) / t) if x < bm else 1 - 0.5 * math.exp(-(x - bm) / t) for x in r)
    return bm, m


@pytest.mark.parametrize("seed", range(12))
def test_brute_force_small_rows(seed):
    g = np.random.Generator(np.random.PCG64(600 + seed))
    n = int(g.integers(2, 9))
    r = g.standard_normal(n).round(1 if seed % 3 == 0 else 6)  # rounding makes ties
    k = int(g.integers(1, n))
    t = float(g.choice([1e-3, 0.1, 1.0, 10.0]))
    bm, m = oracle.midpoint_mass(r, k, t)
    bb, mb = brute(list(r), k, t)
    assert bm == bb
    assert abs(m - mb) <= 1e-12 * max(1.0, mb)


def test_ties_at_the_midpoint():
    """When the k-th and (k+1)-th largest are equal, b_mid is that value and
    every score equal to it gets p = 1/2."""
    r = np.array([0.1, 2.0, 0.7, 0.7, 0.7, -1.0])
    bm, m = oracle.midpoint_mass(r, 2, 1e-4)
    assert bm == 0.7
    assert abs(m - (1.0 + 3 * 0.5)) <= 1e-12  # 2.0 -> 1, the three 0.7 -> 1/2, the rest -> 0


def test_zero_temperature_limit_gives_k():
    """As t -> 0 every score above the midpoint tends to p = 1 and every one
    below to 0, so the mass tends to exactly k (section 2.3)."""
    g = np.random.Generator(np.random.PCG64(611))
    r = g.standard_normal((4, 500))
    for k in (1, 37, 250, 499):
        _, m = oracle.midpoint_mass(r, k, 1e-7)
        assert np.all(np.abs(m - k) <= 1e-9)


def test_mass_sign_matches_the_lapsum_threshold():
    """f(b) = sum F((r - b)/t) is strictly decreasing and equals k at the
    LapSum threshold, so mass > k exactly when b_mid lies below it."""
    g = np.random.Generator(np.random.PCG64(612))
    for trial in range(20):
        n = int(g.integers(20, 400))
        r = np.abs(g.standard_normal(n)) ** 1.5
        k = int(g.integers(1, n))
        t = float(g.choice([0.01, 0.1, 0.5]))
        bm, m = oracle.midpoint_mass(r, k, t)
        _, b = oracle.forward(r, float(k), t)
        if abs(bm - b) > 1e-9 * t:
            assert (m > k) == (bm < b), (trial, bm, b, m, k)


def test_shift_and_scale():
    g = np.random.Generator(np.random.PCG64(613))
    r = g.standard_normal((3, 300))
    bm, m = oracle.midpoint_mass(r, 20, 0.05)
    bm2, m2 = oracle.midpoint_mass(r + 3.0, 20, 0.05)
    assert np.allclose(bm2, bm + 3.0, atol=1e-12) and np.allclose(m2, m, rtol=1e-12)
    bm3, m3 = oracle.midpoint_mass(4.0 * r, 20, 0.2)
    assert np.allclose(bm3, 4.0 * bm, atol=1e-12) and np.allclose(m3, m, rtol=1e-12)


def test_rejects_non_integer_and_out_of_range_k():
    r = np.arange(5.0)
    for k in (0, 5, 2.5):
        with pytest.raises(ValueError):
            oracle.midpoint_mass(r, k, 0.1)
