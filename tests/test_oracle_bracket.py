"""Pins of the oracle's probabilistic-bracketing pieces.

Source: "Fast LapSum: Exact Differentiable Top-k at Million Scale",
section 2.2, "Probabilistic Bracketing": step 1 draws a small sample of
kernel-noised scores and takes binomial order statistics as a bracket
[a_L, a_R) holding b with high probability; step 2 folds the scores outside
the bracket into tail sums through Laplace-CDF identities.
"""
import math

import numpy as np
import pytest
import scipy.stats

from oracle import bracket as ob


def rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


# ------------------------------------------------ binomial order statistics
@pytest.mark.parametrize("n,k,m,delta", [
    (100_000_000, 1e5, 65536, 1e-6),       # extreme single row
    (3_317_760, 600, 65536, 1e-6),         # attack-shaped row
    (65536, 3277, 4096, 1e-6),             # coder-shaped rows
    (2000, 100, 256, 0.2),
    (1000, 999, 64, 0.01),
    (1000, 1, 64, 0.01),
])
def test_binomial_indices_against_scipy(n, k, m, delta):
    lo, hi = ob.binomial_bracket(n, k, m, delta)
    q = 1.0 - k / n
    N = scipy.stats.binom(m, q)
    half = delta / 2
    # lo: largest l with P(N <= l-1) <= delta/2
    if lo >= 1:
        assert N.cdf(lo - 1) <= half * (1 + 1e-9)
    if lo < m:
        assert N.cdf(lo) > half * (1 - 1e-9)
    # hi: smallest h with P(N >= h) <= delta/2
    if hi <= m:
        assert N.sf(hi - 1) <= half * (1 + 1e-9)
    if hi >= 2:
        assert N.sf(hi - 2) > half * (1 - 1e-9)
    assert 0 <= lo < hi <= m + 1


def test_binomial_indices_of_the_workloads():
    # the values the bracketing configurations run with (m, delta as read)
    assert ob.binomial_bracket(100_000_000, 1e5, 65536, 1e-6) == (65427, 65507)
    lo, hi = ob.binomial_bracket(3_317_760, 600, 65536, 1e-6)
    assert hi == 65537 and lo == 65504
    assert ob.binomial_bracket(65536, 3277, 4096, 1e-6) == (3820, 3957)


# ------------------------------------------------------------------ Philox
def test_philox_words_are_uniform_and_streams_differ():
    m = 1 << 16
    j = np.arange(m, dtype=np.uint64)
    z = np.zeros(m, np.uint64)
    words = ob.philox4x32_10(j, z, z, z, 12345, 678)
    for w in words:
        counts = np.bincount((w >> np.uint64(24)).astype(np.int64), minlength=256)
        chi2 = ((counts - m / 256) ** 2 / (m / 256)).sum()
        assert scipy.stats.chi2.sf(chi2, 255) > 1e-4
        assert np.unique(w).size > m - 5          # 32-bit words: collisions are rare
    other = ob.philox4x32_10(j, z + np.uint64(1), z, z, 12345, 678)[0]
    assert np.mean(other == words[0]) < 1e-3
    other_key = ob.philox4x32_10(j, z, z, z, 12346, 678)[0]
    assert np.mean(other_key == words[0]) < 1e-3
    # adjacent counters are not correlated
    a = words[0].astype(np.float64)
    assert abs(np.corrcoef(a[:-1], a[1:])[0, 1]) < 0.02


def test_sample_indices_uniform_and_noise_is_laplace():
    n = 1000
    r = np.zeros(n, np.float32)
    m = 1 << 16
    x = ob.sample(r, 1.0, m, seed=99)
    # r = 0: X is pure Laplace(0, 1) noise rounded to fp32
    assert scipy.stats.kstest(x.astype(np.float64), scipy.stats.laplace.cdf).pvalue > 1e-4
    # index uniformity: tag each score with its index
    r2 = np.arange(n, dtype=np.float32)
    xi = ob.sample(r2, 1e-30, m, seed=99)
    idx = np.rint(xi).astype(np.int64)
    counts = np.bincount(idx, minlength=n)
    chi2 = ((counts - m / n) ** 2 / (m / n)).sum()
    assert scipy.stats.chi2.sf(chi2, n - 1) > 1e-4


def test_bracket_coverage_by_simulation(oracle_mod):
    """At delta = 0.2 the bracket misses b with probability <= 0.2 (<= 0.1
    per side); 2000 independent seeds must agree within a binomial CI.  This
    also checks that the noised sample really follows 1 - f(x)/n."""
    g = rng(5)
    n, k, t, m, delta = 2000, 100.0, 0.1, 256, 0.2
    r = g.standard_normal(n).astype(np.float32)
    _, b = oracle_mod.forward(r, k, t)
    lo, hi = ob.binomial_bracket(n, k, m, delta)
    miss_lo = miss_hi = 0
    trials = 2000
    for s in range(trials):
        xs = np.sort(ob.sample(r, t, m, seed=1000 + s))
        if lo >= 1 and xs[lo - 1] > b:
            miss_lo += 1
        if hi <= m and xs[hi - 1] <= b:
            miss_hi += 1
    q = scipy.stats.binom(m, 1 - k / n)
    p_lo = q.cdf(lo - 1)              # exact miss probabilities of the design
    p_hi = q.sf(hi - 1)
    for miss, pe in ((miss_lo, p_lo), (miss_hi, p_hi)):
        lo_ci, hi_ci = scipy.stats.binom(trials, pe).ppf([1e-4, 1 - 1e-4])
        assert lo_ci <= miss <= hi_ci, (miss, pe * trials)


# ------------------------------------------------------------- tail sums
@pytest.mark.parametrize("seed", [81, 82, 83])
def test_tail_sum_identity(oracle_mod, seed):
    """For b inside [a_L, a_R):
       f(b) = S_L e^{(a_L-b)/t}/2 + sum_band F((u-b)/t) + c_R - S_R e^{(b-a_R)/t}/2."""
    g = rng(seed)
    n, k, t = 5000, 150.0, 0.05
    r = g.standard_normal(n).astype(np.float32)
    _, b = oracle_mod.forward(r, k, t)
    for a_lo, a_hi in ((b - 0.1, b + 0.07), (b - 1e-3, math.inf), (-math.inf, b + 0.2), (b, b + 1e-9)):
        ts = oracle_mod.tail_sums(r, a_lo, a_hi, t)
        r64 = r.astype(np.float64)
        band = r64[(r64 >= a_lo) & (r64 < a_hi)]
        assert ts["M"] == band.size
        assert ts["c_L"] + ts["c_R"] + ts["M"] == n
        assert ts["c_L"] == np.sum(r64 < a_lo) and ts["c_R"] == np.sum(r64 >= a_hi)
        z = (band - b) / t
        fband = np.where(z < 0, 0.5 * np.exp(np.minimum(z, 0)), 1 - 0.5 * np.exp(-np.maximum(z, 0))).sum()
        left = 0.5 * ts["S_L"] * math.exp((a_lo - b) / t) if ts["c_L"] else 0.0
        right = 0.5 * ts["S_R"] * math.exp((b - a_hi) / t) if ts["c_R"] else 0.0
        total = left + fband + ts["c_R"] - right
        assert total == pytest.approx(oracle_mod.budget(r, b, t), abs=1e-9 * n)
        assert total == pytest.approx(k, abs=1e-9 * n)
