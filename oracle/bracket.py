"""Oracle side of the probabilistic-bracketing localisation step.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "Fast LapSum: Exact Differentiable Top-k at Million Scale", section
2.2, "Probabilistic Bracketing", step 1 (localisation): draw a small sample of
kernel-noised scores and use binomial order statistics to find a narrow
bracket [a_L, a_R) that holds the true threshold b with high probability.

Readings taken where the pages are silent:
  * "kernel-noised" = an index drawn uniformly with replacement plus
    Laplace(0, t) noise: X = r_I + t L.  Then P(X <= x) = 1 - f(x)/n, so b is
    exactly the (1 - k/n)-quantile of X and #{X_j <= b} ~ Bin(m, 1 - k/n).
  * lo and hi are equal-tailed at delta/2 each; lo = 0 means a_L = -inf and
    hi = m + 1 means a_R = +inf.
  * the random numbers come from Philox-4x32-10 (Salmon, Moraes, Dror, Shaw,
    "Parallel random numbers: as easy as 1, 2, 3", SC'11), implemented here
    from that published definition: key = (seed low 32 bits, seed high 32
    bits), counter = (sample index j, row, 0, 0).  Output words x0, x1 give
    the index I = floor((x1 * 2^32 + x0) * n / 2^64); x2 gives
    u = (x2 + 1/2) / 2^32 and L = F^-1(u) (unit Laplace quantile, fp64).
    X is rounded to fp32.
"""
from __future__ import annotations

import math

import numpy as np

PHILOX_M0 = np.uint64(0xD2511F53)
PHILOX_M1 = np.uint64(0xCD9E8D57)
PHILOX_W0 = np.uint64(0x9E3779B9)
PHILOX_W1 = np.uint64(0xBB67AE85)
_MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(c0, c1, c2, c3, k0: int, k1: int):
    """Philox-4x32 with 10 rounds on arrays of counters (uint32 values held
    in uint64 arrays).  Each round: two 32x32->64 products of the multipliers
    with counter words 0 and 2; the new counter is
    (hi(M1*c2) ^ c1 ^ k0, lo(M1*c2), hi(M0*c0) ^ c3 ^ k1, lo(M0*c0)); the key
    is bumped by the Weyl constants between rounds."""
    c0 = np.asarray(c0, dtype=np.uint64) & _MASK32
    c1 = np.asarray(c1, dtype=np.uint64) & _MASK32
    c2 = np.asarray(c2, dtype=np.uint64) & _MASK32
    c3 = np.asarray(c3, dtype=np.uint64) & _MASK32
    key0 = np.uint64(k0 & 0xFFFFFFFF)
    key1 = np.uint64(k1 & 0xFFFFFFFF)
    for rnd in range(10):
        if rnd > 0:
            key0 = (key0 + PHILOX_W0) & _MASK32
            key1 = (key1 + PHILOX_W1) & _MASK32
        p0 = PHILOX_M0 * c0
        p1 = PHILOX_M1 * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK32
        c0, c1, c2, c3 = (hi1 ^ c1 ^ key0), lo1, (hi0 ^ c3 ^ key1), lo0
    return c0, c1, c2, c3


def _binom_log_pmf(m: int, q: float) -> np.ndarray:
    j = np.arange(m + 1, dtype=np.float64)
    lg = np.array([math.lgamma(x + 1.0) for x in range(m + 1)])
    lq = math.log(q) if q > 0 else -math.inf
    l1q = math.log1p(-q) if q < 1 else -math.inf
    with np.errstate(invalid="ignore"):
        out = lg[m] - lg - lg[::-1] + j * lq + (m - j) * l1q
    if q == 0:
        out = np.where(j == 0, 0.0, -np.inf)
    if q == 1:
        out = np.where(j == m, 0.0, -np.inf)
    return out


def binomial_bracket(n: int, k: float, m: int, delta: float):
    """Equal-tailed order-statistic indices (lo, hi), 1-based, for a sample of
    m draws with N = #{X <= b} ~ Bin(m, q), q = 1 - k/n:
        lo = max{l in [0, m]   : P(N <= l - 1) <= delta/2}
        hi = min{h in [1, m+1] : P(N <= h - 1) >= 1 - delta/2}
    so P(X_(lo) > b) <= delta/2 and P(X_(hi) <= b) <= delta/2.
    Both tails are summed directly from the pmf (no 1 - CDF cancellation)."""
    q = 1.0 - float(k) / float(n)
    pmf = np.exp(_binom_log_pmf(m, q))
    lower = np.cumsum(pmf)                 # lower[x] = P(N <= x)
    upper = np.cumsum(pmf[::-1])[::-1]     # upper[x] = P(N >= x)
    half = 0.5 * delta
    lo = 0
    for l in range(1, m + 1):
        if lower[l - 1] <= half:
            lo = l
        else:
            break
    hi = m + 1
    for h in range(m, 0, -1):
        # P(N <= h-1) >= 1 - half  <=>  P(N >= h) <= half
        if upper[h] <= half:
            hi = h
        else:
            break
    return lo, hi


def default_sample_log2(n: int) -> int:
    """m = min(2^16, 2^floor(log2(n/16))), at least 2^4."""
    if n < 256:
        return 4
    return int(min(16, max(4, math.floor(math.log2(n / 16.0)))))


def sample(r_row, t: float, m: int, seed: int, row: int = 0) -> np.ndarray:
    """The m kernel-noised sample values X_j = fp32(r_I + t L) of one row."""
    r = np.asarray(r_row)
    n = r.size
    j = np.arange(m, dtype=np.uint64)
    x0, x1, x2, _ = philox4x32_10(j, np.full(m, row, dtype=np.uint64), np.zeros(m, np.uint64),
                                  np.zeros(m, np.uint64), seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)
    nn = np.uint64(n)
    idx = (x1 * nn + ((x0 * nn) >> np.uint64(32))) >> np.uint64(32)
    u = (x2.astype(np.float64) + 0.5) * 2.0 ** -32
    lap = np.where(u < 0.5, np.log(2.0 * u), -np.log(2.0 * (1.0 - u)))
    x = r.astype(np.float64)[idx.astype(np.int64)] + float(t) * lap
    return x.astype(np.float32)


def bracket(r_row, k: float, t: float, m: int, delta: float, seed: int, row: int = 0):
    """(a_L, a_R) = (X_(lo), X_(hi)) as fp64 values, +-inf at missing ends."""
    n = np.asarray(r_row).size
    lo, hi = binomial_bracket(n, k, m, delta)
    xs = np.sort(sample(r_row, t, m, seed, row))
    a_lo = -math.inf if lo < 1 else float(xs[lo - 1])
    a_hi = math.inf if hi > m else float(xs[hi - 1])
    return a_lo, a_hi, lo, hi
