"""Plain fp64 CPU oracle for the Fast LapSum exact soft top-k operator.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The HIP library
never loads it, and it imports nothing from the HIP library: the two share no
code, only the seeded input generators (which hold none of the method's
arithmetic).

Source: "Fast LapSum: Exact Differentiable Top-k at Million Scale"
(gist.science summaries), section 2.1 (LapSum operator, eqs. (1)-(2), analytic
VJP) and section 2.2 (full-sort solver; probabilistic bracketing).

Contents
  forward / backward   -- C, fp64: b by bisection on the monotone budget
                          function (the definition of eq. (2) written out),
                          p = F((r - b)/t), and the analytic VJP.
  solve_sorted         -- C, fp64: the full-sort solver's own steps.
  budget, tail_sums    -- C, fp64 helpers (f(b); bracketing tail sums).
  bracket              -- numpy: counter-based sampling, binomial
                          order-statistic indices, the bracket itself.
  brute                -- mpmath: exhaustive solve for n <= 8.
  midpoint_mass        -- C, fp64: the DFTopK threshold (section 2.3) and the
                          mass the Laplace kernel assigns at it.

Every function here is pinned by ``tests/test_oracle_*.py`` against facts
that do not come from the oracle itself (closed forms, brute force,
symmetries, limits, finite differences, scipy's distributions).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lapsum_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liblapsum_oracle.so")
_lib = None


def build() -> str:
    """Compile the C oracle with gcc (plain -O2, no fast-math, OpenMP)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
           "-o", _LIB_PATH + ".tmp", _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    dp = ctypes.POINTER(ctypes.c_double)
    i64 = ctypes.c_int64
    lib.oracle_forward.argtypes = [dp, i64, i64, ctypes.c_double, ctypes.c_double, dp, dp, ctypes.c_int]
    lib.oracle_forward.restype = ctypes.c_int
    lib.oracle_backward.argtypes = [dp, dp, dp, i64, i64, ctypes.c_double, dp, dp, ctypes.c_int]
    lib.oracle_backward.restype = ctypes.c_int
    lib.oracle_solve_sorted.argtypes = [dp, i64, ctypes.c_double, ctypes.c_double, dp, ctypes.POINTER(i64)]
    lib.oracle_solve_sorted.restype = ctypes.c_int
    lib.oracle_budget.argtypes = [dp, i64, ctypes.c_double, ctypes.c_double, ctypes.c_int]
    lib.oracle_budget.restype = ctypes.c_double
    lib.oracle_tail_sums.argtypes = [dp, i64, ctypes.c_double, ctypes.c_double, ctypes.c_double,
                                     dp, dp, ctypes.POINTER(i64), ctypes.POINTER(i64), ctypes.POINTER(i64)]
    lib.oracle_tail_sums.restype = None
    lib.oracle_midpoint_mass.argtypes = [dp, i64, i64, i64, ctypes.c_double, dp, dp, ctypes.c_int]
    lib.oracle_midpoint_mass.restype = ctypes.c_int
    lib.oracle_laplace_cdf.argtypes = [ctypes.c_double]
    lib.oracle_laplace_cdf.restype = ctypes.c_double
    lib.oracle_laplace_quantile.argtypes = [ctypes.c_double]
    lib.oracle_laplace_quantile.restype = ctypes.c_double
    _lib = lib
    return lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def laplace_cdf(z: float) -> float:
    """Unit-scale Laplace CDF (section 2.1, eq. (1))."""
    return _load().oracle_laplace_cdf(float(z))


def laplace_quantile(u: float) -> float:
    return _load().oracle_laplace_quantile(float(u))


def forward(r, k: float, t: float, threads: int | None = None):
    """p, b for every row of r ([rows, n] or [n]); fp64 results.

    b is the unique root of sum_i F((r_i - b)/t) = k (eq. (2)), found by
    bisection; p_i = F((r_i - b)/t) (eq. (1))."""
    r64 = _f64(r)
    squeeze = r64.ndim == 1
    if squeeze:
        r64 = r64[None, :]
    rows, n = r64.shape
    p = np.empty_like(r64)
    b = np.empty(rows, dtype=np.float64)
    rc = _load().oracle_forward(_ptr(r64), rows, n, float(k), float(t), _ptr(p), _ptr(b),
                                threads or default_threads())
    if rc != 0:
        raise ValueError("oracle_forward: invalid arguments (need n >= 1, 0 < k < n, t > 0)")
    return (p[0], b[0]) if squeeze else (p, b)


def backward(r, b, g, t: float, threads: int | None = None):
    """Analytic VJP of the forward: returns dr (like r) and dk (per row)."""
    r64 = _f64(r)
    g64 = _f64(g)
    squeeze = r64.ndim == 1
    if squeeze:
        r64 = r64[None, :]
        g64 = g64[None, :]
    b64 = _f64(np.atleast_1d(b))
    rows, n = r64.shape
    dr = np.empty_like(r64)
    dk = np.empty(rows, dtype=np.float64)
    rc = _load().oracle_backward(_ptr(r64), _ptr(b64), _ptr(g64), rows, n, float(t), _ptr(dr), _ptr(dk),
                                 threads or default_threads())
    if rc != 0:
        raise ValueError("oracle_backward: invalid arguments")
    return (dr[0], dk[0]) if squeeze else (dr, dk)


def solve_sorted(r_row, k: float, t: float):
    """The full-sort solver's route to b for one row: returns (b, j), j the
    located knot index (-1 when b is below every score)."""
    r64 = _f64(r_row).ravel()
    b = ctypes.c_double()
    j = ctypes.c_int64()
    rc = _load().oracle_solve_sorted(_ptr(r64), r64.size, float(k), float(t), ctypes.byref(b), ctypes.byref(j))
    if rc != 0:
        raise ValueError("oracle_solve_sorted: invalid arguments")
    return b.value, j.value


def budget(r_row, b: float, t: float, threads: int = 1) -> float:
    """f(b) = sum_i F((r_i - b)/t)."""
    r64 = _f64(r_row).ravel()
    return _load().oracle_budget(_ptr(r64), r64.size, float(b), float(t), threads)


def tail_sums(r_row, a_lo: float, a_hi: float, t: float):
    """Bracketing step 2 for the bracket [a_lo, a_hi): returns a dict with
    S_L, S_R (tail sums shifted to the bracket ends), c_L, c_R and M."""
    r64 = _f64(r_row).ravel()
    sl, sr = ctypes.c_double(), ctypes.c_double()
    cl, cr, m = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    _load().oracle_tail_sums(_ptr(r64), r64.size, float(a_lo), float(a_hi), float(t),
                             ctypes.byref(sl), ctypes.byref(sr), ctypes.byref(cl), ctypes.byref(cr),
                             ctypes.byref(m))
    return {"S_L": sl.value, "S_R": sr.value, "c_L": cl.value, "c_R": cr.value, "M": m.value}


def midpoint_mass(r, k: int, t: float, threads: int | None = None):
    """Section 2.3 (relation to DFTopK): per row, the fixed threshold
    b_mid = (s_(k) + s_(k+1))/2 (k-th and (k+1)-th largest scores, k an
    integer in [1, n-1]) and mass = sum_i F((r_i - b_mid)/t).  Returns
    (b_mid, mass), one value per row (scalars for a 1-D row)."""
    r64 = _f64(r)
    squeeze = r64.ndim == 1
    if squeeze:
        r64 = r64[None, :]
    rows, n = r64.shape
    if int(k) != k:
        raise ValueError("midpoint_mass: k must be an integer")
    bm = np.empty(rows, dtype=np.float64)
    ms = np.empty(rows, dtype=np.float64)
    rc = _load().oracle_midpoint_mass(_ptr(r64), rows, n, int(k), float(t), _ptr(bm), _ptr(ms),
                                      threads or default_threads())
    if rc != 0:
        raise ValueError("oracle_midpoint_mass: invalid arguments (need 1 <= k <= n-1, t > 0)")
    return (bm[0], ms[0]) if squeeze else (bm, ms)
