"""Comparison helpers for the GPU parity tests (tolerances of the operator's
accuracy bar, written out here):

  max|p_gpu - p_oracle|            <= 2e-5
  |sum p_gpu - k|                  <= 1e-5 max(1, k)      (per row, fp64 sum)
  |b_gpu - b_oracle| / t           <= 1e-4
  ||dr_gpu - dr_oracle|| / ||dr_oracle||            <= 1e-4 (per row)
  |dk_gpu - dk_oracle| / sum_i (d_i/D)|g_i|         <= 1e-4 (dk is the
                                     d-weighted mean of g; that is its scale)
  each gradient bound replaced by the resolution floor of fp32
  probabilities only where that floor is larger (see check_backward)

The budget bound follows the pages' reported normalisation error (< 1e-5 at
all scales, "Fast LapSum: Exact Differentiable Top-k at Million Scale",
section 4.1).
"""
import math
import sys

import numpy as np

TOL_P = 2e-5
TOL_SUM = 1e-5
TOL_B = 1e-4
TOL_GRAD = 1e-4


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def check_forward(name, k, t, p_gpu, b_gpu, p_or, b_or, rows_idx=None):
    p_gpu = np.asarray(p_gpu, dtype=np.float64)
    p_or = np.asarray(p_or, dtype=np.float64)
    b_gpu = np.atleast_1d(np.asarray(b_gpu, dtype=np.float64))
    b_or = np.atleast_1d(np.asarray(b_or, dtype=np.float64))
    dp = float(np.max(np.abs(p_gpu - p_or))) if p_gpu.size else 0.0
    db = float(np.max(np.abs(b_gpu - b_or))) / t
    assert np.all(np.isfinite(p_gpu)) and np.all(np.isfinite(b_gpu)), name
    assert dp <= TOL_P, f"{name}: max|dp| = {dp:.3e}"
    assert db <= TOL_B, f"{name}: max|db|/t = {db:.3e}"
    return dp, db


def check_budget(name, k, p_gpu):
    p = np.asarray(p_gpu, dtype=np.float64)
    if p.ndim == 1:
        p = p[None, :]
    sums = np.array([math.fsum(row) for row in p])
    err = float(np.max(np.abs(sums - k)))
    assert err <= TOL_SUM * max(1.0, k), f"{name}: |sum p - k| = {err:.3e}"
    return err


def check_backward(name, r, b_or, g, t, dr_gpu, dk_gpu, dr_or, dk_or):
    """Per row, the plain gradient bounds
        ||dr_gpu - dr_or|| <= 1e-4 ||dr_or||,   |dk_gpu - dk_or| <= 1e-4 scale_dk,
    unless the resolution of fp32 probabilities alone exceeds them.  The
    backward receives p in fp32, and for p > 1/2 the value 1 - p is known only
    to 2^-25 absolutely, so d = min(p, 1 - p)/t carries up to 2^-25/t
    (taken as 2^-24/t) of absolute error that no kernel can remove; dr and dk
    inherit it as floor_dr = 2^-24/t ||g - dk||_{p>1/2} and
    floor_dk = 2^-24/t sum_{p>1/2} |g - dk| / D.  The bound used is
    max(plain bound, floor), never their sum: where the floor is below the
    plain bound the check is exactly the plain one.
    Returns the worst plain relative errors (err / ||dr_or||, err / scale_dk);
    check_backward.last holds the worst floor / plain-bound ratios and the
    number of rows whose bound the floor decided."""
    r = np.asarray(r, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    if r.ndim == 1:
        r, g = r[None, :], g[None, :]
    dr_gpu = np.asarray(dr_gpu, dtype=np.float64).reshape(r.shape)
    dr_or = np.asarray(dr_or, dtype=np.float64).reshape(r.shape)
    dk_gpu = np.atleast_1d(np.asarray(dk_gpu, dtype=np.float64))
    dk_or = np.atleast_1d(np.asarray(dk_or, dtype=np.float64))
    u = 2.0 ** -24
    rel_dr = rel_dk = 0.0
    ratio_dr = ratio_dk = 0.0
    floor_rows = 0
    for i in range(r.shape[0]):
        zed = (r[i] - b_or[i]) / t
        above = zed > 0                      # p > 1/2
        dev = g[i] - dk_or[i]
        floor_dr = (u / t) * float(np.linalg.norm(dev[above]))
        norm_dr = float(np.linalg.norm(dr_or[i]))
        err_dr = float(np.linalg.norm(dr_gpu[i] - dr_or[i]))
        assert err_dr <= max(TOL_GRAD * norm_dr, floor_dr), (
            f"{name}: row {i}: ||ddr|| = {err_dr:.3e}, ||dr|| = {norm_dr:.3e}, floor {floor_dr:.3e}")
        if norm_dr > 0:
            rel_dr = max(rel_dr, err_dr / norm_dr)
            ratio_dr = max(ratio_dr, floor_dr / (TOL_GRAD * norm_dr))
        a = np.abs(zed)
        w = np.exp(-(a - a.min()))
        scale = float(np.sum(w * np.abs(g[i])) / np.sum(w))
        D = float(np.sum(0.5 * np.exp(-a))) / t
        floor_dk = (u / t) * float(np.sum(np.abs(dev[above]))) / D if D > 0 else math.inf
        err_dk = abs(dk_gpu[i] - dk_or[i])
        if math.isfinite(floor_dk):
            assert err_dk <= max(TOL_GRAD * scale, floor_dk), (
                f"{name}: row {i}: |ddk| = {err_dk:.3e}, scale {scale:.3e}, floor {floor_dk:.3e}")
        if scale > 0:
            rel_dk = max(rel_dk, err_dk / scale)
            if math.isfinite(floor_dk):
                ratio_dk = max(ratio_dk, floor_dk / (TOL_GRAD * scale))
        if floor_dr > TOL_GRAD * norm_dr or (math.isfinite(floor_dk) and floor_dk > TOL_GRAD * scale):
            floor_rows += 1
    check_backward.last = (ratio_dr, ratio_dk, floor_rows)
    return rel_dr, rel_dk


check_backward.last = (0.0, 0.0, 0)
