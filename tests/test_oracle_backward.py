"""Pins of the oracle's analytic VJP.

Source: "Fast LapSum: Exact Differentiable Top-k at Million Scale",
section 2.1: the backward pass is an analytic vector-Jacobian product (no
straight-through surrogate).  The formula is not printed; the oracle derives
it by implicit differentiation of eq. (2).  These tests pin it to central
finite differences of the forward (bisection on the definition), and to the
invariances that the definition implies.
"""
import numpy as np
import pytest


def rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _fd_jacobian_t_g(oracle_mod, r, k, t, g, h):
    """sum_i g_i dp_i/dr_j by central differences, one column at a time."""
    n = r.size
    out = np.empty(n)
    for j in range(n):
        rp = r.copy()
        rm = r.copy()
        rp[j] += h
        rm[j] -= h
        pp, _ = oracle_mod.forward(rp, k, t, threads=1)
        pm, _ = oracle_mod.forward(rm, k, t, threads=1)
        out[j] = np.dot(g, pp - pm) / (2 * h)
    return out


@pytest.mark.parametrize("seed,n,k,t", [(61, 8, 3.0, 0.5), (62, 24, 5.5, 0.2), (63, 40, 1.0, 1.0),
                                        (64, 33, 30.0, 0.05)])
def test_vjp_matches_central_differences(oracle_mod, seed, n, k, t):
    g0 = rng(seed)
    r = g0.standard_normal(n) * 0.3
    g = g0.standard_normal(n)
    _, b = oracle_mod.forward(r, k, t, threads=1)
    dr, dk = oracle_mod.backward(r, b, g, t, threads=1)
    h = 1e-6 * t
    fd = _fd_jacobian_t_g(oracle_mod, r, k, t, g, h)
    scale = np.linalg.norm(fd)
    assert np.linalg.norm(dr - fd) <= 1e-6 * scale
    # dk by central differences on k
    hk = 1e-6
    pp, _ = oracle_mod.forward(r, k + hk, t, threads=1)
    pm, _ = oracle_mod.forward(r, k - hk, t, threads=1)
    fdk = np.dot(g, pp - pm) / (2 * hk)
    assert dk == pytest.approx(fdk, rel=1e-6, abs=1e-9)


def test_vjp_random_direction_large_row(oracle_mod):
    """v . dr against a directional finite difference for a larger row."""
    g0 = rng(70)
    n, k, t = 3000, 100.0, 0.05
    r = g0.standard_normal(n)
    g = g0.standard_normal(n)
    v = g0.standard_normal(n)
    _, b = oracle_mod.forward(r, k, t)
    dr, _ = oracle_mod.backward(r, b, g, t)
    h = 1e-6 * t
    pp, _ = oracle_mod.forward(r + h * v, k, t)
    pm, _ = oracle_mod.forward(r - h * v, k, t)
    fd = np.dot(g, pp - pm) / (2 * h)
    assert np.dot(v, dr) == pytest.approx(fd, rel=1e-6)


def test_vjp_invariances(oracle_mod):
    g0 = rng(71)
    n, k, t = 500, 20.0, 0.1
    r = g0.standard_normal(n)
    g = g0.standard_normal(n)
    _, b = oracle_mod.forward(r, k, t)
    dr, dk = oracle_mod.backward(r, b, g, t)
    # a common shift of r leaves p unchanged: the columns of dp/dr sum to zero
    assert abs(dr.sum()) <= 1e-12 * np.abs(dr).sum()
    # a constant upstream gradient c sees only sum p = k: dr = 0 and dk = c
    drc, dkc = oracle_mod.backward(r, b, np.full(n, 2.5), t)
    assert np.max(np.abs(drc)) <= 1e-12
    assert dkc == pytest.approx(2.5, rel=1e-14)
    # scaling r and t together scales dr by 1/alpha and leaves dk alone
    _, b2 = oracle_mod.forward(3.0 * r, k, 3.0 * t)
    dr2, dk2 = oracle_mod.backward(3.0 * r, b2, g, 3.0 * t)
    np.testing.assert_allclose(dr2, dr / 3.0, rtol=1e-9, atol=1e-14)
    assert dk2 == pytest.approx(dk, rel=1e-10)


def test_vjp_tiny_temperature_keeps_dk_finite(oracle_mod):
    """Far below the score gaps every d_i underflows in fp64; dk is a ratio of
    d-weighted sums and stays the weighted mean of g over the scores nearest
    the threshold."""
    r = np.array([0.0, 1.0, 2.0, 3.0])
    g = np.array([1.0, 2.0, 3.0, 4.0])
    _, b = oracle_mod.forward(r, 2.0, 1e-4)
    assert b == pytest.approx(1.5, abs=1e-12)
    dr, dk = oracle_mod.backward(r, b, g, 1e-4)
    assert np.all(np.isfinite(dr)) and np.max(np.abs(dr)) == 0.0
    # scores 1 and 2 sit at equal distance from b = 1.5: dk = (2 + 3)/2
    assert dk == pytest.approx(2.5, rel=1e-12)
