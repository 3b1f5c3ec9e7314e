"""The spread fallback of the bracketing path (lapsum_options.spread_fallback):
a row whose bracket misses, or whose band overflows, is not widened or solved
by the one workgroup that found the miss; it is recorded in a state array of
its own and solved by the whole-row bucket launches that follow the band
solve, on every workgroup.

Solvers: "Fast LapSum: Exact Differentiable Top-k at Million Scale",
section 2.2 (probabilistic bracketing, step 4: a failed certification falls
back to an exact solve; section 5: pathological distributions).  Every row is
checked against the oracle; a missed row's b must equal the bucket path's b
for that row bit for bit (the same kernels on the same keys), and a row that
hit must equal the default call's result bit for bit.
"""
import numpy as np
import pytest

from parity import check_backward, check_budget, check_forward, log

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def L():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_selection_primitive_amd as lib
    lib.load_library()
    return lib


@pytest.fixture(scope="module")
def O():
    import oracle
    oracle._load()
    return oracle


def _fwd(L, r, k, t, **opts):
    rt = torch.from_numpy(np.ascontiguousarray(r)).cuda()
    kt = torch.from_numpy(np.asarray(k, dtype=np.float64)).cuda() if isinstance(k, np.ndarray) else k
    p, b, st = L.lapsum_forward(rt, kt, t, stats=True, **opts)
    torch.cuda.synchronize()
    return p.cpu().numpy(), b.cpu().numpy(), st


def _check_rows(name, O, r, k, t, p, b, g=None, L=None):
    rows = r.shape[0]
    for i in range(rows):
        ki = float(k[i]) if isinstance(k, np.ndarray) else k
        p_or, b_or = O.forward(r[i], ki, t)
        check_forward(f"{name} row {i}", ki, t, p[i], b[i], p_or, b_or)
        check_budget(f"{name} row {i}", ki, p[i][None, :])


def test_spread_forced_miss(L, O):
    """A bracket forced above every row's b: every row is solved by the
    spread whole-row solve, flagged FALLBACK, equal to the oracle and to the
    bucket path bit for bit; the VJP from its b matches the oracle's."""
    from sparse_selection_primitive_amd import workloads
    w = workloads.coder(rows=4, n=300_000)
    _, b_or = O.forward(w.r, w.k, w.t)
    lo = float(np.max(b_or)) + 0.5
    log(f"[case] spread forced miss 4 x 300000 bracket ({lo}, {lo + 1})")
    p, b, st = _fwd(L, w.r, w.k, w.t, path="bracket", bracket_override=(lo, lo + 1.0), spread_fallback=True)
    fl = st["flags"].numpy()
    assert np.all(fl & L.FLAG_FALLBACK) and not np.any(fl & (L.FLAG_HIT | L.FLAG_WIDENED)), fl
    _check_rows("spread forced miss", O, w.r, w.k, w.t, p, b)
    pb, bb, _ = _fwd(L, w.r, w.k, w.t, path="bucket")
    assert np.array_equal(b, bb) and np.array_equal(p, pb)
    rt = torch.from_numpy(w.r).cuda()
    dr, dk = L.lapsum_backward(torch.from_numpy(w.g).cuda(), torch.from_numpy(p).cuda(),
                               torch.from_numpy(b).cuda(), w.t)
    torch.cuda.synchronize()
    dr_or, dk_or = O.backward(w.r, b_or, w.g, w.t)
    check_backward("spread forced miss", w.r, b_or, w.g, w.t, dr.cpu().numpy(), dk.cpu().numpy(), dr_or, dk_or)
    del rt


def test_spread_natural_misses(L, O):
    """delta = 0.9 on the coder batch: a first bracket this narrow misses on
    many rows.  Missed rows equal the bucket path bit for bit, rows that hit
    equal the default call without widening bit for bit, the stats hold the
    first bracket on every row, and every row matches the oracle."""
    from sparse_selection_primitive_amd import workloads
    w = workloads.coder(rows=32)
    log(f"[case] spread natural misses {w.r.shape} delta=0.9")
    p, b, st = _fwd(L, w.r, w.k, w.t, path="bracket", delta=0.9, seed=5, spread_fallback=True)
    fl = st["flags"].numpy()
    miss = (fl & L.FLAG_FALLBACK) != 0
    log(f"  rows missed: {int(miss.sum())} of {len(fl)}")
    assert miss.sum() > 0, fl
    assert not np.any(fl & L.FLAG_WIDENED)
    assert np.all(((fl & L.FLAG_HIT) != 0) == ~miss)
    _check_rows("spread natural misses", O, w.r, w.k, w.t, p, b)
    pd, bd, std = _fwd(L, w.r, w.k, w.t, path="bracket", delta=0.9, seed=5, widen_steps=-1)
    pb, bb, _ = _fwd(L, w.r, w.k, w.t, path="bucket")
    assert np.array_equal(std["flags"].numpy(), fl)
    for i in range(len(fl)):
        if miss[i]:
            assert b[i] == bb[i] and np.array_equal(p[i], pb[i]), i
        else:
            assert b[i] == bd[i] and np.array_equal(p[i], pd[i]), i
    for key in ("a_lo", "a_hi", "tail_lo", "tail_hi", "count_lo", "count_hi", "band"):
        assert np.array_equal(st[key].numpy(), std[key].numpy()), key


def test_spread_band_overflow(L, O):
    """Heavy ties around b overflow the band of every row: each row takes the
    spread whole-row solve (flags OVERFLOW and FALLBACK)."""
    g0 = np.random.Generator(np.random.PCG64(5207))
    n = 400_000
    r = (np.floor(g0.standard_normal((3, n)) * 8.0) / 8.0).astype(np.float32)
    k, t = 0.25 * n + 0.5, 1e-3
    log(f"[case] spread band overflow 3 x {n} k={k}")
    p, b, st = _fwd(L, r, k, t, path="bracket", band_capacity=64, spread_fallback=True)
    fl = st["flags"].numpy()
    assert np.all(fl & L.FLAG_OVERFLOW) and np.all(fl & L.FLAG_FALLBACK), fl
    _check_rows("spread band overflow", O, r, k, t, p, b)
    pb, bb, _ = _fwd(L, r, k, t, path="bucket")
    assert np.array_equal(b, bb) and np.array_equal(p, pb)


def test_spread_per_row_budgets(L, O):
    """Per-row budgets with a forced miss: each row's spread solve uses its
    own k; a row whose k is out of range gets NaN and no solve."""
    g0 = np.random.Generator(np.random.PCG64(5209))
    n = 1_200_000
    r = g0.standard_normal((3, n)).astype(np.float32)
    k = np.array([1000.5, -1.0, 250_000.0])
    t = 0.02
    log(f"[case] spread per-row budgets 3 x {n} k={k.tolist()}")
    p, b, st = _fwd(L, r, k, t, path="bracket", bracket_override=(10.0, 11.0), spread_fallback=True)
    fl = st["flags"].numpy()
    assert fl[1] & L.FLAG_INVALID and np.isnan(b[1]) and np.all(np.isnan(p[1])), fl
    assert np.all(fl[[0, 2]] & L.FLAG_FALLBACK), fl
    for i in (0, 2):
        p_or, b_or = O.forward(r[i], float(k[i]), t)
        check_forward(f"spread per-row row {i}", k[i], t, p[i], b[i], p_or, b_or)
        check_budget(f"spread per-row row {i}", k[i], p[i][None, :])


def test_spread_second_level(L, O):
    """A 4.5M-score row (second bucket level on) whose forced miss lands in
    a crowded bucket: solved by both spread levels, equal to the bucket path
    bit for bit and to the oracle."""
    g0 = np.random.Generator(np.random.PCG64(5211))
    n = 4_500_000
    r = g0.standard_normal((1, n)).astype(np.float32)
    k, t = float(np.sum(r > 1.06)) + 0.5, 0.01
    log(f"[case] spread second level 1 x {n} k={k}")
    p, b, st = _fwd(L, r, k, t, path="bracket", bracket_override=(-5.0, -4.0), spread_fallback=True)
    assert st["flags"][0].item() & L.FLAG_FALLBACK
    _check_rows("spread second level", O, r, k, t, p, b)
    pb, bb, _ = _fwd(L, r, k, t, path="bucket")
    assert np.array_equal(b, bb) and np.array_equal(p, pb)
