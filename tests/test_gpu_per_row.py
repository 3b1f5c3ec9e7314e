"""GPU parity with a budget k and a temperature t per row (device arrays),
against the oracle solved row by row with that row's values.

Operator: "Fast LapSum: Exact Differentiable Top-k at Million Scale",
section 2.1 (eqs. (1)-(2), analytic VJP) -- the operator is defined per
row, so per-row k and t change nothing but which values each row uses.
Paths: on-chip (wave teams and one-workgroup rows), bucket (AUTO above
8192 scores up to 2^20) and bracketing (AUTO above 2^20, or forced), where
every row's order-statistic indices come from its own k (section 2.2,
probabilistic bracketing, step 1) and its sample is noised with its own t.
Tolerances: tests/parity.py.
"""
import ctypes
import math

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


def _case(seed, rows, n, k_lo, k_hi, t_lo, t_hi):
    g0 = np.random.Generator(np.random.PCG64(seed))
    r = g0.standard_normal((rows, n)).astype(np.float32)
    g = g0.standard_normal((rows, n)).astype(np.float32)
    k = g0.uniform(k_lo, k_hi, rows)
    t = np.exp(g0.uniform(np.log(t_lo), np.log(t_hi), rows))
    return r, g, k, t


def _run(L, r, g, k, t, **opts):
    rt = torch.from_numpy(r).cuda()
    kt = torch.from_numpy(np.asarray(k, dtype=np.float64)).cuda() if isinstance(k, np.ndarray) else k
    tt = torch.from_numpy(np.asarray(t, dtype=np.float64)).cuda() if isinstance(t, np.ndarray) else t
    out = L.lapsum_forward(rt, kt, tt, **opts)
    p, b = out[0], out[1]
    res = {"p": p, "b": b}
    if len(out) > 2:
        res["stats"] = out[2]
    if g is not None:
        dr, dk = L.lapsum_backward(torch.from_numpy(g).cuda(), p, b, tt)
        res["dr"], res["dk"] = dr, dk
    torch.cuda.synchronize()
    return {key: (v.cpu().numpy() if isinstance(v, torch.Tensor) else v) for key, v in res.items()}


def _check_rows(name, O, r, g, k, t, res, rows_idx=None):
    rows = r.shape[0]
    for i in (range(rows) if rows_idx is None else rows_idx):
        p_or, b_or = O.forward(r[i], float(k[i]), float(t[i]))
        check_forward(f"{name} row {i}", k[i], t[i], res["p"][i], res["b"][i], p_or, b_or)
        check_budget(f"{name} row {i}", k[i], res["p"][i][None, :])
        if g is not None:
            dr_or, dk_or = O.backward(r[i][None, :], np.array([b_or]), g[i][None, :], float(t[i]))
            check_backward(f"{name} row {i}", r[i][None, :], np.array([b_or]), g[i][None, :], float(t[i]),
                           res["dr"][i][None, :], res["dk"][i:i + 1], dr_or, dk_or)


@pytest.mark.parametrize("rows,n,k_hi", [(512, 256, 40.0), (96, 1000, 900.0), (24, 3000, 2990.0)])
def test_per_row_onchip(L, O, rows, n, k_hi):
    """Routing-like rows, each with its own k (small and near n: the window
    and its complement, or the whole-row sort) and t (two decades)."""
    r, g, k, t = _case(4101 + n, rows, n, 0.5, k_hi, 0.01, 1.0)
    log(f"[case] per-row on-chip rows={rows} n={n}")
    res = _run(L, r, g, k, t, stats=True)
    assert not np.any(res["stats"]["flags"].numpy() & L.FLAG_INVALID)
    _check_rows("per-row on-chip", O, r, g, k, t, res)


def test_per_row_bucket(L, O):
    """Rows above the on-chip size take the bucket path (AUTO), each with
    its own budget and temperature."""
    r, g, k, t = _case(4201, 6, 20000, 1.0, 19000.0, 1e-3, 0.5)
    assert L.plan(6, 20000, 0.0, 0.0, k_rows_ptr=4096, t_rows_ptr=4096)["path"] == L.PATH_BUCKET
    log("[case] per-row bucket rows=6 n=20000")
    res = _run(L, r, g, k, t, stats=True)
    _check_rows("per-row bucket", O, r, g, k, t, res)


def _same_end(got, want):
    return got == want if math.isinf(want) else abs(got - want) <= 2.5e-7 * abs(want) + 1e-30


def _check_brackets(L, r, k, t, stats, seed=0, delta=1e-6):
    """Each valid row's bracket ends against the oracle's own sample of that
    row (noised with its t) and the binomial indices of its k."""
    from oracle import bracket as ob
    rows, n = r.shape
    m = 1 << ob.default_sample_log2(n)
    flags = stats["flags"].numpy()
    for i in range(rows):
        if flags[i] & L.FLAG_INVALID:
            continue
        want = ob.bracket(r[i], float(k[i]), float(t[i]), m, delta, seed, row=i)
        got = (stats["a_lo"][i].item(), stats["a_hi"][i].item())
        assert _same_end(got[0], want[0]) and _same_end(got[1], want[1]), (i, got, want[:2], want[2:])


def test_per_row_large_rows(L, O):
    """Two 2.5M-score rows with their own k and t: AUTO takes the
    bracketing path, each row's bracket comes from its own k's indices and
    its own t's noise and holds b; the streaming backward reads t per row."""
    g0 = np.random.Generator(np.random.PCG64(4301))
    r = g0.standard_normal((2, 2_500_000)).astype(np.float32)
    g = g0.standard_normal((2, 2_500_000)).astype(np.float32)
    k = np.array([1000.5, 123456.0])
    t = np.array([1e-3, 0.05])
    plan = L.plan(2, 2_500_000, 0.0, 0.0, k_rows_ptr=4096, t_rows_ptr=4096)
    assert plan["path"] == L.PATH_BRACKET and plan["lo"] == -1 and plan["band_onchip"] == 0
    log("[case] per-row large rows 2 x 2.5M")
    res = _run(L, r, g, k, t, stats=True)
    flags = res["stats"]["flags"].numpy()
    log(f"  flags {flags}")
    assert np.all(flags & L.FLAG_HIT) and not np.any(flags & (L.FLAG_FALLBACK | L.FLAG_INVALID)), flags
    _check_brackets(L, r, k, t, res["stats"])
    _check_rows("per-row large", O, r, g, k, t, res)


def test_per_row_bracket_forced_wide_budgets(L, O):
    """Forced bracketing on shorter rows whose budgets run from near 0 to
    near n (open lower or upper bracket ends) with temperatures over three
    decades: brackets and results against the oracle, row by row."""
    rows, n = 8, 300_000
    r, g, _, _ = _case(4501, rows, n, 1.0, 2.0, 0.1, 0.2)
    k = np.array([0.5, 3.0, 600.0, 0.25 * n, 0.5 * n + 0.5, n - 700.0, n - 2.0, n - 0.5])
    t = np.exp(np.random.Generator(np.random.PCG64(4502)).uniform(np.log(1e-3), np.log(1.0), rows))
    log(f"[case] per-row forced bracket rows={rows} n={n}")
    res = _run(L, r, g, k, t, path="bracket", stats=True)
    flags = res["stats"]["flags"].numpy()
    log(f"  flags {flags}")
    assert np.all(flags & L.FLAG_BRACKET) and not np.any(flags & L.FLAG_INVALID), flags
    _check_brackets(L, r, k, t, res["stats"])
    _check_rows("per-row forced bracket", O, r, g, k, t, res)


def test_per_row_bracket_invalid_rows(L, O):
    """Bracketing rows whose k or t is out of range get NaN outputs and the
    INVALID flag; the other rows of the call are unaffected."""
    rows, n = 4, 1_500_000
    r, g, _, _ = _case(4601, rows, n, 1.0, 2.0, 0.1, 0.2)
    k = np.array([800.0, 0.0, 5000.5, 900.0])
    t = np.array([0.01, 0.01, 0.02, -1.0])
    log("[case] per-row bracket invalid rows")
    res = _run(L, r, g, k, t, stats=True)
    flags = res["stats"]["flags"].numpy()
    log(f"  flags {flags}")
    for i in (1, 3):
        assert flags[i] & L.FLAG_INVALID, (i, flags)
        assert np.all(np.isnan(res["p"][i])) and np.isnan(res["b"][i]), i
    for i in (0, 2):
        assert not flags[i] & L.FLAG_INVALID and flags[i] & L.FLAG_HIT, (i, flags)
    _check_brackets(L, r, k, t, res["stats"])
    _check_rows("per-row bracket valid rows", O, r, None, k, t, res, rows_idx=[0, 2])


@pytest.mark.parametrize("n", [256, 3000, 20000])
def test_per_row_equal_values_match_scalar_call(L, n):
    """Per-row arrays holding one value everywhere give bitwise the results
    of the scalar call (same kernels' arithmetic, values read per row)."""
    r, g, _, _ = _case(4401 + n, 16, n, 1.0, 2.0, 0.1, 0.2)
    k, t = 0.25 * n + 0.5, 0.07
    a = _run(L, r, g, k, t)
    b = _run(L, r, g, np.full(16, k), np.full(16, t))
    for key in ("p", "b", "dr", "dk"):
        assert np.array_equal(a[key], b[key]), (n, key)


@pytest.mark.parametrize("n", [256, 20000])
def test_per_row_invalid_values_give_nan_rows(L, O, n):
    """Rows whose k or t is out of range (k <= 0, k >= n, t <= 0, t = inf,
    NaN) get NaN p, b, dr, dk and the INVALID flag; the other rows are
    unaffected."""
    rows = 8
    r, g, k, t = _case(4501 + n, rows, n, 2.0, 0.5 * n, 0.05, 0.5)
    bad = {1: ("k", 0.0), 2: ("k", float(n)), 3: ("t", 0.0), 4: ("t", np.inf), 5: ("k", np.nan), 6: ("t", -1.0)}
    for i, (which, v) in bad.items():
        (k if which == "k" else t)[i] = v
    rt = torch.from_numpy(r).cuda()
    kt, tt = torch.from_numpy(k).cuda(), torch.from_numpy(t).cuda()
    p, b, st = L.lapsum_forward(rt, kt, tt, stats=True)
    sbuf = torch.zeros(rows * ctypes.sizeof(L.RowStats), dtype=torch.uint8, device="cuda")
    dr, dk = L.lapsum_backward(torch.from_numpy(g).cuda(), p, b, tt, stats_buf=sbuf)
    torch.cuda.synchronize()
    fl = st["flags"].numpy()
    bfl = L.decode_stats(sbuf, rows)["flags"].numpy()
    p, b, dr, dk = p.cpu().numpy(), b.cpu().numpy(), dr.cpu().numpy(), dk.cpu().numpy()
    for i in range(rows):
        if i in bad:
            assert fl[i] & L.FLAG_INVALID and np.all(np.isnan(p[i])) and np.isnan(b[i]), i
            if bad[i][0] == "t":
                assert bfl[i] & L.FLAG_INVALID and np.all(np.isnan(dr[i])) and np.isnan(dk[i]), i
        else:
            assert not fl[i] & L.FLAG_INVALID
            p_or, b_or = O.forward(r[i], float(k[i]), float(t[i]))
            check_forward(f"valid row {i}", k[i], t[i], p[i], b[i], p_or, b_or)


def test_autograd_per_row_budget_gradient(L, O):
    """soft_topk with a per-row budget tensor that requires grad: k.grad is
    the VJP's dk (the oracle's per row), r.grad its dr."""
    r, g, k, t = _case(4601, 32, 256, 1.0, 30.0, 0.02, 0.3)
    rt = torch.from_numpy(r).cuda().requires_grad_(True)
    kt = torch.from_numpy(k).cuda().requires_grad_(True)
    tt = torch.from_numpy(t).cuda()
    p = L.soft_topk(rt, kt, tt)
    (p * torch.from_numpy(g).cuda()).sum().backward()
    kg, rg = kt.grad.cpu().numpy(), rt.grad.cpu().numpy()
    for i in range(32):
        _, b_or = O.forward(r[i], float(k[i]), float(t[i]))
        dr_or, dk_or = O.backward(r[i][None, :], np.array([b_or]), g[i][None, :], float(t[i]))
        check_backward(f"autograd per-row row {i}", r[i][None, :], np.array([b_or]), g[i][None, :], float(t[i]),
                       rg[i][None, :], kg[i:i + 1].astype(np.float32), dr_or, dk_or)
