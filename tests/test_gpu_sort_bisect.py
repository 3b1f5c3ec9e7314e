"""GPU parity of the whole-row sort path, the bisection baseline and the
DFTopK midpoint diagnostic, through the C ABI, against the CPU oracle.

"Fast LapSum: Exact Differentiable Top-k at Million Scale", section 2.2: the
full-sort solver (sort every score, one stable prefix/suffix scan, index
lookup, closed-form root) replaces the iterative bisection of earlier
implementations; both must reach the same unique threshold b (section 2.1,
eq. (2)).  Section 2.3: DFTopK fixes the threshold at the midpoint of the
k-th and (k+1)-th largest scores.  Tolerances: tests/parity.py.
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


def gpu(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def check(name, L, O, r, g, k, t, path, **kw):
    log(f"[case] {name} path={path} shape={r.shape} k={k} t={t}")
    rt = gpu(r)
    p, b = L.lapsum_forward(rt, k, t, path=path, **kw)
    out = {}
    if g is not None:
        dr, dk = L.lapsum_backward(gpu(g), p, b, t)
        out["dr"], out["dk"] = dr.cpu().numpy(), dk.cpu().numpy()
    torch.cuda.synchronize()
    pg, bg = p.cpu().numpy(), b.cpu().numpy()
    p_or, b_or = O.forward(r, k, t)
    dp, db = check_forward(f"{name} ({path})", k, t, pg, bg, p_or, b_or)
    err = check_budget(f"{name} ({path})", k, pg)
    msg = f"  max|dp|={dp:.2e} max|db|/t={db:.2e} |sum-k|={err:.2e}"
    if g is not None:
        dr_or, dk_or = O.backward(r, b_or, g, t)
        edr, edk = check_backward(f"{name} ({path})", r, b_or, g, t, out["dr"], out["dk"], dr_or, dk_or)
        msg += f" dr_rel={edr:.2e} dk_rel={edk:.2e}"
    log(msg)
    return pg, bg


PATHS = ["sort", "bisect"]


@pytest.mark.parametrize("path", PATHS)
def test_workloads(L, O, path):
    from sparse_selection_primitive_amd import workloads
    for w in (workloads.tiny(), workloads.coder(), workloads.routing(rows=2048)):
        check(w.name, L, O, w.r, w.g, w.k, w.t, path)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("n,rows", [(1, 3), (2, 2), (3, 4), (7, 2), (100, 3), (1023, 2), (1025, 2), (4095, 2),
                                    (4096, 2), (4097, 2), (16383, 2), (16384, 2), (16385, 2), (70001, 2),
                                    (300_001, 1)])
def test_ragged_sizes(L, O, path, n, rows):
    """Sizes across the sort tiles (4096), the solve tiles (16384), the
    on-chip bisection limits (1024, 4096, 16384) and odd tails."""
    g0 = np.random.Generator(np.random.PCG64(8000 + n))
    r = g0.standard_normal((rows, n)).astype(np.float32)
    g = g0.standard_normal((rows, n)).astype(np.float32)
    k = min(max(0.5, 0.1 * n), n - 0.5)
    check(f"n={n}", L, O, r, g, k, 0.05, path)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("k_frac", [1e-6, 0.5, 1 - 1e-6])
def test_end_budgets(L, O, path, k_frac):
    g0 = np.random.Generator(np.random.PCG64(8101))
    n = 20000
    r = g0.standard_normal((2, n)).astype(np.float32)
    k = min(max(k_frac * n, 1e-3), n - 1e-3)
    check(f"end budget k={k}", L, O, r, None, k, 0.05, path)


@pytest.mark.parametrize("path", PATHS)
def test_ties_constant_rows_and_tiny_t(L, O, path):
    g0 = np.random.Generator(np.random.PCG64(8102))
    vals = g0.standard_normal(64).astype(np.float32)
    r = vals[g0.integers(0, 64, size=(3, 5000))]
    r[2, :] = 0.25  # constant row
    check("ties", L, O, r, None, 40.5, 0.05, path)
    r2 = np.sort(g0.standard_normal((2, 30000)).astype(np.float32), axis=1)
    check("sorted rows, tiny t", L, O, r2, None, 1000.5, 1e-6, path)
    r3 = -np.abs(g0.standard_normal((2, 9000))).astype(np.float32)  # -0.0 and +0.0 included
    r3[:, :50] = 0.0
    r3[:, 50:100] = -0.0
    check("signed zeros", L, O, r3, None, 75.0, 0.01, path)


@pytest.mark.parametrize("path", PATHS)
def test_per_row_budget_and_temperature(L, O, path):
    g0 = np.random.Generator(np.random.PCG64(8103))
    for rows, n in ((64, 300), (6, 20000)):
        r = g0.standard_normal((rows, n)).astype(np.float32)
        k = g0.uniform(1.0, n - 1.0, rows)
        t = np.exp(g0.uniform(np.log(0.01), np.log(0.5), rows))
        log(f"[case] per-row {path} rows={rows} n={n}")
        p, b = L.lapsum_forward(gpu(r), gpu(k), gpu(t), path=path)
        torch.cuda.synchronize()
        pg, bg = p.cpu().numpy(), b.cpu().numpy()
        for i in range(rows):
            p_or, b_or = O.forward(r[i], float(k[i]), float(t[i]))
            check_forward(f"per-row {path} row {i}", float(k[i]), float(t[i]), pg[i], bg[i:i + 1], p_or, [b_or])
            check_budget(f"per-row {path} row {i}", float(k[i]), pg[i])


@pytest.mark.parametrize("path", PATHS)
def test_determinism(L, path):
    from sparse_selection_primitive_amd import workloads
    w = workloads.coder(rows=4)
    rt = gpu(w.r)
    a = L.lapsum_forward(rt, w.k, w.t, path=path)
    b = L.lapsum_forward(rt, w.k, w.t, path=path)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_sort_path_agrees_with_bucket_and_bracket(L):
    """The same threshold from three exact routes (whole-row sort, bucket
    selection, certified bracketing), up to rounding."""
    from sparse_selection_primitive_amd import workloads
    w = workloads.coder()
    rt = gpu(w.r)
    bs = L.lapsum_forward(rt, w.k, w.t, path="sort")[1]
    bb = L.lapsum_forward(rt, w.k, w.t, path="bucket")[1]
    br = L.lapsum_forward(rt, w.k, w.t, path="bracket")[1]
    torch.cuda.synchronize()
    assert float((bs - bb).abs().max()) / w.t <= 1e-6
    assert float((bs - br).abs().max()) / w.t <= 1e-6


# ------------------------------------------------------- DFTopK midpoint
def check_midpoint(name, L, O, r, k, t):
    log(f"[case] midpoint {name} shape={r.shape} k={k} t={t}")
    bm, mass = L.midpoint_mass(gpu(r), k, t)
    torch.cuda.synchronize()
    bm, mass = bm.cpu().numpy(), mass.cpu().numpy()
    bm_or, mass_or = O.midpoint_mass(r, k, t)
    bm_or, mass_or = np.atleast_1d(bm_or), np.atleast_1d(mass_or)
    # both sides take (s_(k) + s_(k+1))/2 in fp64 of the same fp32 scores
    assert np.array_equal(bm, bm_or), (name, bm[:4], bm_or[:4])
    err = float(np.max(np.abs(mass - mass_or)))
    assert err <= 1e-5 * max(1.0, k), (name, err)
    drift = float(np.mean(mass_or / k - 1.0))
    log(f"  |dmass|={err:.2e} mean drift (mass/k - 1)={drift:.3e}")
    return drift


def test_midpoint_workloads(L, O):
    from sparse_selection_primitive_amd import workloads
    for w in (workloads.tiny(), workloads.routing(rows=4096), workloads.coder(), workloads.attack()):
        check_midpoint(w.name, L, O, w.r, int(round(w.k)), w.t)


@pytest.mark.parametrize("n", [2, 3, 5, 8, 4096, 4097, 70001])
def test_midpoint_sizes_and_end_budgets(L, O, n):
    g0 = np.random.Generator(np.random.PCG64(8200 + n))
    r = g0.standard_normal((3, n)).astype(np.float32)
    for k in sorted({1, max(1, n // 2), n - 1}):
        check_midpoint(f"n={n}", L, O, r, k, 0.1)


def test_midpoint_ties(L, O):
    g0 = np.random.Generator(np.random.PCG64(8210))
    vals = g0.standard_normal(16).astype(np.float32)
    r = vals[g0.integers(0, 16, size=(4, 1000))]
    check_midpoint("ties", L, O, r, 100, 0.05)


def test_midpoint_rejects_bad_k(L):
    r = gpu(np.zeros((1, 10), dtype=np.float32))
    for k in (0, 10):
        with pytest.raises(L.LapsumError, match="status 3"):
            L.midpoint_mass(r, k, 0.1)
