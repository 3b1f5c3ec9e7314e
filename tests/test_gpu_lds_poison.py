"""The LDS-poisoning debug build (liblapsum_ldspoison.so, compiled with
LAPSUM_LDS_POISON): the on-chip forward kernels, the on-chip band solve, the
filter and its per-row totals, and the bucket kernels (count, scans,
scatter, aggregates, locate) set every byte of their LDS to 0xFF (NaN as
fp32 and fp64, all ones as an integer) at entry.  Run against it, the parity
cases below would show NaN or wrong values wherever a kernel read LDS that no
thread of its launch had written.  The library is loaded in a child process
(LAPSUM_LIBRARY), so the product build of this process is untouched.
"""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
POISON = os.path.join(ROOT, "sparse_selection_primitive_amd", "liblapsum_ldspoison.so")

CHILD = r'''
import sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
import numpy as np, torch
import sparse_selection_primitive_amd as L
import oracle
from parity import check_forward, check_backward, check_budget
from sparse_selection_primitive_amd import workloads
assert L.LIB_PATH.endswith("liblapsum_ldspoison.so"), L.LIB_PATH
L.load_library()

def case(name, r, k, t, g=None, **opts):
    rt = torch.from_numpy(r).cuda()
    p, b = L.lapsum_forward(rt, k, t, **opts)[:2]
    res = {{"p": p.cpu().numpy(), "b": b.cpu().numpy()}}
    if g is not None:
        dr, dk = L.lapsum_backward(torch.from_numpy(g).cuda(), p, b, t)
        res["dr"], res["dk"] = dr.cpu().numpy(), dk.cpu().numpy()
    torch.cuda.synchronize()
    assert np.all(np.isfinite(res["p"])) and np.all(np.isfinite(res["b"])), name
    p_or, b_or = oracle.forward(r, k, t)
    check_forward(name, k, t, res["p"], res["b"], p_or, b_or)
    check_budget(name, k, res["p"])
    if g is not None:
        dr_or, dk_or = oracle.backward(r, b_or, g, t)
        check_backward(name, r, b_or, g, t, res["dr"], res["dk"], dr_or, dk_or)
    print("ok", name, flush=True)

rng = np.random.Generator(np.random.PCG64(5101))
w = workloads.routing(rows=1024)
case("routing window", w.r, w.k, w.t, w.g)
case("routing complement", w.r, 256 - 6.5, w.t)
for n in (100, 700, 1024, 3000, 8192):  # ragged wave rows and one-workgroup rows
    r = rng.standard_normal((6, n)).astype(np.float32)
    case(f"on-chip n={{n}}", r, 0.3 * n + 0.5, 0.05, rng.standard_normal((6, n)).astype(np.float32))
c = workloads.coder(rows=4)
case("bracket coder (on-chip band)", c.r, c.k, c.t, c.g, path="bracket")
r = (np.abs(rng.laplace(size=(1, 1_500_000)))).astype(np.float32)
case("bracket attack-like row", r, 600.0, 1e-3, rng.standard_normal((1, 1_500_000)).astype(np.float32))
# the bucket kernels: whole rows (few count workgroups, one-thread scan),
# a bucketed band (capacity above the on-chip band), a 4.5M row whose crowded
# balancing bucket takes the second level (wide scan), and a forced miss
# solved by the spread fallback
r = rng.standard_normal((3, 20000)).astype(np.float32)
case("bucket rows", r, 3000.5, 0.05, rng.standard_normal((3, 20000)).astype(np.float32), path="bucket")
r = rng.standard_normal((2, 600_000)).astype(np.float32)
case("bracket bucketed band", r, 150_000.5, 0.01, path="bracket")
r = rng.standard_normal((1, 4_500_000)).astype(np.float32)
case("bucket second level", r, float(np.sum(r > 1.06)) + 0.5, 0.01, path="bucket")
case("spread fallback", r, float(np.sum(r > 1.06)) + 0.5, 0.01, path="bracket", bracket_override=(-5.0, -4.0),
     spread_fallback=True)
print("all poison cases ok", flush=True)
'''


def test_parity_with_poisoned_lds():
    if not os.path.exists(POISON):
        pytest.skip("liblapsum_ldspoison.so is not built (python __graft_entry__.py builds it)")
    env = dict(os.environ)
    env["LAPSUM_LIBRARY"] = POISON
    src = CHILD.format(root=ROOT, tests=os.path.join(ROOT, "tests"))
    res = subprocess.run([sys.executable, "-c", src], capture_output=True, text=True, timeout=300, env=env)
    print(res.stdout[-3000:])
    assert res.returncode == 0, res.stdout[-2000:] + res.stderr[-4000:]
    assert "all poison cases ok" in res.stdout
