"""The backward entry point that allocates nothing (lapsum_backward_noalloc)
against lapsum_backward, through the C ABI: the same kernels run on the
library's fixed device buffer instead of a caller workspace, so dr and dk must
be bitwise equal.  Calls run back to back, each smaller than the one before,
so the fixed buffer still holds the previous call's partials when the next
call starts: a result that depended on stale contents would differ."""
import ctypes

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def L():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_selection_primitive_amd as lib
    lib.load_library()
    return lib


def _case(L, rows, n, t, seed, per_row_t=False):
    g0 = np.random.Generator(np.random.PCG64(seed))
    r = torch.from_numpy(g0.standard_normal((rows, n)).astype(np.float32)).cuda()
    g = torch.from_numpy(g0.standard_normal((rows, n)).astype(np.float32)).cuda()
    k = max(1.0, 0.01 * n)
    tt = torch.from_numpy(np.exp(g0.uniform(np.log(0.02), np.log(0.2), rows))).cuda() if per_row_t else t
    p, b = L.lapsum_forward(r, k, tt)
    return g, p, b, tt


def _noalloc(L, g, p, b, t):
    """Direct C-ABI call; outputs preallocated here, nothing else passed."""
    lib = L.load_library()
    rows, n = g.shape
    dr = torch.full_like(g, float("nan"))
    dk = torch.full((rows,), float("nan"), dtype=torch.float32, device=g.device)
    opt = L.make_options()
    ts = 1.0
    if isinstance(t, torch.Tensor):
        opt.t_rows = t.data_ptr()
    else:
        ts = float(t)
    stream = torch.cuda.current_stream().cuda_stream
    rc = lib.lapsum_backward_noalloc(g.data_ptr(), p.data_ptr(), b.data_ptr(), rows, n, ts, dr.data_ptr(),
                                     dk.data_ptr(), ctypes.byref(opt), stream)
    assert rc == 0, lib.lapsum_status_string(rc)
    return dr, dk


@pytest.mark.parametrize("sizes", [
    [(64, 300_000), (3, 5000)],             # streaming: 4096 partials, then 3 x 2
    [(20000, 1028), (1, 2_000_000)],        # one partial per row (20000), then one long row
    [(100, 256), (7, 1000)],                # on-chip rows: no scratch at all
])
def test_noalloc_backward_matches_backward(L, sizes):
    for i, (rows, n) in enumerate(sizes):
        print(f"[case] noalloc backward rows={rows} n={n} (call {i + 1} of {len(sizes)})", flush=True)
        g, p, b, t = _case(L, rows, n, 0.05, seed=9100 + 7 * rows + i, per_row_t=(i == 1))
        dr_ref, dk_ref = L.lapsum_backward(g, p, b, t)
        dr, dk = _noalloc(L, g, p, b, t)
        torch.cuda.synchronize()
        assert torch.equal(dr, dr_ref) and torch.equal(dk, dk_ref), (rows, n)


def test_noalloc_backward_python_wrapper(L):
    g, p, b, t = _case(L, 5, 50_000, 0.03, seed=9200)
    dr_ref, dk_ref = L.lapsum_backward(g, p, b, t)
    dr, dk = L.lapsum_backward_noalloc(g, p, b, t)
    torch.cuda.synchronize()
    assert torch.equal(dr, dr_ref) and torch.equal(dk, dk_ref)
