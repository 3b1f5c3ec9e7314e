"""The C-ABI library: it loads, exports every function include/lapsum.h
declares, and its host-only logic (argument checks, path choice, bracket
indices, workspace sizes) is right.  No GPU is needed: nothing here launches
a kernel.
"""
import ctypes
import math
import os
import re
import subprocess

import pytest
import scipy.stats

import sparse_selection_primitive_amd as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lapsum.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        from sparse_selection_primitive_amd import build
        build.build()
    return L.load_library()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lapsum_[a-z_]+)\s*\(", text)))


def test_header_declares_the_north_star_entry_points():
    fns = header_functions()
    for name in ("lapsum_forward", "lapsum_backward", "lapsum_workspace_bytes", "lapsum_status_string"):
        assert name in fns
    assert set(fns) == set(L.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (lapsum_\w+)", out))
    for name in header_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_struct_layouts_match_header():
    # sizes fixed by the header's field lists (natural alignment on x86-64)
    assert ctypes.sizeof(L.RowStats) == 4 * 8 + 3 * 8 + 2 * 4
    assert ctypes.sizeof(L.Options) == 4 + 4 + 8 + 8 + 8 + 8 + 8 + 8 + 4 + 4 + 8 + 8
    assert ctypes.sizeof(L.PlanInfo) == 4 + 4 + 4 * 8 + 4 + 4 + 8 + 8


def test_flag_and_path_constants_match_header():
    text = open(HEADER).read()
    flags = dict(re.findall(r"#define LAPSUM_FLAG_(\w+) (0x[0-9a-fA-F]+)", text))
    assert flags, "no flags parsed"
    for name, value in flags.items():
        assert getattr(L, "FLAG_" + name) == int(value, 16), name
    paths = dict(re.findall(r"LAPSUM_PATH_(\w+) = (\d+)", text))
    for name, value in paths.items():
        assert getattr(L, "PATH_" + name) == int(value), name


def test_status_strings(lib):
    for code in range(9):
        s = lib.lapsum_status_string(code).decode()
        assert s and s != "unknown status"
    assert lib.lapsum_status_string(99).decode() == "unknown status"


@pytest.mark.parametrize("n,k,m,delta", [
    (100_000_000, 1e5, 65536, 1e-6),
    (3_317_760, 600, 65536, 1e-6),
    (65536, 3277, 4096, 1e-6),
    (2000, 100, 256, 0.2),
    (1000, 999, 64, 0.01),
    (1000, 1, 64, 0.01),
    (10**7, 123.5, 1 << 14, 1e-3),
])
def test_bracket_indices_match_scipy(lib, n, k, m, delta):
    lo, hi = L.bracket_indices(n, k, m, delta)
    N = scipy.stats.binom(m, 1 - k / n)
    half = delta / 2
    if lo >= 1:
        assert N.cdf(lo - 1) <= half * (1 + 1e-9)
    if lo < m:
        assert N.cdf(lo) > half * (1 - 1e-9)
    if hi <= m:
        assert N.sf(hi - 1) <= half * (1 + 1e-9)
    if hi >= 2:
        assert N.sf(hi - 2) > half * (1 - 1e-9)


def test_bracket_indices_of_the_workloads(lib):
    assert L.bracket_indices(100_000_000, 1e5, 65536, 1e-6) == (65427, 65507)
    assert L.bracket_indices(3_317_760, 600, 65536, 1e-6) == (65504, 65537)
    assert L.bracket_indices(65536, 3277, 4096, 1e-6) == (3820, 3957)


def test_path_choice_and_plan(lib):
    assert L.plan(16384, 256, 8, 0.05)["path"] == L.PATH_ONCHIP
    assert L.plan(8, 1024, 32, 0.1)["path"] == L.PATH_ONCHIP
    assert L.plan(8, 1024, 32, 0.1)["forward_bytes"] == 0
    p = L.plan(32, 65536, 3277, 0.01)
    assert p["path"] == L.PATH_FULLSORT and p["forward_bytes"] > 2 * 32 * 65536 * 4
    p = L.plan(1, 3_317_760, 600, 1e-3)
    assert p["path"] == L.PATH_BRACKET and p["m"] == 65536 and p["band_onchip"] == 1
    assert (p["lo"], p["hi"]) == (65504, 65537)
    p = L.plan(1, 100_000_000, 1e5, 1e-2)
    assert p["path"] == L.PATH_BRACKET and p["m"] == 65536 and p["band_onchip"] == 0
    assert p["band_capacity"] % 4096 == 0 and p["band_capacity"] >= 3 * 122_070
    # the fallback needs room for a full sort of the row: two key buffers
    assert p["forward_bytes"] >= 2 * 100_000_000 * 4
    p = L.plan(32, 65536, 3277, 0.01, path="bracket")
    assert p["m"] == 4096 and (p["lo"], p["hi"]) == (3820, 3957) and p["band_onchip"] == 1
    assert L.plan(4, 2000, 10, 1.0)["backward_bytes"] > 0
    assert L.plan(4, 1000, 10, 1.0)["backward_bytes"] == 0


@pytest.mark.parametrize("args,code", [
    ((0, 10, 1.0, 1.0), 2), ((1, 0, 0.5, 1.0), 2), ((1, 10, 0.0, 1.0), 3), ((1, 10, 10.0, 1.0), 3),
    ((1, 10, math.nan, 1.0), 3), ((1, 10, 1.0, 0.0), 4), ((1, 10, 1.0, math.inf), 4), ((1, 10, 1.0, -1.0), 4),
])
def test_plan_rejects_bad_arguments(lib, args, code):
    with pytest.raises(L.LapsumError, match=f"status {code}"):
        L.plan(*args)


def test_plan_rejects_bad_options(lib):
    with pytest.raises(L.LapsumError, match="status 6"):
        L.plan(1, 10000, 5, 1.0, path="onchip")
    for kw in ({"sample_log2": 3}, {"sample_log2": 21}, {"delta": 1.0}, {"delta": -0.5},
               {"band_capacity": -1}, {"bracket_override": (1.0, 0.0)}, {"path": 7}):
        with pytest.raises(L.LapsumError, match="status 7"):
            L.plan(1, 10000, 5, 1.0, **kw)


def test_plan_per_row_parameters(lib):
    """Per-row k / t (device arrays, never read by the host): the scalars are
    then not checked, AUTO takes the full-sort path above the on-chip size
    (the bracket's sample indices need k on the host), and a forced
    bracketing path is refused."""
    dev = 4096  # a device address stand-in: planning never dereferences it
    assert L.plan(64, 256, 0.0, 0.0, k_rows_ptr=dev, t_rows_ptr=dev)["path"] == L.PATH_ONCHIP
    assert L.plan(2, 3_317_760, 0.0, 1e-3, k_rows_ptr=dev)["path"] == L.PATH_FULLSORT
    assert L.plan(2, 3_317_760, 600, -1.0, t_rows_ptr=dev)["path"] == L.PATH_FULLSORT
    with pytest.raises(L.LapsumError, match="status 6"):
        L.plan(2, 3_317_760, 600, 1e-3, path="bracket", k_rows_ptr=dev)
    with pytest.raises(L.LapsumError, match="status 3"):  # the scalar k is still checked without k_rows
        L.plan(2, 20000, 0.0, 1e-3, t_rows_ptr=dev)


def test_plan_widen_steps_range(lib):
    for w in (-1, 0, 1, 4):
        L.plan(1, 3_317_760, 600, 1e-3, widen_steps=w)
    for w in (-2, 5):
        with pytest.raises(L.LapsumError, match="status 7"):
            L.plan(1, 3_317_760, 600, 1e-3, widen_steps=w)


def test_forward_rejects_null_and_small_workspace_without_launching(lib):
    opt = L.make_options()
    # NULL r with a valid shape: checked before anything is launched
    rc = lib.lapsum_forward(None, 1, 100, 5.0, 1.0, None, None, None, 0, ctypes.byref(opt), None)
    assert rc == 1
    # a bracketing call with too small a workspace
    rc = lib.lapsum_forward(ctypes.c_void_p(256), 1, 2_000_000, 5.0, 1.0, ctypes.c_void_p(256),
                            ctypes.c_void_p(256), ctypes.c_void_p(256), 1024, ctypes.byref(opt), None)
    assert rc == 5
    # misaligned workspace
    need = L.workspace_bytes(1, 2_000_000, 5.0, 1.0)
    rc = lib.lapsum_forward(ctypes.c_void_p(256), 1, 2_000_000, 5.0, 1.0, ctypes.c_void_p(256),
                            ctypes.c_void_p(256), ctypes.c_void_p(257), need, ctypes.byref(opt), None)
    assert rc == 5
    rc = lib.lapsum_backward(None, None, None, 1, 100, 1.0, None, None, None, 0, None, None)
    assert rc == 1
