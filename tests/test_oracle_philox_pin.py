"""Pin of the oracle's Philox-4x32-10 stream (oracle/bracket.py) against an
independent implementation: the engine of ROCm's rocRAND library, built as a
small host program from its installed header (tests/philox_ref/).

The bracketing localisation step ("Fast LapSum: Exact Differentiable Top-k at
Million Scale", section 2.2, Probabilistic Bracketing, step 1) draws the
kernel-noised sample from a counter-based generator; the build reads it as
Philox-4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11) with key (seed low word,
seed high word) and counter (sample index, row, 0, 0).  A wrong multiplier,
Weyl constant, round count or word order would change every output word.
CPU only; skipped where hipcc or the rocRAND header is missing.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle.bracket import philox4x32_10

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "philox_ref", "rocrand_philox.cpp")


@pytest.fixture(scope="module")
def ref_bin(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc) or not os.path.exists("/opt/rocm/include/rocrand/rocrand_kernel.h"):
        pytest.skip("hipcc or the rocRAND header is not installed")
    out = str(tmp_path_factory.mktemp("philox") / "rocrand_philox")
    res = subprocess.run([hipcc, "-O1", "-o", out, SRC], capture_output=True, text=True, timeout=600)
    if res.returncode != 0:
        pytest.skip(f"could not build the rocRAND reference: {res.stderr[-500:]}")
    return out


def reference_blocks(binary, seed, row, j0, count):
    res = subprocess.run([binary, str(seed), str(row), str(j0), str(count)], capture_output=True, text=True,
                         check=True, timeout=120)
    rows = np.array([[int(x) for x in line.split()] for line in res.stdout.strip().splitlines()], dtype=np.uint64)
    assert rows.shape == (count, 5) and np.array_equal(rows[:, 0], np.arange(j0, j0 + count, dtype=np.uint64))
    return rows[:, 1:]


@pytest.mark.parametrize("seed,row,j0,count", [
    (0, 0, 0, 64),
    (0x123456789ABCDEF0, 0, 0, 64),
    (7, 5, 1000, 64),
    (2**64 - 1, 2**24 - 1, 2**32 - 64, 64),  # every key bit set; the largest row and sample words
    (1000 + 17, 3, 65536 - 32, 64),          # a bench hit-rate seed, across a sample-size boundary
])
def test_oracle_philox_matches_rocrand(ref_bin, seed, row, j0, count):
    ref = reference_blocks(ref_bin, seed, row, j0, count)
    j = np.arange(j0, j0 + count, dtype=np.uint64)
    zeros = np.zeros(count, dtype=np.uint64)
    rowv = np.full(count, row, dtype=np.uint64)
    words = philox4x32_10(j, rowv, zeros, zeros, seed & 0xFFFFFFFF, seed >> 32)
    got = np.stack([np.asarray(w, dtype=np.uint64) for w in words], axis=1)
    assert np.array_equal(got, ref), (got[:2], ref[:2])
