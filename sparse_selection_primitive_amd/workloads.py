"""Seeded synthetic workloads for the LapSum soft top-k operator.

This module only draws random inputs; it holds none of the operator's
arithmetic, so the tests may feed the same arrays to the HIP library and to
the CPU oracle.  Every array is drawn with numpy's PCG64 generator in fp64
and rounded to fp32.

The shapes stand in for the uses named in "Fast LapSum: Exact Differentiable
Top-k at Million Scale": section 1 (token routing, batched short rows),
section 4.2 (the differentiable image coder's 256x256 coefficient maps and
the sparse attack's 3x1280x864 gradient maps, about 600 of 3.3M pixels), and
section 3 (a single row of 1e8 scores).  No dataset, image or trained model
is used: the value distributions are synthetic stand-ins.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass
class Workload:
    name: str
    r: np.ndarray          # fp32 [rows, n]
    g: np.ndarray          # fp32 [rows, n], upstream gradient
    k: float
    t: float
    path: str              # path the workload is meant to exercise
    meta: dict = field(default_factory=dict)

    @property
    def rows(self) -> int:
        return self.r.shape[0]

    @property
    def n(self) -> int:
        return self.r.shape[1]


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def tiny(rows: int = 8, n: int = 1024, k: float = 32, t: float = 0.1, seed: int = 101) -> Workload:
    """Plumbing case: N(0,1) scores, full-sort on-chip path."""
    r = _rng(seed).standard_normal((rows, n)).astype(np.float32)
    g = _rng(seed + 1).standard_normal((rows, n)).astype(np.float32)
    return Workload("tiny_8x1024", r, g, k, t, "lds")


def routing(rows: int = 16384, n: int = 256, k: float = 8, t: float = 0.05, seed: int = 201,
            tie_fraction: float = 0.05) -> Workload:
    """Routing-shaped batch: N(0,1) logits, plus a fraction of rows filled by
    drawing n values with replacement from 64 distinct N(0,1) values (about
    4 exact copies of each value, so ties straddle the k-th rank).  The first
    tie row is the constant 0.5."""
    r = _rng(seed).standard_normal((rows, n)).astype(np.float32)
    g = _rng(seed + 1).standard_normal((rows, n)).astype(np.float32)
    rt = _rng(seed + 2)
    n_tie = int(np.floor(tie_fraction * rows))
    tie_rows = np.sort(rt.choice(rows, size=n_tie, replace=False)) if n_tie else np.zeros(0, np.int64)
    for j, row in enumerate(tie_rows):
        if j == 0:
            r[row, :] = np.float32(0.5)
            continue
        vals = rt.standard_normal(64).astype(np.float32)
        r[row, :] = vals[rt.integers(0, 64, size=n)]
    return Workload(f"routing_{rows}x{n}", r, g, k, t, "lds", {"tie_rows": tie_rows})


def coder(rows: int = 32, n: int = 65536, k: float = 3277, t: float = 0.01, seed: int = 301) -> Workload:
    """Coder-shaped batch: |N(0,1)|^1.5 magnitudes over 256x256 maps, k = 5%."""
    r = (np.abs(_rng(seed).standard_normal((rows, n))) ** 1.5).astype(np.float32)
    g = _rng(seed + 1).standard_normal((rows, n)).astype(np.float32)
    return Workload(f"coder_{rows}x{n}", r, g, k, t, "fullsort+bracket")


def attack(n: int = 3 * 1280 * 864, k: float = 600, t: float = 1e-3, seed: int = 401) -> Workload:
    """Adversarial-perturbation-shaped single row: |Laplace(0,1)| gradient
    magnitudes (scale 1, i.e. Exp(1)) over 3x1280x864 pixels, k = 600."""
    r = np.abs(_rng(seed).laplace(0.0, 1.0, size=(1, n))).astype(np.float32)
    g = _rng(seed + 1).standard_normal((1, n)).astype(np.float32)
    return Workload(f"attack_1x{n}", r, g, k, t, "bracket")


def extreme(n: int = 100_000_000, k: float = 1e5, t: float = 1e-2, seed: int = 501,
            with_grad: bool = True) -> Workload:
    """Extreme single row: mixture 0.9 N(0,1) + 0.1 N(3, sd 0.5)."""
    rng = _rng(seed)
    r = rng.standard_normal(n)
    hi = rng.random(n) < 0.1
    r[hi] = 3.0 + 0.5 * rng.standard_normal(int(hi.sum()))
    r = r.astype(np.float32).reshape(1, n)
    if with_grad:
        g = _rng(seed + 1).standard_normal((1, n), dtype=np.float32)
    else:
        g = np.zeros((1, 0), np.float32)
    return Workload(f"extreme_1x{n}", r, g, k, t, "bracket")


def by_name(name: str, **kw) -> Workload:
    return {"tiny": tiny, "routing": routing, "coder": coder, "attack": attack, "extreme": extreme}[name](**kw)
