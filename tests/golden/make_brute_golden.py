"""Writes brute_small.json: exact thresholds for tiny rows.

The pages ("Fast LapSum: Exact Differentiable Top-k at Million Scale") print
no worked numeric example, so the fixtures here are computed by the oracle's
exhaustive 50-digit solve of section 2.1's eqs. (1)-(2) (oracle/brute.py),
which enumerates the set of scores above the threshold and solves the
resulting quadratic: no sorting, scanning or bisection is involved.

Run from the repository root:  python tests/golden/make_brute_golden.py
"""
import json
import os
import sys

import mpmath
import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
from oracle import brute  # noqa: E402


def main():
    g = np.random.Generator(np.random.PCG64(20260810))
    cases = []
    for n in range(1, 9):
        for t in (1e-3, 0.1, 1.0, 10.0):
            for ties in (False, True):
                if ties and n < 2:
                    continue
                r = g.standard_normal(n).astype(np.float32)
                if ties:
                    r[: max(2, n // 2)] = r[-1]
                for k in sorted({x for x in (0.5, 1.0, n / 2, n - 0.5) if 0 < x < n}):
                    b, _ = brute.solve(r, k, t)
                    cases.append({"r": [float(x) for x in r], "k": float(k), "t": t, "b": mpmath.nstr(b, 30)})
    out = {
        "source": "Fast LapSum: Exact Differentiable Top-k at Million Scale, section 2.1, eqs. (1)-(2); "
                  "values from oracle/brute.py (50-digit exhaustive solve)",
        "cases": cases,
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "brute_small.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=0)
    print(f"wrote {len(cases)} cases to {path}")


if __name__ == "__main__":
    main()
