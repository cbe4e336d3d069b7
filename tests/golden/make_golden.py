"""Writes the stored expected values under tests/golden/.

The inputs are tiny and drawn from a fixed seed here; the expected values come
only from oracle/bruteforce.py (50-digit mpmath, linear-domain mixture
evaluation). Run from the repository root:

    python tests/golden/make_golden.py
"""
from __future__ import annotations

import json
import os
import sys

import mpmath
import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import bruteforce  # noqa: E402


def _case(seed, N, d, K, spread):
    rng = np.random.default_rng(seed)
    X = rng.normal(0.0, spread, (N, d)).round(3)
    mu = rng.normal(0.0, spread, (K, d)).round(3)
    var = rng.uniform(0.4, 2.5, (K, d)).round(3)
    w = rng.dirichlet(np.ones(K))
    logw = np.log(w).round(6)
    return X, mu, var, logw


def _s(v):
    return mpmath.nstr(v, 30)


def write_case(name, seed, N, d, K, spread, note):
    X, mu, var, logw = _case(seed, N, d, K, spread)
    R, l, Nk, Sx, Sxx, L = bruteforce.estep_linear(X.tolist(), mu.tolist(), var.tolist(), logw.tolist())
    doc = {
        "note": note,
        "source": "oracle/bruteforce.py estep_linear (mpmath, 50 digits, linear domain)",
        "X": X.tolist(), "mu": mu.tolist(), "var": var.tolist(), "logw": logw.tolist(),
        "R": [[_s(v) for v in row] for row in R],
        "l": [_s(v) for v in l],
        "Nk": [_s(v) for v in Nk],
        "Sx": [[_s(v) for v in row] for row in Sx],
        "Sxx": [[_s(v) for v in row] for row in Sxx],
        "L": _s(L),
    }
    with open(os.path.join(HERE, name), "w") as f:
        json.dump(doc, f, indent=1)


if __name__ == "__main__":
    write_case("estep_tiny_a.json", 11, 8, 3, 3, 1.5,
               "E-step of a 3-component diagonal Gaussian mixture on 8 points in 3-D "
               "(Turbo-GMM abstract: scoring N points against K components, normalising "
               "responsibilities and accumulating sufficient statistics).")
    write_case("estep_tiny_b.json", 12, 5, 2, 2, 0.7,
               "Overlapping 2-component mixture on 5 points in 2-D (dense responsibilities).")
    print("wrote golden files to", HERE)
