"""Seeded synthetic inputs for the Gaussian-mixture E-step.

This module only draws numbers: blob data X and the starting mixture
parameters (mu, var, logw). It holds none of the EM arithmetic, so the float64
oracle and the HIP path can both be fed from it without sharing any code.

The workloads are the five blob configurations the mixture-model pages are
benchmarked on (Gaussian blobs, diagonal covariance, K components, d features),
re-drawn here because the pages name no dataset:

  tiny    N=4096      d=16  K=8     centres ~N(0, 9 I), per-dim std ~U(0.5, 1.5), equal weights
  ref     N=1048576   d=128 K=256   centres ~N(0, 4 I), std 1, Dirichlet(1) weights
  smallk  N=16777216  d=32  K=16    centres ~N(0, 16 I), per-dim std ~U(0.3, 2.0), equal weights
  largek  N=4194304   d=128 K=4096  centres ~N(0, I), std 0.25, equal weights
  ivf     N=10000000  d=96  K=1024  unit-norm centres + N(0, 0.05^2 I) noise, rows renormalised, X in fp16

Draw order (PCG64 via numpy.random.default_rng(seed)): centres, per-blob std,
mixing weights, labels, noise in fixed 2**20-row chunks, then the init indices.
The init is the same for every workload: mu = K distinct points drawn uniformly
without replacement, var = 1, logw = -log K.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

CHUNK_ROWS = 1 << 20


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    N: int
    d: int
    K: int
    seed: int
    x_dtype: str  # "f32" or "f16"


WORKLOADS = {
    "tiny": Workload("tiny", 4096, 16, 8, 0, "f32"),
    "ref": Workload("ref", 1 << 20, 128, 256, 1, "f32"),
    "smallk": Workload("smallk", 1 << 24, 32, 16, 2, "f32"),
    "largek": Workload("largek", 1 << 22, 128, 4096, 3, "f32"),
    "ivf": Workload("ivf", 10_000_000, 96, 1024, 4, "f16"),
}


def _noise_rows(rng, N, d, out_dtype, fill):
    """Fill rows [0, N) in fixed-size chunks; ``fill(lo, hi, noise)`` writes them."""
    for lo in range(0, N, CHUNK_ROWS):
        hi = min(N, lo + CHUNK_ROWS)
        fill(lo, hi, rng.standard_normal((hi - lo, d)))


def _init_params(rng, X, K):
    idx = rng.choice(X.shape[0], K, replace=False)
    mu = X[idx].astype(np.float32)
    var = np.ones_like(mu, dtype=np.float32)
    logw = np.full(K, -math.log(K), dtype=np.float32)
    return mu, var, logw


def make_workload(name: str, N: int | None = None, centre_scale: float = 1.0):
    """Draw (X, mu, var, logw) for a named workload.

    ``N`` overrides the row count (same recipe, fewer or more rows);
    ``centre_scale`` multiplies the blob centres (a low-separation stress
    variant uses 0.1). X is float32, or float16 for the "ivf" workload.
    """
    w = WORKLOADS[name]
    N = w.N if N is None else int(N)
    K_blobs, d = w.K, w.d
    rng = np.random.default_rng(w.seed)
    x_dt = np.float16 if w.x_dtype == "f16" else np.float32
    X = np.empty((N, d), dtype=x_dt)

    if name == "tiny":
        C = rng.normal(0.0, 3.0, (K_blobs, d)) * centre_scale
        S = rng.uniform(0.5, 1.5, (K_blobs, d))
        lab = rng.integers(0, K_blobs, N)

        def fill(lo, hi, z):
            X[lo:hi] = C[lab[lo:hi]] + z * S[lab[lo:hi]]
    elif name == "ref":
        C = rng.normal(0.0, 2.0, (K_blobs, d)) * centre_scale
        wts = rng.dirichlet(np.ones(K_blobs))
        lab = rng.choice(K_blobs, N, p=wts)

        def fill(lo, hi, z):
            X[lo:hi] = C[lab[lo:hi]] + z
    elif name == "smallk":
        C = rng.normal(0.0, 4.0, (K_blobs, d)) * centre_scale
        S = rng.uniform(0.3, 2.0, (K_blobs, d))
        lab = rng.integers(0, K_blobs, N)

        def fill(lo, hi, z):
            X[lo:hi] = C[lab[lo:hi]] + z * S[lab[lo:hi]]
    elif name == "largek":
        C = rng.normal(0.0, 1.0, (K_blobs, d)) * centre_scale
        lab = rng.integers(0, K_blobs, N)

        def fill(lo, hi, z):
            X[lo:hi] = C[lab[lo:hi]] + 0.25 * z
    elif name == "ivf":
        C = rng.normal(0.0, 1.0, (K_blobs, d))
        C /= np.linalg.norm(C, axis=1, keepdims=True)
        C *= centre_scale
        lab = rng.integers(0, K_blobs, N)

        def fill(lo, hi, z):
            v = C[lab[lo:hi]] + 0.05 * z
            v /= np.linalg.norm(v, axis=1, keepdims=True)
            X[lo:hi] = v  # float16 by IEEE round-to-nearest-even
    else:  # pragma: no cover
        raise KeyError(name)

    _noise_rows(rng, N, d, x_dt, fill)
    mu, var, logw = _init_params(rng, X, w.K) if N >= w.K else _init_small(rng, X, w.K)
    return X, mu, var, logw


def _init_small(rng, X, K):
    """Init for N < K (only small test shapes): indices drawn with replacement."""
    idx = rng.integers(0, X.shape[0], K)
    mu = X[idx].astype(np.float32)
    return mu, np.ones_like(mu), np.full(K, -math.log(K), dtype=np.float32)


def random_problem(seed: int, N: int, d: int, K: int, *, spread: float = 3.0,
                   var_range=(0.3, 2.0), x_dtype=np.float32):
    """A small generic problem: K blobs, random diagonal variances and weights.

    Used for edge-case shapes (ragged N, odd d, K not a tile multiple).
    The mixture parameters are drawn near, but not equal to, the blobs.
    """
    rng = np.random.default_rng(seed)
    C = rng.normal(0.0, spread, (max(K, 1), d))
    S = rng.uniform(0.5, 1.5, (max(K, 1), d))
    lab = rng.integers(0, max(K, 1), N)
    X = (C[lab] + rng.standard_normal((N, d)) * S[lab]).astype(x_dtype)
    mu = (C + rng.normal(0.0, 0.5, C.shape)).astype(np.float32)[:K]
    var = rng.uniform(var_range[0], var_range[1], (K, d)).astype(np.float32)
    w = rng.dirichlet(np.ones(K)) if K > 0 else np.zeros(0)
    logw = np.log(w).astype(np.float32)
    return X, mu, var, logw


def random_top2(seed: int, N: int, K: int, *, border_frac: float = 0.3):
    """Synthetic top-2 assignments (idx N x 2 int32, resp N x 2 float32) for the
    inverted-list build: a uniform first pick, a different uniform second
    pick (-1 when K = 1), resp[:, 0] in [0.5, 1), and resp[:, 1] drawn below
    1 - resp[:, 0], with about border_frac of the rows given a large second
    responsibility. Random numbers only; no mixture arithmetic."""
    rng = np.random.default_rng(seed)
    idx = np.empty((N, 2), dtype=np.int32)
    idx[:, 0] = rng.integers(0, K, N)
    if K > 1:
        off = rng.integers(1, K, N)
        idx[:, 1] = (idx[:, 0] + off) % K
    else:
        idx[:, 1] = -1
    r0 = rng.uniform(0.5, 1.0, N)
    big = rng.random(N) < border_frac
    r1 = np.where(big, (1.0 - r0) * rng.uniform(0.5, 1.0, N), (1.0 - r0) * rng.uniform(0.0, 0.02, N))
    if K == 1:
        r1[:] = 0.0
    resp = np.stack([r0, r1], axis=1).astype(np.float32)
    return idx, resp
