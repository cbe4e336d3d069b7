"""GPU parity where most responsibilities are exactly zero.

The fp32 statistics loop of the fused kernels visits, per wave, only the
points with a nonzero responsibility among the wave's 32 components (a zero
adds exactly zero). These cases make that skip extreme: components come in
groups of 32 (one wave's slice each) whose centres are so far apart that a
point's responsibilities outside its own group underflow to exactly zero.
With rows sorted by group whole tiles belong to one group, so seven of eight
waves skip every point; shuffled rows give every wave a few points per tile
(odd counts included); K = 200 leaves the last wave with padding only.
Everything is compared with the float64 oracle at the usual bars, in the
single sweep and in the second pass of the two-pass regime.
"""
import numpy as np
import pytest

import oracle
from tests import parity

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def G():
    from soft_clustering_gmm_amd import gmm
    gmm.lib()
    return gmm


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def host(t):
    return t.detach().cpu().numpy()


def _grouped(seed, N, d, K, sort_rows):
    rng = np.random.default_rng(seed)
    mu = np.zeros((K, d), np.float32)
    for k0 in range(0, K, 32):
        g = k0 // 32
        mu[k0:k0 + 32] = 60.0 * np.eye(d, dtype=np.float32)[g % d] + rng.normal(0.0, 0.7, (min(32, K - k0), d))
    var = rng.uniform(0.8, 1.2, (K, d)).astype(np.float32)
    logw = np.log(rng.dirichlet(np.ones(K))).astype(np.float32)
    lab = rng.integers(0, K, N)
    if sort_rows:
        lab = np.sort(lab)
    X = (mu[lab] + rng.normal(0.0, 1.0, (N, d))).astype(np.float32)
    return X, mu, var, logw


@pytest.mark.parametrize("regime", [1, 2])
@pytest.mark.parametrize("N,d,K,sort_rows", [(2000, 64, 256, True), (2000, 64, 256, False),
                                              (1500, 40, 200, False), (777, 128, 256, True)])
def test_stats_with_mostly_zero_responsibilities(G, regime, N, d, K, sort_rows):
    X, mu, var, logw = _grouped(900 + N + d + K, N, d, K, sort_rows)
    what = f"grouped N={N} d={d} K={K} sorted={sort_rows} regime={regime}"
    Xd, mud, vard, lwd = dev(X), dev(mu), dev(var), dev(logw)
    Nk, Sx, Sxx, L, lp = G.estep_stats(Xd, mud, vard, lwd, regime=regime, want_point_loglik=True)
    torch.cuda.synchronize()
    ref = oracle.estep(X, mu, var, logw, keep_R=True)
    # the premise: each row's nonzero responsibilities lie in one 32-component slice
    nz = ref["R"] > 0.0
    Kp = 32 * ((K + 31) // 32)
    slices = np.pad(nz, ((0, 0), (0, Kp - K))).reshape(N, Kp // 32, 32).any(axis=2).sum(axis=1)
    assert slices.max() == 1
    X64 = X.astype(np.float64)
    parity.check_loglik_point(host(lp), ref["l"], what)
    es = parity.check_stats((host(Nk), host(Sx), host(Sxx)), ref, X64, ref["R"].T @ np.abs(X64), what)
    parity.check_total(host(L), ref, what)
    print(f"{what}: stats {es[0]:.1e}/{es[1]:.1e}/{es[2]:.1e}", flush=True)
