"""GPU parity of the border-vector inverted-list build (gmm_border_lists)
against the float64 oracle's lists: integer output, so bit-exact.

Inputs are seeded synthetic top-2 assignments (datagen.random_top2), fed to
both sides. Cases cover empty input, one point, a ragged last block, one and
two digit passes (K <= 256 and K > 256, up to the K limit), thresholds that
give no border vectors and all of them, and the IVF shape at full size. An
end-to-end case runs gmm_assign_top2 and the list build on the IVF recipe and
checks the lists against the oracle's top-2 and lists, away from near-ties.
"""
import numpy as np
import pytest

import oracle
from soft_clustering_gmm_amd import datagen
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


def _gpu_lists(G, idx, resp, K, thr):
    off, mem = G.border_lists(dev(idx), dev(resp), K, thr)
    torch.cuda.synchronize()
    off = off.cpu().numpy()
    return off, mem.cpu().numpy()[:off[-1]]


@pytest.mark.parametrize("N,K,thr", [
    (0, 5, 0.1), (1, 1, 0.1), (63, 7, 0.05), (2049, 3, 0.0), (10000, 256, 0.05), (10000, 257, 0.05),
    (100003, 1024, 0.05), (5000, 65536, 0.01), (4097, 33, 2.0), (30000, 4096, 0.1)])
def test_border_lists_bit_exact(G, N, K, thr):
    idx, resp = datagen.random_top2(N + K, N, K)
    off, mem = _gpu_lists(G, idx, resp, K, thr)
    roff, rmem = oracle.border_lists(idx, resp, K, thr)
    assert np.array_equal(off, roff), f"offsets differ (N={N} K={K})"
    assert np.array_equal(mem, rmem), f"members differ (N={N} K={K})"
    print(f"N={N} K={K} thr={thr}: {off[-1]} entries", flush=True)


def test_border_lists_full_ivf_shape(G):
    N, K = 10_000_000, 1024
    idx, resp = datagen.random_top2(11, N, K)
    off, mem = _gpu_lists(G, idx, resp, K, 0.05)
    roff, rmem = oracle.border_lists(idx, resp, K, 0.05)
    assert np.array_equal(off, roff) and np.array_equal(mem, rmem)


def test_border_lists_deterministic(G):
    idx, resp = datagen.random_top2(3, 50000, 300)
    a = _gpu_lists(G, idx, resp, 300, 0.05)
    b = _gpu_lists(G, idx, resp, 300, 0.05)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_border_lists_end_to_end_ivf(G):
    """assign_top2 + lists on the IVF recipe vs the oracle's top-2 and lists.
    Points whose top-2 is a near-tie, or whose second responsibility lies
    within the responsibility bar of the threshold, may differ; no other."""
    X, mu, var, logw = datagen.make_workload("ivf", N=6000)
    K, thr = mu.shape[0], 2e-3
    idx, resp = G.assign_top2(dev(X), dev(mu), dev(var), dev(logw))
    off, mem = G.border_lists(idx, resp, K, thr)
    torch.cuda.synchronize()
    off = off.cpu().numpy()
    mem = mem.cpu().numpy()[:off[-1]]
    ridx, rr = oracle.top2(X, mu, var, logw)
    roff, rmem = oracle.border_lists(ridx, rr.astype(np.float32), K, thr)
    S = oracle.component_scores(X, mu, var, logw)
    top = -np.sort(-S, axis=1)
    tol = 1e-9 * np.maximum(np.abs(top[:, 0]), 1.0)
    amb = ((top[:, 0] - top[:, 1]) <= tol) | ((top[:, 1] - top[:, 2]) <= tol) | (np.abs(rr[:, 1] - thr) <= parity.R_TOL)
    for k in range(K):
        a = set(mem[off[k]:off[k + 1]].tolist())
        b = set(rmem[roff[k]:roff[k + 1]].tolist())
        bad = [n for n in a ^ b if not amb[n]]
        assert not bad, f"list {k}: points {bad[:5]} differ"
    print(f"end-to-end: {off[-1]} entries for {X.shape[0]} points, {int(amb.sum())} ambiguous", flush=True)
