"""GPU parity where most responsibilities are zero or negligible.

The statistics leave out responsibilities at or below rho / max(1, |x|^2)
(rho = 2^-20 / N): the single sweep per wave (a point whose responsibilities
for the wave's 32 components are all below it), the two-pass regime per
256-component slab (the second pass walks only the rows listed for each
slab). What is left out moves any statistic by at most about rho N = 2^-20.
These cases make that skip extreme: components come in groups of 32 (one
wave's slice each) whose centres are so far apart that a point's
responsibilities outside its own group underflow to exactly zero. With rows
sorted by group whole tiles belong to one group, so seven of eight waves skip
every point; shuffled rows give every wave a few points per tile (odd counts
included); K = 200 leaves the last wave with padding only. Everything is
compared with the float64 oracle at the usual bars, in both regimes; the
row lists' extremes (an empty slab, a slab of 37 rows) have a case of their
own.
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


@pytest.mark.parametrize("regime", [1, 2])
def test_statistics_skip_bound_on_negligible_responsibilities(G, regime):
    """Two blobs (std 0.5) 9.6 apart (components 0 and 1), thirty components far
    from everything (2..31, responsibilities exactly zero), and two components
    10 and 10.5 away from both blobs (32 and 33, the second wave's
    32-component slice): every point's responsibilities for 32 and 33 are
    tiny but mostly far above the fp32 underflow, so the statistics skip
    leaves the second slice out for every point. Each statistic of the GPU must then be within
    the skip's bound, 2^-20 (1 + 2E) summed over all points, plus the fp32
    accumulation of the kept mass, of the oracle's."""
    rng = np.random.default_rng(77)
    N, d, K = 50_000, 8, 34
    mu = np.zeros((K, d))
    mu[0, 0], mu[1, 0] = -4.8, 4.8
    mu[2:32] = 60.0 * np.eye(d)[2] + rng.normal(0.0, 1.0, (30, d))
    mu[32, 1], mu[33, 1] = 8.77, 9.34
    lab = rng.integers(0, 2, N)
    X = (mu[lab] + rng.normal(0.0, 0.5, (N, d))).astype(np.float32)
    mu = mu.astype(np.float32)
    var = np.ones((K, d), np.float32)
    logw = np.full(K, -np.log(K), np.float32)
    ref = oracle.estep(X, mu, var, logw, keep_R=True)
    far = ref["R"][:, 32:34]
    assert far.max() < 1e-12 and (far > 1e-40).mean() > 0.5, "premise: negligible, mostly representable"
    Nk, Sx, Sxx, L, lp = G.estep_stats(dev(X), dev(mu), dev(var), dev(logw), regime=regime,
                                        want_point_loglik=True)
    torch.cuda.synchronize()
    X64 = X.astype(np.float64)
    what = f"negligible responsibilities regime={regime}"
    parity.check_loglik_point(host(lp), ref["l"], what)
    parity.check_stats((host(Nk), host(Sx), host(Sxx)), ref, X64, ref["R"].T @ np.abs(X64), what)
    bound = 1.1 * 2.0 ** -20
    absx = ref["R"].T @ np.abs(X64)  # the fp32 accumulation of Sx scales with sum r |x|
    for key, gpu, scale in (("Nk", host(Nk), ref["Nk"]), ("Sx", host(Sx), absx), ("Sxx", host(Sxx), ref["Sxx"])):
        err = np.abs(gpu.astype(np.float64) - ref[key])
        kept = 1e-6 * np.abs(scale if scale.ndim == err.ndim else scale[:, None])
        assert (err <= bound + kept).all(), f"{what}: {key} off by {err.max():.3e}"
    # the negligible components: everything the oracle gives them is below the bound
    assert np.all(np.abs(host(Nk)[32:34] - ref["Nk"][32:34]) <= bound)
    print(f"{what}: Nk of the negligible components {host(Nk)[32:34]} (oracle {ref['Nk'][32:34]})", flush=True)


def test_normaliser_fallback_on_tied_slab_maximum(G):
    """K = 300 (two 256-component slabs in the two-pass regime) with twelve exact
    copies of one component near the data in the first slab: every row's
    largest fp32 score is shared by twelve entries, more than the first
    pass records per slab, so the merge cannot settle those rows from its
    records and the fp64 normaliser pass takes them; twelve copies in the
    second slab, below the row maxima, must not disturb anything. Against
    the oracle, element by element; the copies' responsibilities must be
    bitwise equal."""
    rng = np.random.default_rng(5)
    N, d, K = 3000, 24, 300
    mu = rng.normal(0.0, 3.0, (K, d))
    centre = rng.normal(0.0, 1.0, d)
    mu[10:22] = centre              # ties at the row maximum, first slab
    mu[270:282] = centre + 6.0      # ties below the row maximum, second slab
    var = rng.uniform(0.8, 1.5, (K, d))
    var[10:22] = 1.0
    var[270:282] = 1.0
    mu, var = mu.astype(np.float32), var.astype(np.float32)
    logw = np.full(K, -np.log(K), np.float32)
    X = (centre + rng.normal(0.0, 1.0, (N, d))).astype(np.float32)
    ref = oracle.estep(X, mu, var, logw, keep_R=True)
    args = (dev(X), dev(mu), dev(var), dev(logw))
    Nk, Sx, Sxx, L, lp = G.estep_stats(*args, regime=2, want_point_loglik=True)
    R, lr = G.estep_resp(*args, regime=2)
    torch.cuda.synchronize()
    X64 = X.astype(np.float64)
    what = "tied slab maximum, two-pass"
    parity.check_loglik_point(host(lp), ref["l"], what)
    parity.check_resp(host(R), ref["R"], what)
    parity.check_stats((host(Nk), host(Sx), host(Sxx)), ref, X64, ref["R"].T @ np.abs(X64), what)
    parity.check_total(host(L), ref, what)
    tie = host(R)[:, 10:22]
    assert np.all(tie == tie[:, :1]), "exact copies must get bitwise equal responsibilities"


def test_two_pass_row_lists_empty_and_sparse_slabs(G):
    """K = 1024 (four 256-component slabs) for the second pass's per-slab row
    lists: slab 0 near blob A (19963 rows), slab 1 far from all data (its
    list is empty, so every second-pass block of that slab has no rows),
    slab 2 near blob B (37 rows: one ragged chunk, the other blocks of the
    slab empty), slab 3 split between both blobs (every row). Against the
    oracle at the usual bars; l_n bitwise equal to the launch that also
    writes R (which walks every row of every slab)."""
    rng = np.random.default_rng(31)
    N, d, K, nb = 20_000, 16, 1024, 37
    ca, cb = np.zeros(d), 30.0 * np.eye(d)[0]
    mu = np.empty((K, d))
    mu[0:256] = ca + rng.normal(0.0, 1.5, (256, d))
    mu[256:512] = 200.0 * np.eye(d)[1] + rng.normal(0.0, 1.5, (256, d))
    mu[512:768] = cb + rng.normal(0.0, 1.5, (256, d))
    mu[768:896] = ca + rng.normal(0.0, 1.5, (128, d))
    mu[896:1024] = cb + rng.normal(0.0, 1.5, (128, d))
    lab = np.zeros(N, np.int64)
    lab[rng.choice(N, nb, replace=False)] = 1
    X = (np.where(lab[:, None] == 1, cb, ca) + rng.normal(0.0, 1.0, (N, d))).astype(np.float32)
    mu = mu.astype(np.float32)
    var = rng.uniform(0.8, 1.2, (K, d)).astype(np.float32)
    logw = np.full(K, -np.log(K), np.float32)
    ref = oracle.estep(X, mu, var, logw, keep_R=True)
    # the premise, with the statistics skip threshold 2^-20 / N / max(1, |x|^2)
    thr = 2.0 ** -20 / N / np.maximum(1.0, (X.astype(np.float64) ** 2).sum(1))
    kept = (ref["R"].reshape(N, 4, 256).max(axis=2) > thr[:, None]).sum(axis=0)
    assert kept[1] == 0 and kept[2] == nb and kept[0] == N - nb and kept[3] == N, kept
    args = (dev(X), dev(mu), dev(var), dev(logw))
    Nk, Sx, Sxx, L, lp = G.estep_stats(*args, regime=2, want_point_loglik=True)
    R, lr = G.estep_resp(*args, regime=2)
    torch.cuda.synchronize()
    X64 = X.astype(np.float64)
    what = "row lists: empty and 37-row slabs"
    parity.check_loglik_point(host(lp), ref["l"], what)
    parity.check_stats((host(Nk), host(Sx), host(Sxx)), ref, X64, ref["R"].T @ np.abs(X64), what)
    parity.check_total(host(L), ref, what)
    assert np.array_equal(host(lp), host(lr)), f"{what}: l_n differs from the R-writing launch"
    assert np.all(host(Nk)[256:512] == 0.0) and np.all(host(Sx)[256:512] == 0.0)
    print(f"{what}: kept rows per slab {kept.tolist()}, Nk of slab 2 {host(Nk)[512:768].sum():.6f} "
          f"(oracle {ref['Nk'][512:768].sum():.6f})", flush=True)
