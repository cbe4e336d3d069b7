"""Float64 CPU oracle for the Gaussian-mixture EM E-step, M-step and top-2 assignment.

TEST INFRASTRUCTURE ONLY. This module is the slow, obviously correct
definition that the HIP kernels are checked against. Only the tests, the
smoke check and the benchmark's CPU-baseline leg may import it; the product
path never calls it. It shares no code with the HIP path.

What it follows
---------------
* "Turbo-GMM: FlashAttention-Inspired GPU-Accelerated Gaussian Mixture Model",
  abstract: EM for a Gaussian mixture scores N points against K components,
  normalises the responsibilities and accumulates sufficient statistics; the
  fused kernels are algebraically equivalent to standard EM in real
  arithmetic. The oracle therefore *is* standard EM, written out: it
  materialises the responsibility matrix (in row chunks) and sums it.
* "Flash-GMM: a memory-efficient kernel for scalable soft clustering",
  abstract: responsibilities are used to assign border vectors to several
  clusters; the oracle's ``top2`` returns each point's two most responsible
  components with their responsibilities.

Readings where the pages are silent (each also listed in the design notes):
* covariance is diagonal per component; the score is the full log-density
  including -d/2 log(2 pi) and -1/2 sum_j log var_kj;
* the M-step variance is the biased ML estimate E[x^2] - mu^2 clamped from
  below, var = max(var_hat, var_floor);
* a component whose Nk falls below EMPTY_REL * N keeps its mean and variance,
  and its log-weight becomes log(max(Nk, 1e-300) / N);
* weights are Nk / N with no renormalisation;
* top-2 ties go to the lower index, and r of each pick is normalised over all
  K components (not renormalised over the pair).

Everything is float64. fp32 and fp16 inputs are promoted exactly.
"""
from __future__ import annotations

import math

import numpy as np

LOG_2PI = math.log(2.0 * math.pi)
EMPTY_REL = 1e-12

# Rows per chunk when materialising the responsibility matrix, and the element
# budget for one (rows x components x features) difference block.
_ROW_CHUNK = 4096
_BLOCK_ELEMS = 1 << 22


def _f64(a):
    return np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------------------------
# Scores
# ---------------------------------------------------------------------------

def log_gauss_diag(X, mu, var):
    """log N(x_n | mu_k, diag(var_k)) for every (n, k), difference form.

    log N = -1/2 * sum_j [ log(2 pi var_kj) + (x_nj - mu_kj)^2 / var_kj ].
    This is the definition of the diagonal-covariance Gaussian log-density
    that the E-step scores with (Turbo-GMM abstract: "scoring N data points
    against K mixture components").
    """
    X, mu, var = _f64(X), _f64(mu), _f64(var)
    n, d = X.shape
    K = mu.shape[0]
    out = np.empty((n, K), dtype=np.float64)
    lognorm = -0.5 * (d * LOG_2PI + np.log(var).sum(axis=1))  # (K,)
    kb = max(1, _BLOCK_ELEMS // max(1, n * d))
    for k0 in range(0, K, kb):
        k1 = min(K, k0 + kb)
        diff = X[:, None, :] - mu[None, k0:k1, :]            # (n, kb, d)
        maha = (diff * diff / var[None, k0:k1, :]).sum(axis=2)
        out[:, k0:k1] = lognorm[None, k0:k1] - 0.5 * maha
    return out


def log_gauss_diag_expanded(X, mu, var):
    """The same log-density through the expansion of the square.

    sum_j (x - mu)^2 / var = sum_j x^2/var - 2 sum_j x mu/var + sum_j mu^2/var,
    evaluated with two float64 matrix products. Used only to make the oracle
    fast at large N; tests check it against the difference form.
    """
    X, mu, var = _f64(X), _f64(mu), _f64(var)
    d = X.shape[1]
    iv = 1.0 / var
    lognorm = -0.5 * (d * LOG_2PI + np.log(var).sum(axis=1))
    quad = (X * X) @ iv.T - 2.0 * (X @ (mu * iv).T) + (mu * mu * iv).sum(axis=1)[None, :]
    return lognorm[None, :] - 0.5 * quad


def component_scores(X, mu, var, logw, form="difference"):
    """s_nk = log w_k + log N(x_n | mu_k, var_k)."""
    f = log_gauss_diag if form == "difference" else log_gauss_diag_expanded
    return _f64(logw)[None, :] + f(X, mu, var)


def row_logsumexp(S):
    """l_n = m_n + log sum_k exp(s_nk - m_n), m_n = max_k s_nk.

    The responsibility normaliser (Turbo-GMM abstract: "responsibility
    normalization"); it is also the per-point log-likelihood. A row whose
    scores are all -inf gets -inf.
    """
    S = _f64(S)
    m = S.max(axis=1)
    safe = np.where(np.isfinite(m), m, 0.0)
    with np.errstate(invalid="ignore"):
        z = np.exp(S - safe[:, None]).sum(axis=1)
    with np.errstate(divide="ignore"):
        return safe + np.log(z)


def responsibilities(S, l=None):
    """r_nk = exp(s_nk - l_n); each row sums to one."""
    S = _f64(S)
    if l is None:
        l = row_logsumexp(S)
    with np.errstate(invalid="ignore"):
        return np.exp(S - l[:, None])


# ---------------------------------------------------------------------------
# E-step with sufficient statistics
# ---------------------------------------------------------------------------

def estep(X, mu, var, logw, *, form="difference", keep_R=False, row_chunk=_ROW_CHUNK, abs_x=False):
    """Standard (unfused) E-step and sufficient statistics.

    For each row chunk: scores -> row log-sum-exp -> materialised R ->
    Nk = sum_n r_nk, Sx_k = sum_n r_nk x_n, Sxx_k = sum_n r_nk x_n^2
    (elementwise square). L = sum_n l_n.

    Returns a dict with Nk (K,), Sx (K,d), Sxx (K,d), l (N,), L (scalar) and,
    if ``keep_R``, the full R (N,K); if ``abs_x``, also absx (K,d) =
    sum_n r_nk |x_n| (elementwise), the magnitude against which a sum of
    signed values such as Sx is judged.
    """
    X = _f64(X)
    mu, var, logw = _f64(mu), _f64(var), _f64(logw)
    N, d = X.shape
    K = mu.shape[0]
    Nk = np.zeros(K)
    Sx = np.zeros((K, d))
    Sxx = np.zeros((K, d))
    l_all = np.empty(N)
    R_all = np.empty((N, K)) if keep_R else None
    absx = np.zeros((K, d)) if abs_x else None
    for lo in range(0, N, row_chunk):
        hi = min(N, lo + row_chunk)
        x = X[lo:hi]
        S = component_scores(x, mu, var, logw, form)
        l = row_logsumexp(S)
        R = responsibilities(S, l)
        Nk += R.sum(axis=0)
        Sx += R.T @ x
        Sxx += R.T @ (x * x)
        if abs_x:
            absx += R.T @ np.abs(x)
        l_all[lo:hi] = l
        if keep_R:
            R_all[lo:hi] = R
    out = {"Nk": Nk, "Sx": Sx, "Sxx": Sxx, "l": l_all, "L": float(l_all.sum()) if N else 0.0}
    if keep_R:
        out["R"] = R_all
    if abs_x:
        out["absx"] = absx
    return out


def estep_rows(X, mu, var, logw, rows, *, form="difference"):
    """Per-point l_n and r_n. for a subset of rows (for sampled checks at full size)."""
    x = _f64(X)[np.asarray(rows)]
    S = component_scores(x, mu, var, logw, form)
    l = row_logsumexp(S)
    return l, responsibilities(S, l)


# ---------------------------------------------------------------------------
# M-step and the EM loop
# ---------------------------------------------------------------------------

def mstep(Nk, Sx, Sxx, N, var_floor, mu_prev, var_prev):
    """Diagonal-covariance M-step from the sufficient statistics.

    w_k = Nk / N, mu_k = Sx_k / Nk, var_k = max(Sxx_k / Nk - mu_k^2, var_floor).
    A component with Nk < EMPTY_REL * N keeps mu_prev and var_prev.
    Returns (mu, var, logw) in float64.
    """
    Nk, Sx, Sxx = _f64(Nk), _f64(Sx), _f64(Sxx)
    mu_prev, var_prev = _f64(mu_prev), _f64(var_prev)
    live = Nk >= EMPTY_REL * N
    safe = np.where(live, Nk, 1.0)
    mu = Sx / safe[:, None]
    var = np.maximum(Sxx / safe[:, None] - mu * mu, var_floor)
    mu = np.where(live[:, None], mu, mu_prev)
    var = np.where(live[:, None], var, var_prev)
    logw = np.log(np.maximum(Nk, 1e-300) / N)
    return mu, var, logw


def em(X, mu, var, logw, iters, var_floor, *, form="difference", params_dtype=np.float32):
    """``iters`` EM iterations. Returns (mu, var, logw, L_hist).

    L_hist[t] is the log-likelihood of the parameters *before* the t-th
    M-step. Parameters are rounded to ``params_dtype`` after each M-step, as
    the device stores them (pass ``np.float64`` for pure float64 EM).
    """
    N = _f64(X).shape[0]
    hist = []
    for _ in range(iters):
        e = estep(X, mu, var, logw, form=form)
        hist.append(e["L"])
        mu, var, logw = mstep(e["Nk"], e["Sx"], e["Sxx"], N, var_floor, mu, var)
        mu, var, logw = (np.asarray(a).astype(params_dtype) for a in (mu, var, logw))
    return mu, var, logw, np.array(hist)


# ---------------------------------------------------------------------------
# Top-2 assignment (border-vector multi-assignment)
# ---------------------------------------------------------------------------

def top2(X, mu, var, logw, *, form="difference", row_chunk=_ROW_CHUNK):
    """Each point's two largest-score components and their responsibilities.

    Ties go to the lower component index. r is normalised over all K. With
    K = 1 the second pick is index -1 with r = 0.
    """
    X = _f64(X)
    N = X.shape[0]
    K = np.asarray(mu).shape[0]
    idx = np.full((N, 2), -1, dtype=np.int64)
    r = np.zeros((N, 2))
    for lo in range(0, N, row_chunk):
        hi = min(N, lo + row_chunk)
        S = component_scores(X[lo:hi], mu, var, logw, form)
        l = row_logsumexp(S)
        # stable descending order: equal scores keep ascending index order
        order = np.argsort(-S, axis=1, kind="stable")
        take = min(2, K)
        idx[lo:hi, :take] = order[:, :take]
        sel = np.take_along_axis(S, order[:, :take], axis=1)
        r[lo:hi, :take] = np.exp(sel - l[:, None])
    return idx, r


# ---------------------------------------------------------------------------
# Inverted lists with border vectors (from the top-2 assignment)
# ---------------------------------------------------------------------------

def border_lists(idx, resp, K, threshold):
    """Inverted lists of a soft coarse quantizer with border vectors.

    "Flash-GMM: a memory-efficient kernel for scalable soft clustering",
    abstract: responsibilities let vectors near cluster borders be assigned
    to several clusters. Reading taken: point n is listed under its most
    responsible component idx[n, 0], and also under idx[n, 1] when
    idx[n, 1] >= 0 and resp[n, 1] >= threshold (the comparison is made on the
    float32 responsibility as given). Each list holds point indices in
    increasing order.

    Returns (offsets, members): offsets is int64 of length K + 1 (list k is
    members[offsets[k]:offsets[k + 1]]), members int64 of length offsets[K].
    """
    idx = np.asarray(idx)
    resp = np.asarray(resp, dtype=np.float32)
    N = idx.shape[0]
    n = np.arange(N, dtype=np.int64)
    prim = idx[:, 0] >= 0
    sec = (idx[:, 1] >= 0) & (resp[:, 1] >= np.float32(threshold))
    keys = np.concatenate([idx[prim, 0], idx[sec, 1]]).astype(np.int64)
    vals = np.concatenate([n[prim], n[sec]])
    order = np.lexsort((vals, keys))  # by list, then by point index
    members = vals[order]
    counts = np.bincount(keys, minlength=K)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    return offsets, members


# ---------------------------------------------------------------------------
# Lloyd's k-means (hard-assignment workload)
# ---------------------------------------------------------------------------

def kmeans_assign(X, C, *, form="difference", row_chunk=_ROW_CHUNK):
    """Nearest-centre assignment (Flash-KMeans articles: the assignment step of
    Lloyd's algorithm, an argmin over point-centre distances).

    Returns (assign, dist2): assign[n] = argmin_k ||x_n - c_k||^2 with ties to
    the lower index, dist2[n] the minimum squared distance; float64 throughout.
    form="expanded" evaluates ||x||^2 - 2 x.c + ||c||^2 with a float64 matrix
    product (the same quantity, fast enough for full-size workloads).
    """
    X, C = _f64(X), _f64(C)
    N, K = X.shape[0], C.shape[0]
    assign = np.empty(N, dtype=np.int64)
    dist2 = np.empty(N)
    cc = (C * C).sum(axis=1)
    for lo in range(0, N, row_chunk):
        hi = min(N, lo + row_chunk)
        if form == "expanded":
            x = X[lo:hi]
            D = (x * x).sum(axis=1)[:, None] - 2.0 * (x @ C.T) + cc[None, :]
        else:
            D = ((X[lo:hi, None, :] - C[None, :, :]) ** 2).sum(axis=2)
        a = np.argmin(D, axis=1)  # first minimum: ties go to the lower index
        assign[lo:hi] = a
        dist2[lo:hi] = D[np.arange(hi - lo), a]
    return assign, dist2


def kmeans_update(X, assign, C_prev):
    """Update step of Lloyd's algorithm: each centre becomes the mean of the
    points assigned to it; a centre with no points keeps its previous value
    (reading taken where the pages are silent)."""
    X = _f64(X)
    C = _f64(C_prev).copy()
    K = C.shape[0]
    counts = np.bincount(assign, minlength=K)
    sums = np.zeros_like(C)
    np.add.at(sums, assign, X)
    nz = counts > 0
    C[nz] = sums[nz] / counts[nz, None]
    return C, counts


def kmeans(X, C, iters):
    """`iters` Lloyd iterations from C; returns (C, inertia history), the
    inertia sum_n dist2[n] being that of the centres before each update."""
    hist = []
    for _ in range(iters):
        a, d2 = kmeans_assign(X, C)
        hist.append(d2.sum())
        C, _ = kmeans_update(X, a, C)
    return C, np.array(hist)
