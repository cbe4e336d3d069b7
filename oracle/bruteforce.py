"""Independent brute-force definitions for tiny inputs, in high precision.

TEST INFRASTRUCTURE ONLY (used to pin the float64 oracle and to write the
stored expected values under tests/golden/). Nothing here is fast, and the
product path never imports it.

The mixture is evaluated in the *linear* domain with mpmath at 50 digits:
    p(x | k) = prod_j exp(-(x_j - mu_kj)^2 / (2 var_kj)) / sqrt(2 pi var_kj)
    r_nk     = w_k p(x_n | k) / sum_k' w_k' p(x_n | k')
no logarithms, no log-sum-exp, no matrix products: a different route to the
same quantities as the oracle (the E-step of EM for a Gaussian mixture, as in
the Turbo-GMM abstract), so that a slip in either shows up as a mismatch.
"""
from __future__ import annotations

import math

import mpmath

mpmath.mp.dps = 50


def _mp(v):
    return mpmath.mpf(float(v))


def estep_linear(X, mu, var, logw):
    """Returns (R, l, Nk, Sx, Sxx, L) as nested lists of mpf (tiny inputs only)."""
    N, d, K = len(X), len(X[0]), len(mu)
    R, l = [], []
    Nk = [mpmath.mpf(0)] * K
    Sx = [[mpmath.mpf(0)] * d for _ in range(K)]
    Sxx = [[mpmath.mpf(0)] * d for _ in range(K)]
    for n in range(N):
        x = [_mp(v) for v in X[n]]
        joint = []
        for k in range(K):
            p = mpmath.exp(_mp(logw[k]))
            for j in range(d):
                v = _mp(var[k][j])
                t = x[j] - _mp(mu[k][j])
                p *= mpmath.exp(-t * t / (2 * v)) / mpmath.sqrt(2 * mpmath.pi * v)
            joint.append(p)
        tot = mpmath.fsum(joint)
        row = [p / tot for p in joint]
        R.append(row)
        l.append(mpmath.log(tot))
        for k in range(K):
            Nk[k] += row[k]
            for j in range(d):
                Sx[k][j] += row[k] * x[j]
                Sxx[k][j] += row[k] * x[j] * x[j]
    return R, l, Nk, Sx, Sxx, mpmath.fsum(l)


def top2_loop(S):
    """Two largest entries per row by a plain scan (lower index wins ties)."""
    out = []
    for row in S:
        b1 = b2 = -1
        for k, v in enumerate(row):
            if b1 < 0 or v > row[b1]:
                b2, b1 = b1, k
            elif b2 < 0 or v > row[b2]:
                b2 = k
        out.append((b1, b2))
    return out


def border_lists_loop(idx, resp, K, threshold):
    """The inverted lists by direct enumeration: list k = every n, in order,
    whose first pick is k or whose second pick is k with resp >= threshold."""
    lists = []
    for k in range(K):
        lists.append([n for n in range(len(idx))
                      if idx[n][0] == k or (idx[n][1] == k and float(resp[n][1]) >= float(threshold))])
    return lists


def kmeans_assign_loop(X, C):
    """Nearest centre by direct loops over points, centres and features."""
    assign, dist2 = [], []
    for x in X:
        best, bk = None, -1
        for k, c in enumerate(C):
            s = math.fsum((float(a) - float(b)) ** 2 for a, b in zip(x, c))
            if best is None or s < best:
                best, bk = s, k
        assign.append(bk)
        dist2.append(best)
    return assign, dist2
