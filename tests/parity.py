"""Tolerance checks shared by the GPU parity tests (GPU output vs the float64 oracle).

Bars (per the E-step's accuracy targets): per-point log-likelihood 1e-4
relative, responsibilities 1e-5 absolute, Nk/Sx/Sxx 1e-4 relative. Where a
pure relative error is ill-posed the reading is:
  l_n : |dl| <= 1e-4 * max(|l|, 1)
  Nk  : |dNk| <= 1e-4 * max(Nk, 1)
  Sx  : per component, max_j |dSx_kj| <= 1e-4 * f_k * max_j sum_n r_nk |x_nj|   (Sx sums signed values)
  Sxx : per component, max_j |dSxx_kj| <= 1e-4 * f_k * max_j Sxx_kj
        with f_k = max(Nk, 1) / Nk: as for Nk, a component holding less than one
        point's worth of responsibility is measured against one point's worth
        (its responsibilities are each exact to an absolute, not relative, bound)
  L   : |dL| <= 1e-4 * sum_n max(|l_n|, 1)
"""
from __future__ import annotations

import numpy as np

L_TOL = 1e-4
R_TOL = 1e-5
S_TOL = 1e-4


def check_loglik_point(l_gpu, l_ref, what=""):
    l_gpu = np.asarray(l_gpu, np.float64)
    err = np.abs(l_gpu - l_ref) / np.maximum(np.abs(l_ref), 1.0)
    assert np.isfinite(l_gpu).all(), f"{what}: non-finite l"
    assert err.max() <= L_TOL, f"{what}: l_n rel err {err.max():.3e} at row {err.argmax()}"
    return float(err.max())


def check_resp(R_gpu, R_ref, what=""):
    err = np.abs(np.asarray(R_gpu, np.float64) - R_ref)
    assert err.max() <= R_TOL, f"{what}: |dr| {err.max():.3e} at {np.unravel_index(err.argmax(), err.shape)}"
    return float(err.max())


def check_stats(gpu, ref, X, R_absx=None, what=""):
    """gpu = (Nk, Sx, Sxx) arrays; ref = oracle dict; R_absx = sum_n r_nk |x_n| (K x d)."""
    Nk, Sx, Sxx = (np.asarray(a, np.float64) for a in gpu)
    eN = np.abs(Nk - ref["Nk"]) / np.maximum(ref["Nk"], 1.0)
    assert eN.max() <= S_TOL, f"{what}: Nk rel err {eN.max():.3e} at k={eN.argmax()}"
    f = np.maximum(ref["Nk"], 1.0) / np.maximum(ref["Nk"], 1e-300)
    scale_x = np.maximum(R_absx.max(axis=1) * f, 1e-30)
    eX = np.abs(Sx - ref["Sx"]).max(axis=1) / scale_x
    eX = np.where(ref["Nk"] > 0, eX, 0.0)
    assert eX.max() <= S_TOL, f"{what}: Sx normwise err {eX.max():.3e} at k={eX.argmax()}"
    scale_xx = np.maximum(ref["Sxx"].max(axis=1) * f, 1e-30)
    eXX = np.abs(Sxx - ref["Sxx"]).max(axis=1) / scale_xx
    eXX = np.where(ref["Nk"] > 0, eXX, 0.0)
    assert eXX.max() <= S_TOL, f"{what}: Sxx normwise err {eXX.max():.3e} at k={eXX.argmax()}"
    return float(eN.max()), float(eX.max()), float(eXX.max())


def check_total(L_gpu, ref, what=""):
    bound = L_TOL * np.maximum(np.abs(ref["l"]), 1.0).sum()
    assert abs(float(L_gpu) - ref["L"]) <= max(bound, 1e-9), f"{what}: L {float(L_gpu)} vs {ref['L']}"


def near_tie_rows(X, mu, var, logw, S):
    """Rows whose top-2 order or membership is within the fp32 score error bound.

    delta_n = 2 * gamma * max_k (sum_j |A_kj| x_nj^2 + |B_kj x_nj| + |c_k|),
    gamma = (2d + 2) * 2^-24 (forward error bound of an fp32 dot product of
    length 2d + 2). A row is a near-tie if the gap between its first and second,
    or second and third, largest scores is <= delta_n.
    """
    X = np.asarray(X, np.float64)
    mu = np.asarray(mu, np.float64)
    var = np.asarray(var, np.float64)
    d = X.shape[1]
    iv = 1.0 / var
    A = 0.5 * iv
    B = np.abs(mu * iv)
    c = np.abs(np.asarray(logw, np.float64) - 0.5 * (d * np.log(2 * np.pi) + np.log(var).sum(1)
                                                    + (mu * mu * iv).sum(1)))
    mag = (X * X) @ A.T + np.abs(X) @ B.T + c[None, :]
    gamma = (2 * d + 2) * 2.0 ** -24
    delta = 2 * gamma * mag.max(axis=1)
    top = -np.sort(-S, axis=1)
    g12 = top[:, 0] - top[:, 1] if S.shape[1] > 1 else np.full(len(S), np.inf)
    g23 = top[:, 1] - top[:, 2] if S.shape[1] > 2 else np.full(len(S), np.inf)
    return (g12 <= delta) | (g23 <= delta)
