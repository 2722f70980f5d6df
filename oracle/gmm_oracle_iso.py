"""Float64 CPU oracle for the isotropic-covariance Gaussian-mixture EM step.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check in
``__graft_entry__.smoke`` and the ``cpu_baseline`` leg of ``bench.py`` may import
or run this module.  The product path never calls it and shares no code with
it: plain numpy, float64, written from the method's definition.

Source: "Flash-GMM: A Memory-Efficient Kernel for Scalable Soft Clustering",
Section 2, with the pages' own covariance model Sigma_k = sigma^2_k I (one
variance per component):
  * log z_nk = log pi_k - (D/2) log(2 pi sigma^2_k) - ||x_n - mu_k||^2 / (2 sigma^2_k),
    normalised with log-sum-exp over k (responsibilities r_nk);
  * M-step Eqs. (1)-(3): pi_k = N_k / N, mu_k = sum_n r_nk x_n / N_k and the
    variance from r-weighted squared deviations about the new mean, averaged
    over the D dimensions: sigma^2_k = sum_n r_nk ||x_n - mu_k||^2 / (D N_k).
Statistics carried between the E-step and the M-step: N_k, S1_k = sum_n r_nk x_n
and the scalar Q_k = sum_n r_nk ||x_n||^2, so that
sigma^2_k = (Q_k / N_k - ||mu_k||^2) / D.
Readings (as for the diagonal model): variance floor f applied after every
M-step and at initialisation; components with N_k < 1e-6 keep their previous
mean and variance; LL(theta_t) belongs to the parameters entering iteration
t; parameters are stored in float32 between iterations.  Initialisation:
means are K given rows, every component's variance is the mean over the
dimensions of the population (ddof 0) per-dimension variance, floored.
"""
from __future__ import annotations

import math

import numpy as np

LOG_2PI = math.log(2.0 * math.pi)
EMPTY_NK = 1e-6


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def log_joint(X, weights, means, var_iso, method="direct"):
    """log pi_k + log N(x_n | mu_k, sigma^2_k I) for every (n, k), (N, K).
    direct: squared distances per component; gemm: ||x||^2 - 2 x.mu + ||mu||^2
    through a matrix product (both float64)."""
    x = _f64(X)
    w, mu, v = _f64(weights), _f64(means), _f64(var_iso)
    N, D = x.shape
    K = mu.shape[0]
    with np.errstate(divide="ignore"):
        logw = np.log(w)
    const = logw - 0.5 * D * (LOG_2PI + np.log(v))
    if method == "direct":
        out = np.empty((N, K))
        for k in range(K):
            d2 = np.sum((x - mu[k]) ** 2, axis=1)
            out[:, k] = const[k] - d2 / (2.0 * v[k])
        return out
    d2 = np.sum(x * x, axis=1)[:, None] - 2.0 * (x @ mu.T) + np.sum(mu * mu, axis=1)[None, :]
    return const[None, :] - d2 / (2.0 * v[None, :])


def _logz(L):
    m = np.max(L, axis=1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    return (m + np.log(np.sum(np.exp(L - m), axis=1, keepdims=True)))[:, 0]


def estep_stats(X, weights, means, var_iso, chunk_rows=65536, method="direct"):
    """N_k, S1_k = sum r x, Q_k = sum r ||x||^2 and LL = sum log Z, over row
    chunks.  Returns (Nk (K,), S1 (K, D), Q (K,), LL)."""
    X = np.asarray(X)
    N, D = X.shape
    K = np.shape(means)[0]
    Nk, S1, Q, ll = np.zeros(K), np.zeros((K, D)), np.zeros(K), 0.0
    for s in range(0, N, chunk_rows):
        x = _f64(X[s:s + chunk_rows])
        L = log_joint(x, weights, means, var_iso, method)
        lz = _logz(L)
        r = np.exp(L - lz[:, None])
        Nk += r.sum(axis=0)
        S1 += r.T @ x
        Q += r.T @ np.sum(x * x, axis=1)
        ll += lz.sum()
    return Nk, S1, Q, ll


def mstep(Nk, S1, Q, n_total, var_floor, prev_means, prev_var):
    """pi = N_k / N, mu = S1 / N_k, sigma^2 = max((Q / N_k - ||mu||^2) / D, f);
    empty components keep mean and variance."""
    Nk, S1, Q = _f64(Nk), _f64(S1), _f64(Q)
    prev_means, prev_var = _f64(prev_means), _f64(prev_var)
    D = S1.shape[1]
    weights = Nk / float(n_total)
    live = Nk >= EMPTY_NK
    safe = np.where(live, Nk, 1.0)
    mu = S1 / safe[:, None]
    var = np.maximum((Q / safe - np.sum(mu * mu, axis=1)) / D, var_floor)
    return weights, np.where(live[:, None], mu, prev_means), np.where(live, var, prev_var)


def mstep_two_pass(X, weights, means, var_iso, n_total, var_floor):
    """Eq. (3) literally: the new mean, then sum r ||x - mu_new||^2 / (D N_k)."""
    x = _f64(X)
    L = log_joint(x, weights, means, var_iso)
    r = np.exp(L - _logz(L)[:, None])
    Nk = r.sum(axis=0)
    mu = (r.T @ x) / Nk[:, None]
    D = x.shape[1]
    var = np.array([np.sum(r[:, k] * np.sum((x - mu[k]) ** 2, axis=1)) / (D * Nk[k]) for k in range(mu.shape[0])])
    return Nk / float(n_total), mu, np.maximum(var, var_floor)


def fit(X, weights, means, var_iso, iters, var_floor, method="direct", store_f32=True):
    """iters EM iterations; returns (weights, means, var_iso, ll_hist)."""
    w, mu, v = _f64(weights), _f64(means), _f64(var_iso)
    N = np.shape(X)[0]
    hist = []
    for _ in range(int(iters)):
        Nk, S1, Q, ll = estep_stats(X, w, mu, v, method=method)
        hist.append(ll)
        w, mu, v = mstep(Nk, S1, Q, N, var_floor, mu, v)
        if store_f32:
            w, mu, v = (_f64(a.astype(np.float32)) for a in (w, mu, v))
    return w, mu, v, np.array(hist)


def init(X, rows, var_floor):
    """Means are the given rows; every variance is the mean over dimensions of
    the population per-dimension variance, floored; weights 1/K."""
    x = _f64(X)
    rows = np.asarray(rows, dtype=np.int64)
    K = rows.shape[0]
    v = max(float(np.mean(np.var(x, axis=0))), var_floor)
    return np.full(K, 1.0 / K), x[rows].copy(), np.full(K, v)
