"""Pins for the isotropic float64 oracle: library routines it does not call
(scipy, sklearn), closed forms, invariants and brute force.  Each ``check_*``
takes an oracle-like namespace ``o`` (the isotropic oracle or a copy with a
planted mistake) and raises AssertionError on a mismatch."""
from __future__ import annotations

import math
import statistics
import warnings

import numpy as np
from scipy import stats as sps

import oracle.gmm_oracle as diag
from soft_clustering_amd import datagen
from tests.oracle_pins import _close


def tiny_iso(seed=0, N=7, K=3, D=3):
    rng = np.random.default_rng(seed)
    X = rng.normal(0.0, 2.0, (N, D)).astype(np.float32)
    w = rng.dirichlet(np.ones(K)).astype(np.float32)
    mu = rng.normal(0.0, 1.5, (K, D)).astype(np.float32)
    v = rng.uniform(0.5, 3.0, K).astype(np.float32)
    return X, w, mu, v


def check_iso_log_joint_scipy(o):
    """log pi_k + scipy's multivariate normal log-pdf with covariance s^2 I,
    and a pure-Python product of one-dimensional densities."""
    for seed in range(3):
        X, w, mu, v = tiny_iso(seed, N=5, K=3, D=4)
        L = o.log_joint(X, w, mu, v, method="direct")
        for n in range(X.shape[0]):
            for k in range(mu.shape[0]):
                x, m, s2 = X[n].astype(np.float64), mu[k].astype(np.float64), float(v[k])
                ref = math.log(float(w[k])) + sps.multivariate_normal.logpdf(x, m, s2 * np.eye(x.shape[0]))
                p = float(w[k])
                for d in range(x.shape[0]):
                    p *= math.exp(-(x[d] - m[d]) ** 2 / (2 * s2)) / math.sqrt(2 * math.pi * s2)
                _close(L[n, k], ref, 1e-10, 1e-10, "iso log_joint vs multivariate_normal")
                _close(L[n, k], math.log(p), 1e-10, 1e-10, "iso log_joint vs brute force")


def check_iso_gemm_matches_direct(o):
    X, w, mu, v = tiny_iso(4, N=40, K=5, D=6)
    _close(o.log_joint(X, w, mu, v, method="gemm"), o.log_joint(X, w, mu, v, method="direct"), 1e-10, 1e-10,
           "iso gemm vs direct")


def check_iso_equals_diagonal_with_equal_variances(o):
    """The isotropic model is the diagonal one with sigma^2_kd = sigma^2_k for
    every d; Q_k is then the sum over d of the diagonal S2_kd."""
    X, w, mu, v = tiny_iso(6, N=60, K=4, D=5)
    vd = np.repeat(v[:, None], X.shape[1], axis=1)
    _close(o.log_joint(X, w, mu, v, method="direct"), diag.log_joint(X, w, mu, vd, method="direct"), 1e-12, 1e-12,
           "iso vs diagonal log-joint")
    Nk, S1, Q, ll = o.estep_stats(X, w, mu, v)
    Nk2, S12, S22, ll2 = diag.estep_stats(X, w, mu, vd, method="direct")
    _close(Nk, Nk2, 1e-12, 1e-12, "N_k")
    _close(S1, S12, 1e-12, 1e-12, "S1")
    _close(Q, S22.sum(axis=1), 1e-12, 1e-12, "Q vs sum_d S2")
    _close(ll, ll2, 1e-12, 0, "LL")


def check_iso_stats_invariants(o):
    """sum_k N_k = N, sum_k S1_k = sum_n x_n, sum_k Q_k = sum_n ||x_n||^2."""
    X, w, mu, v = tiny_iso(7, N=300, K=6, D=4)
    x = X.astype(np.float64)
    Nk, S1, Q, _ = o.estep_stats(X, w, mu, v)
    _close(Nk.sum(), x.shape[0], 1e-12, 0, "sum N_k")
    _close(S1.sum(axis=0), x.sum(axis=0), 1e-11, 1e-11, "sum S1")
    _close(Q.sum(), math.fsum((x * x).ravel()), 1e-12, 0, "sum Q")


def check_iso_k1_closed_form(o):
    """K=1: mu = sample mean, sigma^2 = mean over d of the population
    variance, LL(theta_1) = -(N D / 2)(log 2 pi + log sigma^2 + 1)."""
    rng = np.random.default_rng(13)
    X = (rng.normal(1.0, 2.0, (400, 3)) * np.array([1.0, 0.5, 2.0])).astype(np.float32)
    x = X.astype(np.float64)
    N, D = x.shape
    w, mu, v, hist = o.fit(X, np.ones(1), np.zeros((1, D)), np.ones(1), 2, 1e-9, store_f32=False)
    mean = np.array([math.fsum(x[:, d]) / N for d in range(D)])
    s2 = math.fsum(statistics.pvariance(x[:, d].tolist()) for d in range(D)) / D
    _close(w, [1.0], 1e-14, 0, "K=1 weight")
    _close(mu[0], mean, 1e-12, 1e-12, "K=1 mean")
    _close(v[0], s2, 1e-10, 0, "K=1 variance")
    _close(hist[1], -0.5 * N * D * (math.log(2 * math.pi) + math.log(s2) + 1.0), 1e-11, 0, "K=1 LL(theta_1)")


def check_iso_two_pass(o):
    X, w, mu, v = tiny_iso(8, N=200, K=4, D=3)
    Nk, S1, Q, _ = o.estep_stats(X, w, mu, v)
    a = o.mstep(Nk, S1, Q, X.shape[0], 1e-9, mu, v)
    b = o.mstep_two_pass(X, w, mu, v, X.shape[0], 1e-9)
    for p, q, what in zip(a, b, ("weights", "means", "variances")):
        _close(p, q, 1e-9, 1e-12, f"{what} one- vs two-pass")


def check_iso_sklearn_one_step(o):
    """One EM iteration against sklearn's GaussianMixture(spherical) from the
    same initial parameters (reg_covar=0; the floor does not bind)."""
    from sklearn.exceptions import ConvergenceWarning
    from sklearn.mixture import GaussianMixture
    K, D, N = 4, 3, 400
    mix = datagen.mixture("tiny", D, K, seed=3)
    X = datagen.sample(mix, N, seed=3).numpy()
    rng = np.random.default_rng(21)
    w0 = rng.dirichlet(np.ones(K))
    mu0 = rng.normal(0.0, 3.0, (K, D))
    v0 = rng.uniform(2.0, 6.0, K)
    w, mu, v, _ = o.fit(X, w0, mu0, v0, 1, 1e-9, store_f32=False)
    gm = GaussianMixture(n_components=K, covariance_type="spherical", reg_covar=0.0, max_iter=1, tol=0.0,
                         weights_init=w0, means_init=mu0, precisions_init=1.0 / v0, random_state=0)
    with warnings.catch_warnings():
        warnings.simplefilter("ignore", ConvergenceWarning)
        gm.fit(X.astype(np.float64))
    _close(w, gm.weights_, 1e-12, 1e-14, "weights vs sklearn")
    _close(mu, gm.means_, 1e-10, 1e-12, "means vs sklearn")
    _close(v, gm.covariances_, 1e-9, 1e-12, "variances vs sklearn")
    _, _, _, hist2 = o.fit(X, w, mu, v, 1, 1e-9, store_f32=False)
    _close(hist2[0], gm.score(X.astype(np.float64)) * N, 1e-11, 0, "LL vs sklearn score")


def check_iso_floor_and_empty(o):
    X, w, mu, v = tiny_iso(9, N=50, K=3, D=2)
    Nk, S1, Q, _ = o.estep_stats(X, w, mu, v)
    _, _, v1 = o.mstep(Nk, S1, Q, X.shape[0], 1e3, mu, v)
    _close(v1, np.full(3, 1e3), 0, 0, "floor binds")
    Nk2 = Nk.copy()
    Nk2[1] = 1e-7
    _, mu2, v2 = o.mstep(Nk2, S1, Q, X.shape[0], 1e-9, mu, v)
    _close(mu2[1], mu[1], 0, 0, "empty keeps mean")
    _close(v2[1], v[1], 0, 0, "empty keeps variance")


def check_iso_init(o):
    rng = np.random.default_rng(14)
    X = rng.normal(0.0, 3.0, (100, 5)).astype(np.float32)
    rows = np.array([3, 7, 50])
    w, mu, v = o.init(X, rows, 1e-6)
    x = X.astype(np.float64)
    _close(mu, x[rows], 0, 0, "init means")
    ref = sum(statistics.pvariance(x[:, d].tolist()) for d in range(5)) / 5
    _close(v, np.full(3, ref), 1e-12, 0, "init variance")
    _close(w, np.full(3, 1 / 3), 1e-15, 0, "init weights")


def check_iso_ll_monotone(o):
    mix = datagen.mixture("tiny", 4, 5, seed=2)
    X = datagen.sample(mix, 600, seed=2).numpy()
    w, mu, v = o.init(X, np.array([0, 100, 200, 300, 400]), 1e-6)
    _, _, _, hist = o.fit(X, w, mu, v, 8, 1e-6)
    assert np.all(np.diff(hist) >= -1e-9 * np.abs(hist[1:])), hist


ALL_CHECKS = [check_iso_log_joint_scipy, check_iso_gemm_matches_direct, check_iso_equals_diagonal_with_equal_variances,
              check_iso_stats_invariants, check_iso_k1_closed_form, check_iso_two_pass, check_iso_sklearn_one_step,
              check_iso_floor_and_empty, check_iso_init, check_iso_ll_monotone]
