"""Parity tolerances between the HIP path and the float64 oracle.

The target tolerance is relative 1e-4 per EM iteration (both sides start from
the same float32 parameters) and 1e-3 after T iterations (independent
trajectories from the same initial parameters).  "Relative" is made concrete
per quantity, with a scale that keeps it meaningful where a value is near 0:
  LL   |d| <= tol * |LL|
  N_k  |d| <= tol * max(N_k, 1)              (one point's worth of mass)
  pi_k |d| <= tol * max(pi_k, 1/N)
  S1   |d| <= tol * (|S1| + N_k sigma_kd + rms_d)
  S2   |d| <= tol * (|S2| + ms_d)            (ms_d = mean x_d^2: one point)
  mu   |d| <= tol * (|mu| + sigma)           components with oracle N_k >= 1
  s^2  |d| <= tol * s^2 + U * (s^2 + mu^2)  components with oracle N_k >= 1
Components whose oracle N_k < 1 are held to the N_k / pi_k rules only: their
means and variances come from fractional mass at far-away points.

The variance term U * (s^2 + mu^2), U = 1e-6 (16 float32 ulps): Eq. (3) of
the Flash-GMM paper is evaluated from S1 and S2 as s^2 = S2/N_k - mu^2, and
S2 is accumulated from float32 x^2 (the paper's 4-byte storage).  For a
component that has collapsed onto a few points (s^2 at the floor, s^2 <<
mu^2) that difference cancels to the rounding of x^2 itself, about
2^-24 mu^2, whatever the accumulation precision; the float64 oracle has no
such floor.  For well-conditioned components (mu^2 / s^2 up to about 100) U
adds at most about 1e-4 * s^2, so the tolerance stays near relative 1e-4.
"""
from __future__ import annotations

import numpy as np


def _viol(name, got, want, lim):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    err = np.abs(got - want)
    bad = err > lim
    if np.any(bad):
        i = np.unravel_index(np.argmax(err / np.maximum(lim, 1e-300)), err.shape)
        return (f"{name}: {int(bad.sum())} of {bad.size} outside tolerance; worst at {i}: "
                f"got {got[i]!r} want {want[i]!r} (|d|={err[i]:.3e}, lim={lim[i]:.3e})")
    return None


def check_stats(got, want, X_ms, X_rms, sigma, tol):
    """got/want: (Nk, S1, S2, LL); X_ms, X_rms: per-dimension mean of x^2 and
    its square root; sigma: (K, D) standard deviations of the parameters the
    E-step used.  Returns a list of violation messages."""
    Nk_g, S1_g, S2_g, ll_g = (np.asarray(a, np.float64) for a in got)
    Nk, S1, S2, ll = (np.asarray(a, np.float64) for a in want)
    out = []
    out.append(_viol("LL", np.atleast_1d(ll_g), np.atleast_1d(ll), tol * np.abs(np.atleast_1d(ll))))
    out.append(_viol("N_k", Nk_g, Nk, tol * np.maximum(Nk, 1.0)))
    out.append(_viol("S1", S1_g, S1, tol * (np.abs(S1) + Nk[:, None] * sigma + X_rms[None, :])))
    out.append(_viol("S2", S2_g, S2, tol * (np.abs(S2) + X_ms[None, :])))
    return [m for m in out if m]


VAR_ULP = 1e-6  # float32 cancellation floor of s^2 = S2/N_k - mu^2, relative to S2/N_k


def check_params(got, want, Nk_ref, N, tol):
    """got/want: (weights, means, vars) after an M-step; Nk_ref: oracle N_k."""
    w_g, mu_g, v_g = (np.asarray(a, np.float64) for a in got)
    w, mu, v = (np.asarray(a, np.float64) for a in want)
    live = np.asarray(Nk_ref) >= 1.0
    out = [_viol("pi", w_g, w, tol * np.maximum(w, 1.0 / N))]
    sd = np.sqrt(v)
    out.append(_viol("mu", mu_g[live], mu[live], tol * (np.abs(mu[live]) + sd[live])))
    out.append(_viol("var", v_g[live], v[live], tol * v[live] + VAR_ULP * (v[live] + mu[live] ** 2)))
    return [m for m in out if m]


def data_scales(X):
    x = np.asarray(X, np.float64)
    ms = np.mean(x * x, axis=0)
    return ms, np.sqrt(ms)
