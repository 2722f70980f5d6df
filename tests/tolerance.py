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
  s^2  |d| <= tol * s^2                       components with oracle N_k >= 1,
       |d| <= tol * s^2 + U * (s^2 + mu^2)  collapsed ones (below)
Components whose oracle N_k < 1 are held to the N_k / pi_k rules only: their
means and variances come from fractional mass at far-away points.

Collapsed components.  Eq. (3) of the Flash-GMM pages is evaluated from the
statistics as s^2 = S2/N_k - mu^2, and the library's statistics are
float32-grade (x^2 formed in float32, the statistics contraction exact to
float32 rounding, float32 partial sums over at most 2048 rows before each
float64 flush).  Their error is a few float32 ulps of the second moment
S2/N_k = s^2 + mu^2, whatever s^2 is.  For a component whose mass sits on a
few rows the worst case counts: x^2 rounded (1 ulp), the split product's
omitted third-order parts (2), one accumulator rounding per bfloat16 pass
(6), the same again for the S1 that gives mu^2 (twice: 18), the float64
M-step and the float32 store (< 1), so U = 32 * 2^-24.  Where s^2 is more
than 2^-10 of s^2 + mu^2 the tests hold the plain relative tolerance: the
measured error there is below 5e-6 s^2 (many rows' rounding errors do not
add up to the worst case), although U * (s^2 + mu^2) could reach 2^-9 s^2.
Where s^2 <= 2^-10 (s^2 + mu^2) (a component that has collapsed onto a few
points, s^2 often at the floor, s^2 << mu^2) the difference cancels more
than ten of the 24 bits of S2/N_k, and the slack U * (s^2 + mu^2) is added;
the float64 oracle has no such limit.
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


VAR_ULP = 32.0 * 2.0 ** -24    # float32 resolution of S2/N_k (see the module text)
COLLAPSED = 2.0 ** -10          # s^2 / (s^2 + mu^2) at or below which a component counts as collapsed


def check_params(got, want, Nk_ref, N, tol):
    """got/want: (weights, means, vars) after an M-step; Nk_ref: oracle N_k."""
    w_g, mu_g, v_g = (np.asarray(a, np.float64) for a in got)
    w, mu, v = (np.asarray(a, np.float64) for a in want)
    live = np.asarray(Nk_ref) >= 1.0
    out = [_viol("pi", w_g, w, tol * np.maximum(w, 1.0 / N))]
    sd = np.sqrt(v)
    out.append(_viol("mu", mu_g[live], mu[live], tol * (np.abs(mu[live]) + sd[live])))
    vl, ml = v[live], mu[live]
    m2 = vl + ml ** 2
    slack = np.where(vl <= COLLAPSED * m2, VAR_ULP * m2, 0.0)
    out.append(_viol("var", v_g[live], vl, tol * vl + slack))
    return [m for m in out if m]


def data_scales(X):
    x = np.asarray(X, np.float64)
    ms = np.mean(x * x, axis=0)
    return ms, np.sqrt(ms)
