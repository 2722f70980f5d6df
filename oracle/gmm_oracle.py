"""Float64 CPU oracle for the diagonal-covariance Gaussian-mixture EM step.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check in
``__graft_entry__.smoke`` and the ``cpu_baseline`` leg of ``bench.py`` may import
or run this module.  The product path (the HIP library and its Python binding)
never calls it, and it shares no code with that path: plain numpy, float64,
written from the method's definition.

Source of every formula: "Flash-GMM: A Memory-Efficient Kernel for Scalable
Soft Clustering" (Bloch, Gera, Orbach, Eytan, Toledo, arXiv 2606.10896):
  * Section 2 - the mixture density p(x|Theta) = sum_k pi_k N(x | mu_k, Sigma_k),
    the data log-likelihood sum_i log sum_k pi_k N_ik, the E-step
    responsibilities r_ik = z_ik / sum_j z_ij with z_ik = pi_k N_ik computed in
    log space with log-sum-exp, and the M-step Eqs. (1)-(3):
    N_k = sum_i r_ik, pi_k = N_k / N, mu_k = (1/N_k) sum_i r_ik x_i and the
    variance from r-weighted squared deviations about the *new* mean.
  * Section 4.2 - hard assignment to the highest-responsibility component;
    Section 4.3 - multi-assignment of a vector to further components whose
    responsibility clears a threshold.
Readings taken where the pages are silent or differ from the interface built
here (each also listed with its reason in the design notes):
  * Covariance is diagonal, sigma^2_kd, not the pages' isotropic sigma^2_k I;
    Eq. (3) is applied per dimension: sigma^2_kd = sum_i r_ik (x_id - mu_kd)^2 / N_k.
  * pi_k = N_k / N with N the number of rows (Eq. (1)), not N_k / sum N_k'.
  * After each M-step every variance is clamped from below by a floor f.
  * A component with N_k < EMPTY_NK keeps its previous mean and variances.
  * LL(theta_t) is the log-likelihood of the parameters *entering* iteration t.
  * Parameters are stored in float32 between iterations, as the library stores
    them; every arithmetic step is float64.
  * Soft assignment: the argmax component (lowest index on ties) plus up to m
    further components with r >= threshold, ranked by r descending then index
    ascending; inverted lists in CSR form with row ids ascending in each list.
  * Initialisation: means are K given rows, every component gets the
    population (ddof 0) per-dimension variance of the data, floored, and
    weights 1/K.
"""
from __future__ import annotations

import math

import numpy as np

LOG_2PI = math.log(2.0 * math.pi)
EMPTY_NK = 1e-6          # below this effective count a component keeps mu, sigma^2
DIRECT_MAX_WORK = 4e8    # N*K*D up to which log_joint uses the direct form by default


def _f64(a):
    return np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------------- log-densities
def log_joint_direct(X, weights, means, variances):
    """l_nk = log pi_k + log N(x_n | mu_k, diag sigma^2_k), the direct form:
    log pi_k - 1/2 sum_d (x_nd - mu_kd)^2 / sigma^2_kd - 1/2 sum_d log sigma^2_kd - D/2 log 2pi.
    (Section 2, mixture density with a diagonal covariance.)"""
    X, w, mu, var = _f64(X), _f64(weights), _f64(means), _f64(variances)
    N, D = X.shape
    K = mu.shape[0]
    with np.errstate(divide="ignore"):
        logw = np.log(w)
    half_logdet = 0.5 * np.sum(np.log(var), axis=1)
    out = np.empty((N, K))
    for k in range(K):
        maha = np.sum((X - mu[k]) ** 2 / var[k], axis=1)
        out[:, k] = logw[k] - 0.5 * maha - half_logdet[k] - 0.5 * D * LOG_2PI
    return out


def log_joint_gemm(X, weights, means, variances):
    """Same quantity as log_joint_direct, with the squared Mahalanobis term
    expanded as sum x^2/s - 2 sum x mu/s + sum mu^2/s and the two sums over d
    done by matrix products (float64).  An algebraic identity of the direct
    form, used only where the direct form would be too slow; the test suite
    checks the two against each other."""
    X, w, mu, var = _f64(X), _f64(weights), _f64(means), _f64(variances)
    D = X.shape[1]
    inv = 1.0 / var
    with np.errstate(divide="ignore"):
        logw = np.log(w)
    maha = (X * X) @ inv.T - 2.0 * (X @ (mu * inv).T) + np.sum(mu * mu * inv, axis=1)[None, :]
    const = logw - 0.5 * np.sum(np.log(var), axis=1) - 0.5 * D * LOG_2PI
    return const[None, :] - 0.5 * maha


def log_joint(X, weights, means, variances, method="auto"):
    X = np.asarray(X)
    if method == "auto":
        method = "direct" if X.shape[0] * np.shape(means)[0] * X.shape[1] <= DIRECT_MAX_WORK else "gemm"
    if method == "direct":
        return log_joint_direct(X, weights, means, variances)
    if method == "gemm":
        return log_joint_gemm(X, weights, means, variances)
    raise ValueError(method)


# ---------------------------------------------------------------- E-step
def log_normaliser(L):
    """log Z_n = m_n + log sum_k exp(l_nk - m_n), m_n = max_k l_nk (log-sum-exp,
    Section 2)."""
    m = np.max(L, axis=1, keepdims=True)
    return (m + np.log(np.sum(np.exp(L - m), axis=1, keepdims=True)))[:, 0]


def responsibilities(X, weights, means, variances, method="auto"):
    """r_nk = exp(l_nk - log Z_n) and log Z_n (Section 2, E-step)."""
    L = log_joint(X, weights, means, variances, method)
    logz = log_normaliser(L)
    return np.exp(L - logz[:, None]), logz


def estep_stats(X, weights, means, variances, chunk_rows=65536, method="auto"):
    """Sufficient statistics of one E-step, accumulated over row chunks so the
    N x K responsibility matrix never exists whole:
        N_k = sum_n r_nk,  S1_k = sum_n r_nk x_n,  S2_k = sum_n r_nk x_n^2,
        LL  = sum_n log Z_n.
    Returns (Nk (K,), S1 (K,D), S2 (K,D), LL) in float64."""
    X = np.asarray(X)
    N, D = X.shape
    K = np.shape(means)[0]
    Nk = np.zeros(K)
    S1 = np.zeros((K, D))
    S2 = np.zeros((K, D))
    ll = 0.0
    for s in range(0, N, chunk_rows):
        x = _f64(X[s:s + chunk_rows])
        r, logz = responsibilities(x, weights, means, variances, method)
        Nk += r.sum(axis=0)
        S1 += r.T @ x
        S2 += r.T @ (x * x)
        ll += logz.sum()
    return Nk, S1, S2, ll


# ---------------------------------------------------------------- M-step
def mstep(Nk, S1, S2, n_total, var_floor, prev_means, prev_vars):
    """Eqs. (1)-(3) of Section 2 with a diagonal covariance:
        pi_k = N_k / N,  mu_k = S1_k / N_k,
        sigma^2_kd = max(S2_kd / N_k - mu_kd^2, floor)
    (S2/N_k - mu^2 equals sum_n r (x - mu_new)^2 / N_k, Eq. (3) with the new
    mean).  Components with N_k < EMPTY_NK keep their previous mean and
    variances.  Returns float64 (weights, means, vars)."""
    Nk, S1, S2 = _f64(Nk), _f64(S1), _f64(S2)
    prev_means, prev_vars = _f64(prev_means), _f64(prev_vars)
    weights = Nk / float(n_total)
    live = Nk >= EMPTY_NK
    safe = np.where(live, Nk, 1.0)[:, None]
    mu = S1 / safe
    var = np.maximum(S2 / safe - mu * mu, var_floor)
    means = np.where(live[:, None], mu, prev_means)
    variances = np.where(live[:, None], var, prev_vars)
    return weights, means, variances


def mstep_two_pass(X, weights, means, variances, n_total, var_floor, method="auto"):
    """Eq. (3) literally: the new mean first, then the r-weighted squared
    deviations about it (a second pass).  Used by the tests to pin the
    one-pass S2/N_k - mu^2 form of ``mstep``."""
    X = _f64(X)
    r, _ = responsibilities(X, weights, means, variances, method)
    Nk = r.sum(axis=0)
    mu = (r.T @ X) / Nk[:, None]
    var = np.empty_like(mu)
    for k in range(mu.shape[0]):
        var[k] = (r[:, k:k + 1] * (X - mu[k]) ** 2).sum(axis=0) / Nk[k]
    return Nk / float(n_total), mu, np.maximum(var, var_floor)


# ---------------------------------------------------------------- fit
def fit(X, weights, means, variances, iters, var_floor, method="auto", store_f32=True,
        chunk_rows=65536):
    """iters EM iterations from the given parameters.  Returns
    (weights, means, vars, ll_hist) with ll_hist[t] = LL(theta_t), the
    log-likelihood of the parameters entering iteration t."""
    w, mu, var = _f64(weights), _f64(means), _f64(variances)
    N = np.shape(X)[0]
    hist = []
    for _ in range(int(iters)):
        Nk, S1, S2, ll = estep_stats(X, w, mu, var, chunk_rows, method)
        hist.append(ll)
        w, mu, var = mstep(Nk, S1, S2, N, var_floor, mu, var)
        if store_f32:
            w, mu, var = (_f64(a.astype(np.float32)) for a in (w, mu, var))
    return w, mu, var, np.array(hist)


# ---------------------------------------------------------------- init
def init(X, rows, var_floor):
    """Means are the K given rows of X; every component gets the population
    (ddof 0) variance of each dimension over all rows, floored; weights 1/K."""
    X = np.asarray(X)
    rows = np.asarray(rows, dtype=np.int64)
    K = rows.shape[0]
    means = _f64(X[rows])
    v = np.maximum(np.var(_f64(X), axis=0), var_floor)
    variances = np.broadcast_to(v, means.shape).copy()
    return np.full(K, 1.0 / K), means, variances


# ---------------------------------------------------------------- soft assignment
def assign_rows(r, threshold, max_extra):
    """Per row: the argmax component (lowest index on ties, Section 4.2) plus
    up to max_extra other components with r >= threshold ranked by r
    descending, then index ascending (Section 4.3 with the interface's rule).
    Returns a list of int arrays, one per row, argmax first."""
    out = []
    K = r.shape[1]
    idx = np.arange(K)
    for n in range(r.shape[0]):
        rn = r[n]
        top = int(np.argmax(rn))
        cand = idx[(rn >= threshold) & (idx != top)]
        order = np.lexsort((cand, -rn[cand]))  # by -r, then index
        out.append(np.concatenate(([top], cand[order][:max_extra])).astype(np.int64))
    return out


def boundary_rows(r, threshold, max_extra, eps=1e-5):
    """Rows whose list can change when responsibilities move by up to eps
    (the configured 1e-5 exemption, with the rank-tie extension of the
    scope's tolerance table).  With a the argmax and o_1 >= o_2 >= ... the
    other responsibilities of the row:
      * argmax tie: some o_i within eps of r_a (the argmax may move);
      * threshold: some o_i with i <= max_extra (a candidate whose rank keeps
        it if it clears the threshold) within eps of the threshold;
      * rank cut: o_m and o_(m+1), m = max_extra, within eps of each other,
        with o_(m+1) able to clear the threshold (o_(m+1) >= threshold - eps).
    The argmax's own responsibility is never tested against the threshold
    (the argmax is kept whatever its value), and with max_extra = 0 only the
    argmax tie counts."""
    r = np.asarray(r, dtype=np.float64)
    flags = np.zeros(r.shape[0], dtype=bool)
    m = int(max_extra)
    for n in range(r.shape[0]):
        rn = r[n]
        a = int(np.argmax(rn))
        others = np.sort(np.delete(rn, a))[::-1]
        if others.shape[0] == 0:
            continue
        if rn[a] - others[0] <= eps:
            flags[n] = True
            continue
        if m == 0:
            continue
        kept_rank = others[:m]
        if np.any(np.abs(kept_rank - threshold) <= eps):
            flags[n] = True
            continue
        if others.shape[0] > m and others[m] >= threshold - eps and others[m - 1] - others[m] <= eps:
            flags[n] = True
    return flags


def build_csr(lists, K):
    """Inverted lists from per-row component lists: offsets int64[K+1] and
    ids int32[nnz], ids ascending within each list."""
    counts = np.zeros(K, dtype=np.int64)
    for lst in lists:
        counts[lst] += 1
    offsets = np.zeros(K + 1, dtype=np.int64)
    np.cumsum(counts, out=offsets[1:])
    ids = np.empty(offsets[-1], dtype=np.int32)
    fill = offsets[:-1].copy()
    for n, lst in enumerate(lists):  # rows in ascending order
        for k in lst:
            ids[fill[k]] = n
            fill[k] += 1
    return offsets, ids


def soft_assign(X, weights, means, variances, threshold, max_extra, method="auto",
                chunk_rows=65536):
    """CSR inverted lists of the soft assignment, plus the boundary-row flags
    and the per-row lists.  Returns (offsets, ids, lists, boundary)."""
    X = np.asarray(X)
    K = np.shape(means)[0]
    lists, flags = [], []
    for s in range(0, X.shape[0], chunk_rows):
        r, _ = responsibilities(X[s:s + chunk_rows], weights, means, variances, method)
        lists.extend(assign_rows(r, threshold, max_extra))
        flags.append(boundary_rows(r, threshold, max_extra))
    offsets, ids = build_csr(lists, K)
    return offsets, ids, lists, np.concatenate(flags) if flags else np.zeros(0, bool)


def csr_to_lists(offsets, ids, N):
    """Per-row sorted component lists from CSR (for comparisons)."""
    rows = [[] for _ in range(N)]
    offsets = np.asarray(offsets)
    ids = np.asarray(ids)
    for k in range(offsets.shape[0] - 1):
        for n in ids[offsets[k]:offsets[k + 1]]:
            rows[int(n)].append(k)
    return [np.array(sorted(r), dtype=np.int64) for r in rows]
