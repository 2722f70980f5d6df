"""Float64 CPU oracle for the k-means warm start of the mixture.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check in
``__graft_entry__.smoke`` and the ``cpu_baseline`` leg of ``bench.py`` may import
or run this module; the product path never calls it and shares no code with
it.

Source: "Flash-GMM: A Memory-Efficient Kernel for Scalable Soft Clustering"
initialises its mixtures from k-means (the experimental set-up of the IVF
section); the pages give no variant, so this is Lloyd's algorithm as in any
textbook: assign every row to its nearest centre in squared Euclidean
distance, then move every centre to the mean of its rows.
Readings: ties go to the lowest centre index; a centre with no rows keeps its
position; centres are stored in float32 between iterations (as the library
stores them); every arithmetic step is float64.  The mixture built from the
clustering: weights N_k / N, means the centres, variances the population
variance of each cluster's rows about its centre (per dimension, or averaged
over dimensions for the isotropic model), floored; an empty cluster gets the
population variance of all rows.
"""
from __future__ import annotations

import numpy as np


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def assign(X, centres):
    """Index of the nearest centre of every row (lowest index on ties), and
    the squared distances to the two nearest centres (for near-tie checks)."""
    x, c = _f64(X), _f64(centres)
    d2 = np.sum(x * x, axis=1)[:, None] - 2.0 * (x @ c.T) + np.sum(c * c, axis=1)[None, :]
    a = np.argmin(d2, axis=1)
    part = np.partition(d2, 1, axis=1)[:, :2] if d2.shape[1] > 1 else np.repeat(d2, 2, axis=1)
    return a, part


def update(X, a, centres):
    """Counts and means of the rows of each cluster; empty clusters keep
    their centre."""
    x = _f64(X)
    K, D = np.shape(centres)
    counts = np.bincount(a, minlength=K).astype(np.float64)
    sums = np.zeros((K, D))
    np.add.at(sums, a, x)
    new = np.where(counts[:, None] > 0, sums / np.maximum(counts, 1.0)[:, None], _f64(centres))
    return counts, new


def lloyd(X, centres, iters, store_f32=True):
    """iters Lloyd iterations.  Returns (centres, counts of the last
    assignment, assignment history)."""
    c = _f64(centres)
    hist = []
    counts = None
    for _ in range(int(iters)):
        a, _ = assign(X, c)
        hist.append(a)
        counts, c = update(X, a, c)
        if store_f32:
            c = _f64(c.astype(np.float32))
    return c, counts, hist


def mixture_from_clusters(X, centres, var_floor, isotropic=False):
    """Weights, means and variances of the mixture seeded by a clustering
    (one final assignment to the given centres)."""
    x = _f64(X)
    N, D = x.shape
    c = _f64(centres)
    K = c.shape[0]
    a, _ = assign(x, c)
    counts = np.bincount(a, minlength=K).astype(np.float64)
    dev = np.zeros((K, D))
    np.add.at(dev, a, (x - c[a]) ** 2)
    glob = np.var(x, axis=0)
    var = np.where(counts[:, None] > 0, dev / np.maximum(counts, 1.0)[:, None], glob[None, :])
    if isotropic:
        var = np.mean(var, axis=1)
    return counts / N, c, np.maximum(var, var_floor)
