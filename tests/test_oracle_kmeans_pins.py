"""Pins for the k-means oracle (sklearn's Lloyd k-means, brute force, tie
rule, the mixture seeded from a clustering) and planted mistakes the pins
must catch.  CPU only."""
import importlib.util
import os
import warnings

import numpy as np
import pytest

import oracle.kmeans_oracle as KM
from soft_clustering_amd import datagen

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "kmeans_oracle.py")


def _data(seed=0, N=600, D=3, K=5):
    mix = datagen.mixture("tiny", D, K, seed=seed)
    X = datagen.sample(mix, N, seed=seed).numpy()
    rows = np.random.default_rng(seed + 1).choice(N, K, replace=False)
    return X, X[rows].astype(np.float64)


def check_sklearn_lloyd(o):
    """Lloyd iterations against sklearn's KMeans(algorithm="lloyd") from the
    same centres (no empty cluster arises on this data)."""
    from sklearn.cluster import KMeans
    for seed in range(3):
        X, c0 = _data(seed)
        c, counts, _ = o.lloyd(X, c0, 6, store_f32=False)
        km = KMeans(n_clusters=c0.shape[0], init=c0, n_init=1, max_iter=6, tol=0.0, algorithm="lloyd")
        with warnings.catch_warnings():
            warnings.simplefilter("ignore")
            km.fit(X.astype(np.float64))
        np.testing.assert_allclose(c, km.cluster_centers_, rtol=1e-10, atol=1e-10)
        assert counts.sum() == X.shape[0]


def check_bruteforce(o):
    """Assignment and update by explicit loops on a tiny input."""
    X, c0 = _data(4, N=40, D=2, K=3)
    a, _ = o.assign(X, c0)
    x = X.astype(np.float64)
    for n in range(x.shape[0]):
        d = [sum((x[n, j] - c0[k, j]) ** 2 for j in range(2)) for k in range(3)]
        assert a[n] == int(np.argmin(d))
    counts, c1 = o.update(X, a, c0)
    for k in range(3):
        rows = [n for n in range(x.shape[0]) if a[n] == k]
        assert counts[k] == len(rows)
        if rows:
            np.testing.assert_allclose(c1[k], np.mean(x[rows], axis=0), rtol=1e-12)


def check_ties_and_empty(o):
    """Two identical centres: the lower index takes every row; the other is
    empty and keeps its position."""
    X = np.array([[0.0, 0.0], [1.0, 0.0], [0.0, 1.0]], np.float32)
    c0 = np.array([[5.0, 5.0], [0.1, 0.1], [0.1, 0.1]])
    a, _ = o.assign(X, c0)
    assert a.tolist() == [1, 1, 1]
    counts, c1 = o.update(X, a, c0)
    assert counts.tolist() == [0.0, 3.0, 0.0]
    np.testing.assert_array_equal(c1[0], c0[0])
    np.testing.assert_array_equal(c1[2], c0[2])


def check_mixture_from_clusters(o):
    """Hand-computed example: rows (0,0), (2,0), (0,4) around the centre
    (1,2) have squared deviations 1 and 4 in every row, so variances (1, 4)
    (isotropic 2.5); the row (10,10) sits on its centre (variance 0, floored);
    a centre at (100,100) gets no rows, hence the all-rows population
    variances (17, 16.75) of the data; weights 3/4, 1/4, 0.  Then, at a
    converged clustering (every centre the mean of its rows), each cluster's
    variances are numpy's population variance of its rows."""
    X = np.array([[0, 0], [2, 0], [0, 4], [10, 10]], np.float32)
    c = np.array([[1, 2], [10, 10], [100, 100]], np.float64)
    w, mu, v = o.mixture_from_clusters(X, c, 1e-3)
    np.testing.assert_allclose(w, [0.75, 0.25, 0.0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(v, [[1.0, 4.0], [1e-3, 1e-3], [17.0, 16.75]], rtol=1e-15)
    np.testing.assert_array_equal(mu, c)
    _, _, vi = o.mixture_from_clusters(X, c, 1e-3, isotropic=True)
    np.testing.assert_allclose(vi, [2.5, 1e-3, 16.875], rtol=1e-15)
    X, c0 = _data(5, N=300, D=3, K=4)
    c, _, _ = o.lloyd(X, c0, 50, store_f32=False)
    a, _ = o.assign(X, c)
    c_mean = np.stack([X[a == k].astype(np.float64).mean(axis=0) for k in range(4)])
    np.testing.assert_allclose(c, c_mean, rtol=1e-12, atol=1e-12)  # converged
    w, _, v = o.mixture_from_clusters(X, c, 1e-9)
    for k in range(4):
        rows = X[a == k].astype(np.float64)
        np.testing.assert_allclose(w[k], rows.shape[0] / X.shape[0], rtol=1e-15)
        np.testing.assert_allclose(v[k], np.var(rows, axis=0), rtol=1e-10)


CHECKS = [check_sklearn_lloyd, check_bruteforce, check_ties_and_empty, check_mixture_from_clusters]


@pytest.mark.parametrize("check", CHECKS, ids=lambda f: f.__name__)
def test_pin(check):
    check(KM)


def _mutant(old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, old
    spec = importlib.util.spec_from_loader("kmeans_mutant", loader=None)
    mod = importlib.util.module_from_spec(spec)
    exec(compile(src.replace(old, new), "kmeans_mutant", "exec"), mod.__dict__)
    return mod


MUTATIONS = [
    ("farthest instead of nearest", "a = np.argmin(d2, axis=1)", "a = np.argmax(d2, axis=1)", check_bruteforce),
    ("ties to the highest index", "a = np.argmin(d2, axis=1)",
     "a = d2.shape[1] - 1 - np.argmin(d2[:, ::-1], axis=1)", check_ties_and_empty),
    ("sums instead of means", "sums / np.maximum(counts, 1.0)[:, None]", "sums", check_sklearn_lloyd),
    ("empty cluster moved to the origin",
     "new = np.where(counts[:, None] > 0, sums / np.maximum(counts, 1.0)[:, None], _f64(centres))",
     "new = sums / np.maximum(counts, 1.0)[:, None]", check_ties_and_empty),
    ("variance about the origin", "np.add.at(dev, a, (x - c[a]) ** 2)", "np.add.at(dev, a, x ** 2)",
     check_mixture_from_clusters),
    ("sample variance of a cluster", "dev / np.maximum(counts, 1.0)[:, None]",
     "dev / np.maximum(counts - 1.0, 1.0)[:, None]", check_mixture_from_clusters),
    ("isotropic variance summed over dimensions", "var = np.mean(var, axis=1)", "var = np.sum(var, axis=1)",
     check_mixture_from_clusters),
    ("empty cluster gets the floor", "glob = np.var(x, axis=0)", "glob = np.zeros(D)",
     check_mixture_from_clusters),
]


@pytest.mark.parametrize("desc,old,new,check", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(desc, old, new, check):
    with pytest.raises((AssertionError, ValueError)):
        check(_mutant(old, new))
