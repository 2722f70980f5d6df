"""The IVF probe / re-rank / recall harness on the CPU, against a plain numpy
brute force written here: probed lists, returned ids and distances, DCO per
query, recall monotone in nprobe, recall 1 when every list is probed, and the
DCO identity (Flash-GMM pages, Section 4.5) where it is exact (nprobe = K)."""
import numpy as np
import torch

import oracle.gmm_oracle as O
from soft_clustering_amd import datagen, ivf_probe as ivf


def small_index(seed=0, N=3000, D=16, K=24, nq=40, thr=0.1, m=3):
    mix = datagen.mixture("ivf", D, K, seed=seed)
    X = datagen.sample_portable(mix, N, seed=seed)
    Q = datagen.sample_portable(mix, nq, seed=seed + 100)
    w, mu, var = (a.astype(np.float32) for a in (mix.weights, mix.means, mix.stds ** 2))
    off, ids, lists, _ = O.soft_assign(X, w, mu, var, thr, m, method="direct")
    return X, Q, mu, off, ids, lists


def brute_search(X, Q, mu, off, ids, nprobe, k=10):
    out_i, out_d, dco = [], [], []
    for q in Q.astype(np.float64):
        dc = np.array([np.sum((q - c) ** 2) for c in mu.astype(np.float64)])
        probed = sorted(range(len(dc)), key=lambda j: (dc[j], j))[:nprobe]
        seen = {}
        n = 0
        for j in probed:
            for v in ids[off[j]:off[j + 1]]:
                n += 1
                seen[int(v)] = float(np.sum((X[v].astype(np.float64) - q) ** 2))
        best = sorted(seen.items(), key=lambda t: (t[1], t[0]))[:k]
        out_i.append([b[0] for b in best] + [-1] * (k - len(best)))
        out_d.append([int(b[1]) for b in best] + [-1] * (k - len(best)))
        dco.append(n)
    return np.array(out_i), np.array(out_d), np.array(dco)


def brute_exact(X, Q, k=10):
    out = []
    for q in Q.astype(np.float64):
        d = np.sum((X.astype(np.float64) - q) ** 2, axis=1)
        out.append(sorted(range(X.shape[0]), key=lambda v: (d[v], v))[:k])
    return np.array(out)


def test_search_matches_brute_force():
    X, Q, mu, off, ids, _ = small_index()
    Xt, Qt, mut = torch.as_tensor(X), torch.as_tensor(Q), torch.as_tensor(mu)
    offt, idst = torch.as_tensor(off), torch.as_tensor(ids)
    for nprobe in (1, 3, 8):
        fi, fd, dco = ivf.search(Qt, Xt, offt, idst, mut, nprobe, batch=7)
        bi, bd, bdco = brute_search(X, Q, mu, off, ids, nprobe)
        np.testing.assert_array_equal(fi.numpy(), bi)
        np.testing.assert_array_equal(fd.numpy(), bd)
        np.testing.assert_array_equal(dco.numpy(), bdco)
    ti, _ = ivf.exact_topk(Qt, Xt, 10, batch=9)
    np.testing.assert_array_equal(ti.numpy(), brute_exact(X, Q))


def test_recall_monotone_and_complete():
    X, Q, mu, off, ids, _ = small_index(seed=1)
    Xt, Qt, mut = torch.as_tensor(X), torch.as_tensor(Q), torch.as_tensor(mu)
    offt, idst = torch.as_tensor(off), torch.as_tensor(ids)
    truth, _ = ivf.exact_topk(Qt, Xt)
    prev = (-1.0, -1.0)
    K = mu.shape[0]
    for nprobe in (1, 2, 4, 8, 16, K):
        fi, _, dco = ivf.search(Qt, Xt, offt, idst, mut, nprobe)
        r = ivf.recall(fi, truth)
        assert r[0] >= prev[0] and r[1] >= prev[1], "recall fell as nprobe grew"
        prev = r
    assert prev == (1.0, 1.0), "probing every list must find the exact top-10"
    # nprobe = K scans every list: DCO = nnz = nprobe * N * m / K exactly
    assert int(dco[0]) == int(off[-1])
    assert abs(ivf.dco_identity(offt, X.shape[0], K) - off[-1]) < 1e-9


def test_dco_is_the_sum_of_probed_list_sizes():
    X, Q, mu, off, ids, lists = small_index(seed=2, thr=0.05, m=2)
    Xt, Qt, mut = torch.as_tensor(X), torch.as_tensor(Q), torch.as_tensor(mu)
    _, _, dco = ivf.search(Qt, Xt, torch.as_tensor(off), torch.as_tensor(ids), mut, 5)
    pr = ivf.probe(Qt, mut, 5).numpy()
    sizes = np.diff(off)
    np.testing.assert_array_equal(dco.numpy(), sizes[pr].sum(1))
    # the identity's average over all possible probes of one list: mean list size * nprobe
    assert abs(ivf.dco_identity(torch.as_tensor(off), X.shape[0], 5) - 5 * sizes.mean()) < 1e-9
    # multi-assignment: m-bar lists per vector, so nnz = N * m-bar
    assert off[-1] == sum(len(lst) for lst in lists)


def test_duplicates_are_dropped_but_counted():
    """A vector in two probed lists is returned once and scanned twice."""
    X = np.array([[0, 0], [1, 0], [5, 5], [6, 5]], np.float32)
    mu = np.array([[0, 0], [6, 5]], np.float32)
    off = np.array([0, 3, 5], np.int64)
    ids = np.array([0, 1, 2, 2, 3], np.int32)  # vector 2 in both lists
    Q = np.array([[4, 4]], np.float32)
    fi, fd, dco = ivf.search(torch.as_tensor(Q), torch.as_tensor(X), torch.as_tensor(off), torch.as_tensor(ids),
                             torch.as_tensor(mu), 2, k=4)
    assert fi.tolist() == [[2, 3, 1, 0]]
    assert fd.tolist() == [[2, 5, 25, 32]]
    assert dco.tolist() == [5]
