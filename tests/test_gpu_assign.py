"""Soft assignment (argmax + up to m extras with r >= threshold) and its CSR
inverted lists, HIP path against the float64 oracle through the C ABI.

Both sides use the same float32 parameters (trained on the GPU for a few EM
iterations from the oracle's init, so components overlap realistically).
Rows are compared as sets of components; they must match exactly except rows
the oracle flags as boundary rows (some r within 1e-5 of the threshold, an
argmax tie within 1e-5, or a tie at the cut of the m extras)."""
import sys

import numpy as np
import pytest
import torch

import oracle.gmm_oracle as O
from soft_clustering_amd import GMM, GMMError, datagen

pytestmark = pytest.mark.gpu
DEV = "cuda"

# name: (law, N, D, K, ldx, threshold, max_extra, em_iters)
CASES = {
    "tiny": ("tiny", 4_003, 8, 16, None, 0.1, 3, 3),
    "odd_d5_k7": ("tiny", 1_003, 5, 7, 8, 0.05, 2, 2),
    "mid_prefix": ("mid", 5_001, 128, 1024, None, 0.1, 3, 2),
    "ivf_k16384": ("ivf", 20_011, 128, 16_384, None, 0.1, 3, 2),
    "d200_k100": ("mid", 2_005, 200, 100, None, 0.1, 3, 2),
    "embed_d768_m8": ("embed", 2_003, 768, 512, None, 0.01, 8, 1),
    "argmax_only_thr1": ("tiny", 3_001, 8, 16, None, 1.0, 3, 3),
    "argmax_only_m0": ("tiny", 3_001, 8, 16, None, 0.1, 0, 3),
    "low_thr_m8": ("tiny", 3_001, 16, 40, None, 1e-3, 8, 2),
    "fp64_logits_d200": ("mid", 2_005, 200, 100, None, 0.1, 3, 2),
    "fp64_logits_embed": ("embed", 2_003, 768, 512, None, 0.01, 8, 1),
    # the pages' multi-assignment rule (Section 4.3): the argmax plus the
    # second-best component when its responsibility exceeds tau, with tau a
    # small multiple of 1/K (r > tau and r >= tau differ only on exact ties,
    # which the boundary rule excludes)
    "top2_tau_half_over_k": ("ivf", 20_011, 128, 16_384, None, 0.5 / 16_384, 1, 2),
    "top2_tau_1_over_k": ("ivf", 20_011, 128, 16_384, None, 1.0 / 16_384, 1, 2),
    "top2_tau_2_over_k": ("ivf", 20_011, 128, 16_384, None, 2.0 / 16_384, 1, 2),
}


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(Xc, ldx):
    N, D = Xc.shape
    if ldx is None:
        return Xc.to(DEV)
    buf = torch.full((N, ldx), float("nan"), dtype=torch.float32)
    buf[:, :D] = Xc
    return buf.to(DEV)[:, :D]


def trained_params(g, Xg, Xn, K, floor, iters):
    w, mu, var = (torch.as_tensor(a.astype(np.float32)).to(DEV)
                  for a in O.init(Xn, datagen.init_rows(Xn.shape[0], K, seed=1), floor))
    if iters:
        g.fit(Xg, w, mu, var, iters, floor)
    torch.cuda.synchronize()
    return w, mu, var


def csr_rows(offsets, ids, N, width):
    """Per-row sorted component ids as an [N, width] array padded with -1,
    from CSR; also checks the CSR's own structure."""
    off = offsets.cpu().numpy()
    ids = ids.cpu().numpy().astype(np.int64)
    K = off.shape[0] - 1
    assert off[0] == 0 and np.all(np.diff(off) >= 0) and off[-1] == ids.shape[0]
    counts = np.diff(off)
    comps = np.repeat(np.arange(K), counts)
    # ids strictly ascending within each list
    if ids.shape[0] > 1:
        same = comps[1:] == comps[:-1]
        assert np.all(ids[1:][same] > ids[:-1][same]), "ids not ascending within a list"
    assert ids.min(initial=0) >= 0 and ids.max(initial=0) < N
    per_row = np.bincount(ids, minlength=N)
    assert per_row.min() >= 1 and per_row.max() <= width, "every row appears 1..1+m times"
    order = np.lexsort((comps, ids))
    r, c = ids[order], comps[order]
    start = np.searchsorted(r, np.arange(N))
    out = np.full((N, width), -1, dtype=np.int64)
    pos = np.arange(r.shape[0]) - start[r]
    out[r, pos] = c
    return out


def oracle_rows(lists, width):
    out = np.full((len(lists), width), -1, dtype=np.int64)
    for n, lst in enumerate(lists):
        s = np.sort(lst)
        out[n, : s.shape[0]] = s
    return out


def compare(gpu_rows, lists, boundary, what):
    ref = oracle_rows(lists, gpu_rows.shape[1])
    diff = np.any(gpu_rows != ref, axis=1)
    bad = np.nonzero(diff & ~boundary)[0]
    log(f"{what}: rows {gpu_rows.shape[0]}, differing {int(diff.sum())}, boundary {int(boundary.sum())}")
    assert bad.shape[0] == 0, (f"{what}: {bad.shape[0]} non-boundary rows differ, e.g. row {bad[0]}: "
                               f"gpu {gpu_rows[bad[0]]} oracle {ref[bad[0]]}")
    return int(diff.sum())


@pytest.mark.parametrize("mfma", ["split", "fp32"])
@pytest.mark.parametrize("name", list(CASES))
def test_soft_assign_parity(name, mfma):
    """mfma: split-bfloat16 first-pass logits (default, D <= 128) or fp32
    MFMA logits."""
    law, N, D, K, ldx, thr, m, iters = CASES[name]
    log(f"soft_assign parity {name} ({mfma}): N={N} D={D} K={K} thr={thr} m={m}")
    mix = datagen.mixture(law, D, K, seed=0)
    Xc = datagen.sample(mix, N, seed=0)
    Xn = Xc.numpy()
    Xg = to_dev(Xc, ldx)
    floor = 1.0 / 12.0 if law == "ivf" else (1e-5 if law == "embed" else 1e-6)
    g = GMM(K, D, DEV)
    if name.startswith("fp64_logits"):
        from soft_clustering_amd import PREC_FP64
        g.set_precision(PREC_FP64)
    w, mu, var = trained_params(g, Xg, Xn, K, floor, iters)
    if mfma == "fp32":
        from soft_clustering_amd import MFMA_FP32
        g.set_mfma(MFMA_FP32)
    offsets, ids = g.soft_assign(Xg, w, mu, var, thr, m)
    torch.cuda.synchronize()
    wn, mun, varn = (a.cpu().numpy() for a in (w, mu, var))
    method = "direct" if N * D * K <= 3e7 else "gemm"
    _, _, lists, boundary = O.soft_assign(Xn, wn, mun, varn, thr, m, method=method, chunk_rows=2048)
    gpu = csr_rows(offsets, ids, N, 1 + m)
    nd = compare(gpu, lists, boundary, name)
    if nd == 0:
        ref_off, ref_ids, _, _ = O.soft_assign(Xn, wn, mun, varn, thr, m, method=method, chunk_rows=2048)
        assert np.array_equal(offsets.cpu().numpy(), ref_off)
        assert np.array_equal(ids.cpu().numpy(), ref_ids)
    if thr >= 1.0 or m == 0:
        assert ids.shape[0] == N  # argmax only


@pytest.mark.parametrize("mfma", ["split", "fp32"])
def test_soft_assign_exact_duplicate_components(mfma):
    """Components given identical parameters have bit-identical logits on both
    sides, so every row near them holds exact responsibility ties, which the
    rule breaks by the lower index: a row that lists the higher index of a
    duplicated pair must list the lower one too, no row may list a component
    twice, and rows clear of other near-ties match the oracle exactly.  The
    pairs sit in different waves' component groups (k and k + 32, k + 96),
    in one group's two 16-component blocks (k and k + 16), and side by side
    (k and k + 1)."""
    from soft_clustering_amd import MFMA_FP32
    K, D, N = 1024, 128, 30_011
    thr, m = 0.1, 3
    mix = datagen.mixture("ivf", D, K, seed=5)
    pairs = [(7, 39), (300, 396), (512, 528), (700, 701), (900, 932)]
    means, stds = mix.means.copy(), mix.stds.copy()
    for a, b in pairs:
        means[b], stds[b] = means[a], stds[a]
    mix = datagen.Mixture(np.full(K, 1.0 / K), means, stds, "ivf")
    Xc = datagen.sample(mix, N, seed=5)
    Xg = Xc.to(DEV)
    w = np.full(K, 1.0 / K, np.float32)
    mu, var = means.astype(np.float32), (stds ** 2).astype(np.float32)
    g = GMM(K, D, DEV)
    if mfma == "fp32":
        g.set_mfma(MFMA_FP32)
    offsets, ids = g.soft_assign(Xg, *(torch.as_tensor(a).to(DEV) for a in (w, mu, var)), thr, m)
    gpu = csr_rows(offsets, ids, N, 1 + m)  # also: no row twice in a list
    for a, b in pairs:
        has_b = np.any(gpu == b, axis=1)
        assert np.all(np.any(gpu[has_b] == a, axis=1)), f"rows list {b} without its twin {a}"
        assert has_b.sum() > 0, f"no row near the pair ({a}, {b})"
    _, _, lists, boundary = O.soft_assign(Xc.numpy(), w, mu, var, thr, m, method="gemm", chunk_rows=2048)
    # exempt only near-ties other than the exact ones: rank the oracle's r
    # with each duplicate folded into its twin
    r, _ = O.responsibilities(Xc.numpy(), w, mu, var, method="gemm")
    for a, b in pairs:
        r[:, b] = 0.0
    other = O.boundary_rows(r, thr, m)
    compare(gpu, lists, other, f"duplicates ({mfma})")


@pytest.mark.parametrize("mfma", ["split", "fp32"])
@pytest.mark.parametrize("D,m", [(16, 3), (128, 1), (128, 8), (96, 2)])
def test_soft_assign_all_components_tied(D, m, mfma):
    """Every component has the same parameters, so each row's K logits are
    bit-identical on the GPU and every responsibility is exactly 1/K: the
    rule's tie-break by the lower index makes the lists {0, ..., m} for every
    row (threshold 0.5/K).  All of a row's logits then sit inside the float64
    window and clear the candidate bound, so every component group of every
    wave overflows the one-pass refinement and candidate lists (256 entries
    each) and runs the batched branches.  The oracle's lists on the same
    input agree."""
    from soft_clustering_amd import MFMA_FP32
    K, N = 512, 3_001
    thr = 0.5 / K
    rng = np.random.default_rng(11)
    X = rng.standard_normal((N, D)).astype(np.float32)
    mu = np.broadcast_to(rng.standard_normal(D).astype(np.float32), (K, D)).copy()
    var = np.full((K, D), 1.5, np.float32)
    w = np.full(K, 1.0 / K, np.float32)
    log(f"soft_assign all tied ({mfma}): N={N} D={D} K={K} m={m}")
    g = GMM(K, D, DEV)
    if mfma == "fp32":
        g.set_mfma(MFMA_FP32)
    offsets, ids = g.soft_assign(torch.as_tensor(X).to(DEV), *(torch.as_tensor(a).to(DEV) for a in (w, mu, var)),
                                 thr, m)
    gpu = csr_rows(offsets, ids, N, 1 + m)
    want = np.broadcast_to(np.arange(m + 1), (N, m + 1))
    assert np.array_equal(gpu, want), f"rows differ from {{0..{m}}}, e.g. {gpu[np.any(gpu != want, axis=1)][:1]}"
    # the oracle's plain per-component log-densities tie exactly too (its
    # BLAS path need not: a GEMM may round columns differently)
    _, _, lists, _ = O.soft_assign(X[:64], w, mu, var, thr, m, method="direct", chunk_rows=64)
    assert np.array_equal(oracle_rows(lists, 1 + m), want[:64])
    g.close()


def test_soft_assign_chunks_compose():
    """Rows past the first 2^19-row chunk: the lists of X equal the lists of
    its two halves, the second's row ids shifted, whichever way they are
    built: the default (selections kept, one stable sort of (list, row)
    pairs) and, with the assignment limit at 0, chunk by chunk (each chunk
    selected again, rows placed block by block through the list cursors)."""
    N1, N2, D, K = (1 << 19), 3_001, 16, 64
    log(f"soft_assign chunking: N={N1 + N2} D={D} K={K}")
    mix = datagen.mixture("tiny", D, K, seed=3)
    X = torch.empty(N1 + N2, D, dtype=torch.float32, device=DEV)
    datagen.sample_into(X, mix, 0, seed=3)
    g = GMM(K, D, DEV)
    Xn_small = X[:20_000].cpu().numpy()
    w, mu, var = (torch.as_tensor(a.astype(np.float32)).to(DEV)
                  for a in O.init(Xn_small, datagen.init_rows(20_000, K, seed=1), 1e-6))
    g.fit(X, w, mu, var, 2, 1e-6)
    off, ids = g.soft_assign(X, w, mu, var, 0.1, 3)
    offa, idsa = g.soft_assign(X[:N1], w, mu, var, 0.1, 3)
    offb, idsb = g.soft_assign(X[N1:], w, mu, var, 0.1, 3)
    g.set_assign_limit(0)
    offc, idsc = g.soft_assign(X, w, mu, var, 0.1, 3)
    offd, idsd = g.soft_assign(X[:N1], w, mu, var, 0.1, 3)
    off, ids, offa, idsa, offb, idsb, offc, idsc, offd, idsd = (
        t.cpu().numpy() for t in (off, ids, offa, idsa, offb, idsb, offc, idsc, offd, idsd))
    assert np.array_equal(off, offa + offb)
    for k in range(K):
        want = np.concatenate((idsa[offa[k]:offa[k + 1]], idsb[offb[k]:offb[k + 1]] + N1))
        assert np.array_equal(ids[off[k]:off[k + 1]], want), f"list {k}"
    assert np.array_equal(offc, off) and np.array_equal(idsc, ids), "chunked lists differ from the sorted ones"
    assert np.array_equal(offd, offa) and np.array_equal(idsd, idsa), "one-chunk lists differ without the sort"
    g.close()


def test_soft_assign_deterministic_and_capacity():
    law, N, D, K = "tiny", 4_003, 8, 16
    mix = datagen.mixture(law, D, K, seed=0)
    Xc = datagen.sample(mix, N, seed=0)
    Xg = Xc.to(DEV)
    g = GMM(K, D, DEV)
    w, mu, var = trained_params(g, Xg, Xc.numpy(), K, 1e-6, 2)
    o1, i1 = g.soft_assign(Xg, w, mu, var, 0.05, 3)
    o2, i2 = g.soft_assign(Xg, w, mu, var, 0.05, 3)
    assert torch.equal(o1, o2) and torch.equal(i1, i2)
    nnz = i1.shape[0]
    with pytest.raises(GMMError) as ei:
        g.soft_assign(Xg, w, mu, var, 0.05, 3, ids_capacity=nnz - 1)
    assert ei.value.status == 6 and f"nnz={nnz}" in str(ei.value)
    o3, i3 = g.soft_assign(Xg, w, mu, var, 0.05, 3, ids_capacity=nnz)
    assert torch.equal(o1, o3) and torch.equal(i1, i3)


def test_soft_assign_rejects_bad_arguments():
    g = GMM(16, 8, DEV)
    X = torch.zeros(100, 8, device=DEV)
    w = torch.full((16,), 1 / 16, device=DEV)
    mu = torch.zeros(16, 8, device=DEV)
    var = torch.ones(16, 8, device=DEV)
    for thr, m in ((0.0, 3), (1.5, 3), (0.1, -1), (0.1, 9)):
        with pytest.raises(GMMError) as ei:
            g.soft_assign(X, w, mu, var, thr, m)
        assert ei.value.status == 1


def test_soft_assign_ivf_full_size():
    """The IVF workload at its real size: K=16384 trained on a 1e6-row sample
    (3 EM iterations here), then 1e7 base rows assigned.  CSR structure is
    checked on every row; a random sample of 1500 rows is checked against the
    oracle row by row."""
    wl = datagen.WORKLOADS["ivf"]
    K, D, N = wl.K, wl.D, wl.N
    ntrain = wl.extra["train_rows"]
    thr, m = wl.extra["threshold"], wl.extra["max_extra"]
    log(f"soft_assign ivf full size: N={N} train={ntrain} K={K}")
    mix = datagen.mixture(wl.law, D, K, seed=wl.seed)
    Xt = torch.empty(ntrain, D, dtype=torch.float32, device=DEV)
    datagen.sample_into(Xt, mix, 0, seed=wl.seed, stream=1)
    g = GMM(K, D, DEV)
    w, mu, var = g.init(Xt, datagen.init_rows(ntrain, K, seed=wl.init_seed), wl.var_floor)
    g.fit(Xt, w, mu, var, 3, wl.var_floor)
    del Xt
    X = torch.empty(N, D, dtype=torch.float32, device=DEV)
    datagen.sample_into(X, mix, 0, seed=wl.seed)
    offsets, ids = g.soft_assign(X, w, mu, var, thr, m)
    torch.cuda.synchronize()
    gpu = csr_rows(offsets, ids, N, 1 + m)
    log(f"nnz {ids.shape[0]} ({ids.shape[0] / N:.3f} lists per row)")
    rng = np.random.default_rng(7)
    sample = np.sort(rng.choice(N, 1500, replace=False))
    Xs = X[torch.as_tensor(sample, device=DEV)].cpu().numpy()
    wn, mun, varn = (a.cpu().numpy() for a in (w, mu, var))
    _, _, lists, boundary = O.soft_assign(Xs, wn, mun, varn, thr, m, method="gemm", chunk_rows=256)
    compare(gpu[sample], lists, boundary, "ivf sample")
