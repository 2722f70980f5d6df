"""IVF probe, exact re-rank and recall@10 over the inverted lists that
gmm_soft_assign builds: the measurement of the configured IVF workload.

The pages (Flash-GMM, Section 4.1 and Section 4.5) use the trained mixture
as a coarse quantiser: a query probes the nprobe nearest centroids, scans
the vectors of their inverted lists with exact distances and returns the
closest ones; quality is recall@10 against exact search (Table 3) and cost
the number of distance computations (DCO), which averages nprobe * N * m / K
for m lists per vector (the DCO identity of Section 4.5).  This module is
that evaluation, written with torch tensor operations on whatever device the
tensors live on (the GPU in the benchmark); it is not part of the EM path,
whose work all runs in the HIP library.

Readings (the pages leave them open):
  * probing: squared L2 distance from the query to each mean mu_k, computed
    in float64; the nprobe smallest, ties to the lower k;
  * re-rank: squared L2 distance between integer-valued float32 vectors,
    evaluated exactly (every product and partial sum is an integer below
    2^53 in float64); order by (distance, id), so ties go to the lower id;
  * a vector found through several probed lists is kept once (the same id at
    the same distance); DCO counts every scanned entry, duplicates included;
  * recall@10 = |returned top-10 and exact top-10| / 10 averaged over the
    queries (the configured definition); 1-recall@10 = the fraction of
    queries whose exact nearest neighbour is among the returned ten (the
    pages' Table 3 wording).
"""
from __future__ import annotations

import torch

ID_BITS = 25     # vector ids below 2^25
DIST_BITS = 24   # integer squared distances below 2^24 (128 dims of 0..255: < 8.4e6)


def _check_integral(X: torch.Tensor, name: str):
    if X.dtype != torch.float32 or X.dim() != 2:
        raise TypeError(f"{name} must be a 2-D float32 tensor")
    if not bool(torch.all(X == torch.round(X))):
        raise ValueError(f"{name} must hold integer values (exact distances rely on it)")


def _sqdist_f64(Q: torch.Tensor, X: torch.Tensor) -> torch.Tensor:
    """Squared L2 distances (|Q| x |X|) in float64 by the expanded form; exact
    for integer data whose squared norms stay below 2^53."""
    q = Q.to(torch.float64)
    x = X.to(torch.float64)
    return (q * q).sum(1, keepdim=True) + (x * x).sum(1)[None, :] - 2.0 * (q @ x.T)


def probe(Q: torch.Tensor, means: torch.Tensor, nprobe: int) -> torch.Tensor:
    """The nprobe nearest means of every query (float64 squared L2, ties to
    the lower index), nearest first: int64 (nq, nprobe)."""
    d = _sqdist_f64(Q, means)
    order = torch.sort(d, dim=1, stable=True).indices  # stable: equal distances keep index order
    return order[:, :nprobe]


def _keys(d2: torch.Tensor, ids: torch.Tensor) -> torch.Tensor:
    """(distance, id) packed into one int64 whose order is the lexicographic one."""
    di = torch.round(d2).to(torch.int64)
    if bool((di < 0).any()) or bool((di >= (1 << DIST_BITS)).any()):
        raise ValueError("squared distances out of the exact integer range")
    return (di << ID_BITS) | ids.to(torch.int64)


def exact_topk(Q: torch.Tensor, X: torch.Tensor, k: int = 10, batch: int = 64):
    """Brute-force top-k of every query over all rows of X by (distance, id):
    ids int64 (nq, k) and squared distances int64 (nq, k)."""
    _check_integral(Q, "Q")
    _check_integral(X, "X")
    if X.shape[0] >= (1 << ID_BITS):
        raise ValueError("too many base vectors for the id packing")
    ids_all = torch.arange(X.shape[0], device=X.device)
    out_i, out_d = [], []
    for s in range(0, Q.shape[0], batch):
        d2 = _sqdist_f64(Q[s:s + batch], X)
        key = _keys(d2, ids_all[None, :].expand_as(d2))
        del d2
        top = torch.topk(key, k, dim=1, largest=False, sorted=True).values
        out_i.append(top & ((1 << ID_BITS) - 1))
        out_d.append(top >> ID_BITS)
        del key
    return torch.cat(out_i), torch.cat(out_d)


def search(Q: torch.Tensor, X: torch.Tensor, offsets: torch.Tensor, ids: torch.Tensor, means: torch.Tensor,
           nprobe: int, k: int = 10, batch: int = 128):
    """IVF search: probe the nprobe nearest means, scan their lists with exact
    distances, drop repeated ids, return the k best by (distance, id).
    Returns ids int64 (nq, k) (-1 where fewer than k distinct vectors were
    scanned), squared distances int64 (nq, k) and the DCO of every query
    (int64: entries scanned, repeats included)."""
    _check_integral(Q, "Q")
    if X.shape[0] >= (1 << ID_BITS):
        raise ValueError("too many base vectors for the id packing")
    dev = Q.device
    sizes = offsets[1:] - offsets[:-1]
    pr = probe(Q, means, nprobe)
    nq = Q.shape[0]
    out_i = torch.full((nq, k), -1, dtype=torch.int64, device=dev)
    out_d = torch.full((nq, k), -1, dtype=torch.int64, device=dev)
    dco = sizes[pr].sum(1)
    for s in range(0, nq, batch):
        p = pr[s:s + batch]
        B = p.shape[0]
        lens = sizes[p].reshape(-1)
        starts = offsets[:-1][p].reshape(-1)
        total = int(lens.sum())
        if total == 0:
            continue
        seg = torch.repeat_interleave(torch.arange(B * nprobe, device=dev), lens)
        first = torch.cumsum(lens, 0) - lens
        pos = starts[seg] + (torch.arange(total, device=dev) - first[seg])
        cand = ids[pos].to(torch.int64)
        qi = seg // nprobe
        diff = X[cand].to(torch.float64) - Q[s:s + B][qi].to(torch.float64)
        d2 = (diff * diff).sum(1)
        del diff
        key = (qi << (ID_BITS + DIST_BITS)) | _keys(d2, cand)
        key = torch.unique(key, sorted=True)  # sorted by query, distance, id; repeats dropped
        qk = key >> (ID_BITS + DIST_BITS)
        begin = torch.searchsorted(qk, torch.arange(B, device=dev))
        end = torch.searchsorted(qk, torch.arange(B, device=dev), right=True)
        j = begin[:, None] + torch.arange(k, device=dev)[None, :]
        ok = j < end[:, None]
        sel = key[torch.where(ok, j, torch.zeros_like(j))]
        low = sel & ((1 << (ID_BITS + DIST_BITS)) - 1)
        out_i[s:s + B] = torch.where(ok, low & ((1 << ID_BITS) - 1), torch.full_like(low, -1))
        out_d[s:s + B] = torch.where(ok, low >> ID_BITS, torch.full_like(low, -1))
    return out_i, out_d, dco


def recall(found: torch.Tensor, truth: torch.Tensor):
    """(recall@k, 1-recall@k) of found ids (nq, k) against exact top-k ids."""
    k = truth.shape[1]
    hit = (found[:, :, None] == truth[:, None, :]) & (found[:, :, None] >= 0)
    r_at_k = hit.any(1).sum(1).to(torch.float64) / k
    one = (found == truth[:, :1]).any(1).to(torch.float64)
    return float(r_at_k.mean()), float(one.mean())


def dco_identity(offsets: torch.Tensor, n_rows: int, nprobe: int) -> float:
    """nprobe * N * m / K with m = nnz / N, the pages' expected DCO per query."""
    K = offsets.shape[0] - 1
    nnz = int(offsets[-1])
    return nprobe * n_rows * (nnz / n_rows) / K


__all__ = ["probe", "exact_topk", "search", "recall", "dco_identity"]
