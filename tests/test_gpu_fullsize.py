"""Parity at the workloads' real sizes, in the launch configuration bench.py
times (default path and precision).  The float64 oracle cannot run these
sizes whole, so each test checks

  * properties that hold at any size and pin the statistics exactly:
    sum_k N_k = N, sum_k S1_k = sum_n x_n and sum_k S2_k = sum_n x_n^2
    (they follow from sum_k r_nk = 1), computed here in float64;
  * the oracle on outputs it can compute one by one: a random sample of rows
    gathered from the full data set, with the parameters trained at full size
    (E-step statistics at 1e-4, and one M-step);
  * for the 1e6-row workload, one whole EM iteration against the oracle.
"""
import sys

import numpy as np
import pytest
import torch

import oracle.gmm_oracle as O
from soft_clustering_amd import GMM, datagen
from tests.tolerance import check_params, check_stats, data_scales

pytestmark = pytest.mark.gpu
DEV = "cuda"


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def column_sums(X, chunk=1 << 22):
    """float64 sum_n x_n, sum_n x_n^2 and sum_n |x_n| per dimension, in chunks."""
    D = X.shape[1]
    s1 = torch.zeros(D, dtype=torch.float64, device=X.device)
    s2 = torch.zeros(D, dtype=torch.float64, device=X.device)
    sa = torch.zeros(D, dtype=torch.float64, device=X.device)
    for r0 in range(0, X.shape[0], chunk):
        x = X[r0:r0 + chunk].double()
        s1 += x.sum(0)
        s2 += (x * x).sum(0)
        sa += x.abs().sum(0)
    return s1.cpu().numpy(), s2.cpu().numpy(), sa.cpu().numpy()


def check_invariants(Nk, S1, S2, X, what):
    N = X.shape[0]
    s1, s2, sa = column_sums(X)
    dn = abs(Nk.sum() - N)
    d1 = np.abs(S1.sum(0) - s1) / (sa + 1.0)
    d2 = np.abs(S2.sum(0) - s2) / (s2 + 1.0)
    log(f"{what}: |sum N_k - N| = {dn:.3g} (N={N}), max rel S1 {d1.max():.3g}, max rel S2 {d2.max():.3g}")
    # fp32 partial sums over up to 2048 rows before each float64 flush: a few
    # 1e-6 relative; a dropped term or index slip is O(1)
    assert dn <= 2e-5 * N
    assert d1.max() <= 2e-5
    assert d2.max() <= 2e-5


def sampled_oracle(g, X, w, mu, var, n, seed, what):
    """E-step statistics of n sampled rows: GPU (same kernels) vs oracle."""
    idx = np.sort(np.random.default_rng(seed).choice(X.shape[0], n, replace=False))
    Xs = X[torch.as_tensor(idx, device=DEV)].contiguous()
    got = [t.cpu().numpy() for t in g.estep_stats(Xs, w, mu, var)]
    g.check()
    Xn = Xs.cpu().numpy()
    params = tuple(a.cpu().numpy() for a in (w, mu, var))
    want = O.estep_stats(Xn, *params, method="gemm")
    ms, rms = data_scales(Xn)
    errs = check_stats((got[0], got[1], got[2], got[3][0]), want, ms, rms,
                       np.sqrt(params[2].astype(np.float64)), 1e-4)
    log(f"{what}: sampled {n} rows, {len(errs)} tolerance failures")
    assert not errs, "\n".join(errs[:10])


def trained(wl, X, iters):
    g = GMM(wl.K, wl.D, DEV)
    w, mu, var = g.init(X, datagen.init_rows(X.shape[0], wl.K, seed=wl.init_seed), wl.var_floor)
    if iters:
        g.fit(X, w, mu, var, iters, wl.var_floor)
    g.check()
    return g, w, mu, var


def test_large_1e8_rows():
    """N=1e8, D=128, K=1024 (51.2 GB of X in HBM): statistics invariants of
    one E-step after two EM iterations, and sampled rows against the oracle."""
    wl = datagen.WORKLOADS["large"]
    log(f"large: N={wl.N} D={wl.D} K={wl.K}")
    mix = datagen.mixture(wl.law, wl.D, wl.K, seed=wl.seed)
    X = torch.empty(wl.N, wl.D, dtype=torch.float32, device=DEV)
    datagen.sample_into(X, mix, 0, seed=wl.seed)
    g, w, mu, var = trained(wl, X, 2)
    Nk, S1, S2, ll = (t.cpu().numpy() for t in g.estep_stats(X, w, mu, var))
    g.check()
    assert np.isfinite(ll).all()
    check_invariants(Nk, S1, S2, X, "large")
    sampled_oracle(g, X, w, mu, var, 30_000, 11, "large")
    del X
    torch.cuda.empty_cache()


def test_mid_1e6_rows_one_iteration():
    """N=1e6, D=128, K=1024: from parameters after two GPU EM iterations, one
    full EM iteration on both sides (statistics, LL and the M-step)."""
    wl = datagen.WORKLOADS["mid"]
    log(f"mid: N={wl.N} D={wl.D} K={wl.K}")
    mix = datagen.mixture(wl.law, wl.D, wl.K, seed=wl.seed)
    X = torch.empty(wl.N, wl.D, dtype=torch.float32, device=DEV)
    datagen.sample_into(X, mix, 0, seed=wl.seed)
    g, w, mu, var = trained(wl, X, 2)
    th = tuple(a.cpu().numpy().copy() for a in (w, mu, var))
    got = [t.cpu().numpy() for t in g.estep_stats(X, w, mu, var)]
    hist = torch.zeros(1, dtype=torch.float64, device=DEV)
    g.fit(X, w, mu, var, 1, wl.var_floor, hist)
    g.check()
    Xn = X.cpu().numpy()
    check_invariants(got[0], got[1], got[2], X, "mid")
    want = O.estep_stats(Xn, *th, method="gemm")
    ms, rms = data_scales(Xn)
    errs = check_stats((got[0], got[1], got[2], got[3][0]), want, ms, rms, np.sqrt(th[2].astype(np.float64)), 1e-4)
    log(f"mid: E-step {len(errs)} tolerance failures")
    assert not errs, "\n".join(errs[:10])
    assert abs(hist.item() - want[3]) <= 1e-4 * abs(want[3])
    ref = O.mstep(*want[:3], wl.N, wl.var_floor, th[1], th[2])
    errs = check_params((w.cpu(), mu.cpu(), var.cpu()), ref, want[0], wl.N, 1e-4)
    assert not errs, "\n".join(errs[:10])


def test_ivf_training_1e6_rows_k16384():
    """IVF training sample: N=1e6, D=128, K=16384, integer data; invariants of
    one E-step after two EM iterations and sampled rows against the oracle."""
    wl = datagen.WORKLOADS["ivf"]
    n = wl.extra["train_rows"]
    log(f"ivf training: N={n} D={wl.D} K={wl.K}")
    mix = datagen.mixture(wl.law, wl.D, wl.K, seed=wl.seed)
    X = torch.empty(n, wl.D, dtype=torch.float32, device=DEV)
    datagen.sample_into(X, mix, 0, seed=wl.seed, stream=1)
    g, w, mu, var = trained(wl, X, 2)
    Nk, S1, S2, ll = (t.cpu().numpy() for t in g.estep_stats(X, w, mu, var))
    g.check()
    check_invariants(Nk, S1, S2, X, "ivf")
    sampled_oracle(g, X, w, mu, var, 4_000, 12, "ivf")


def test_embed_1e7_rows_d768_k4096():
    """Embedding-like workload: N=1e7, D=768, K=4096 (diffuse
    responsibilities); invariants of one E-step from the initial parameters
    and sampled rows against the oracle."""
    wl = datagen.WORKLOADS["embed"]
    log(f"embed: N={wl.N} D={wl.D} K={wl.K}")
    mix = datagen.mixture(wl.law, wl.D, wl.K, seed=wl.seed)
    X = torch.empty(wl.N, wl.D, dtype=torch.float32, device=DEV)
    datagen.sample_into(X, mix, 0, seed=wl.seed)
    g, w, mu, var = trained(wl, X, 0)
    Nk, S1, S2, ll = (t.cpu().numpy() for t in g.estep_stats(X, w, mu, var))
    g.check()
    check_invariants(Nk, S1, S2, X, "embed")
    sampled_oracle(g, X, w, mu, var, 1_000, 13, "embed")
    del X
    torch.cuda.empty_cache()
