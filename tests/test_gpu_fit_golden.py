"""End-to-end EM against stored float64-oracle fixtures: T iterations of
gmm_fit on the configured workloads (the mid workload in full, prefixes of
the embedding-like and IVF-training workloads), each from the same initial
parameters as the oracle's run, compared at the configured relative 1e-3:
the log-likelihood history of all T iterations, and the parameters after the
fixture's checkpoint iteration (T itself for mid and IVF; 5 of the 20 for the
embedding-like law, whose trajectory is chaotic past that).  Components
whose parameters at the checkpoint a single float32 ulp of the starting
variances moves by more than 1e-4 are left out of the parameter check (at
most 2% of them): the oracle itself rounds parameters to float32 every
iteration, so its trajectory there is not determined to 1e-3.

The fixtures (tests/golden/fit_*.npz) are written by
tests/golden/make_fit_goldens.py, which calls only the oracle; the rows are
regenerated here by datagen.sample_portable and checked against the stored
SHA-256 before anything runs on the GPU."""
import hashlib
import os
import sys

import numpy as np
import pytest
import torch

from soft_clustering_amd import datagen
from tests.tolerance import check_params

pytestmark = pytest.mark.gpu
DEV = "cuda"
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def load(name):
    z = np.load(os.path.join(GOLDEN, f"fit_{name}.npz"), allow_pickle=False)
    return {k: z[k] for k in z.files}


def worst(name, got, want, scale):
    r = np.abs(np.asarray(got, np.float64) - np.asarray(want, np.float64)) / np.maximum(scale, 1e-300)
    return f"{name} {float(r.max()):.2e}"


@pytest.mark.parametrize("name", ["mid", "embed", "ivf"])
def test_fit_matches_oracle_fixture(name):
    from soft_clustering_amd import GMM, PREC_FP64
    g0 = load(name)
    law, N, D, K, T = str(g0["law"]), int(g0["N"]), int(g0["D"]), int(g0["K"]), int(g0["T"])
    tc = int(g0["checkpoint"]) if "checkpoint" in g0 else T
    floor = float(g0["var_floor"])
    mix = datagen.mixture(law, D, K, seed=0)
    X = datagen.sample_portable(mix, N, seed=0)
    assert hashlib.sha256(X.tobytes()).hexdigest() == str(g0["sha256"]), \
        "rows regenerated on this host differ from the fixture's"
    rows = g0["init_rows"]
    # the oracle's initialisation (means: the given rows; variances: the
    # population variance of every dimension, floored; weights 1/K), in
    # float32 as both sides consumed it
    w0 = np.full(K, 1.0 / K, np.float32)
    mu0 = X[rows].copy()
    v0 = np.broadcast_to(np.maximum(np.var(X.astype(np.float64), axis=0), floor).astype(np.float32), (K, D)).copy()
    log(f"[fit-golden] {name}: N={N} D={D} K={K} T={T} parameters after {tc}")
    g = GMM(K, D)
    if name == "embed":
        g.set_precision(PREC_FP64)  # the embedding-like workload's measured setting
    Xg = torch.as_tensor(X).to(DEV)

    def fit(v_init, iters):
        w, mu, var = (torch.as_tensor(a).to(DEV) for a in (w0, mu0, v_init))
        _, _, _, hist = g.fit(Xg, w, mu, var, iters, floor)
        g.check()
        out = (w.cpu().numpy(), mu.cpu().numpy(), var.cpu().numpy())
        if iters < T:  # continue to T for the log-likelihood history
            _, _, _, h2 = g.fit(Xg, w, mu, var, T - iters, floor)
            g.check()
            hist = torch.cat([hist, h2])
        return (*out, hist.cpu().numpy())

    got_w, got_mu, got_v, hist = fit(v0, tc)
    # Conditioning of the run: the same fit from starting variances moved by
    # one float32 ulp (seeded signs).  The oracle rounds its parameters to
    # float32 at each of the T iterations, so where one such rounding of the
    # start moves a component's final parameters by more than 1e-4 (a tenth
    # of the tolerance) its trajectory is not fixed to 1e-3 by the method at
    # this precision; those components are left out of the parameter check
    # (the log-likelihood history still covers every component).
    sign = np.random.default_rng(3).choice([-1.0, 1.0], size=(K, D))
    p_w, p_mu, p_v, _ = fit((v0.astype(np.float64) * (1.0 + sign * 2.0 ** -23)).astype(np.float32), tc)
    comps = g0["comps"]
    want_w, want_mu, want_v = (g0[k].astype(np.float64) for k in ("weights", "means", "vars"))
    sd = np.sqrt(want_v)
    sens_w = np.abs(p_w - got_w) / np.maximum(want_w, 1.0 / N)     # every component
    sens = np.maximum.reduce([sens_w[comps],                         # the stored ones
                              (np.abs(p_mu - got_mu)[comps] / (np.abs(want_mu) + sd)).max(axis=1),
                              (np.abs(p_v - got_v)[comps] / want_v).max(axis=1)])
    ok, ok_w = sens <= 1e-4, sens_w <= 1e-4
    Nk_ref = want_w * N
    live = Nk_ref[comps] >= 1.0
    log(f"[fit-golden] {name}: " + ", ".join([
        worst("LL", hist, g0["loglik"], np.abs(g0["loglik"])),
        worst("pi", got_w[ok_w], want_w[ok_w], np.maximum(want_w[ok_w], 1.0 / N)),
        worst("mu", got_mu[comps][ok], want_mu[ok], np.abs(want_mu[ok]) + sd[ok]),
        worst("var", got_v[comps][ok & live], want_v[ok & live], want_v[ok & live])])
        + f"; {int((~ok & live).sum())} of {int(live.sum())} stored live components and {int((~ok_w).sum())} of "
          f"{K} weights ill-conditioned (one ulp moves them by up to {sens.max():.1e})")
    assert (~ok & live).sum() <= 0.02 * live.sum() and (~ok_w).sum() <= 0.02 * K, \
        "more than 2% of the components ill-conditioned"
    np.testing.assert_allclose(hist, g0["loglik"], rtol=1e-3)
    errs = check_params((got_w[comps][ok], got_mu[comps][ok], got_v[comps][ok]),
                        (want_w[comps][ok], want_mu[ok], want_v[ok]), Nk_ref[comps][ok], N, 1e-3)
    errs += check_params((got_w[ok_w], np.zeros((int(ok_w.sum()), 1)), np.ones((int(ok_w.sum()), 1))),
                         (want_w[ok_w], np.zeros((int(ok_w.sum()), 1)), np.ones((int(ok_w.sum()), 1))),
                         Nk_ref[ok_w], N, 1e-3)
    assert not errs, "\n".join(errs)
    g.close()
