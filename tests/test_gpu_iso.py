"""Isotropic model (Sigma_k = sigma^2_k I) on the HIP path against the
isotropic float64 oracle, through the C ABI: E-step statistics (N_k, S1, Q,
LL), M-step, fit (per iteration and end to end), init, and one full
iteration at 1e6 rows.  Tolerances as for the diagonal model (1e-4 per
iteration, 1e-3 after T), with Q held like the sum over d of S2."""
import sys

import numpy as np
import pytest
import torch

import oracle.gmm_oracle_iso as OI
from soft_clustering_amd import datagen

pytestmark = pytest.mark.gpu
DEV = "cuda"

# name: (law, N, D, K, ldx)
CASES = {
    "tiny": ("tiny", 10_000, 8, 16, None),
    "odd_d5_k7": ("tiny", 1_003, 5, 7, 8),
    "iso_prefix": ("iso", 20_037, 128, 1024, None),
    "d200_k100": ("iso", 2_005, 200, 100, None),
}


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def data(name):
    law, N, D, K, ldx = CASES[name]
    mix = datagen.mixture(law, D, K, seed=0)
    Xc = datagen.sample(mix, N, seed=0, ldx=ldx)
    Xn = Xc.contiguous().numpy()
    rows = datagen.init_rows(N, K, seed=1)
    params = tuple(np.asarray(a, np.float32) for a in OI.init(Xn, rows, 1e-6))
    if ldx is not None:
        buf = torch.full((N, ldx), float("nan"), dtype=torch.float32)
        buf[:, :D] = Xc
        Xg = buf.to(DEV)[:, :D]
    else:
        Xg = Xc.to(DEV)
    return Xn, Xg, params, rows


def gpu(params):
    return tuple(torch.as_tensor(a).to(DEV) for a in params)


def check_stats_iso(got, want, Xn, var_iso, tol):
    Nk_g, S1_g, Q_g, ll_g = (np.asarray(a, np.float64) for a in got)
    Nk, S1, Q, ll = (np.asarray(a, np.float64) for a in want)
    x = Xn.astype(np.float64)
    ms = np.mean(x * x, axis=0)
    sd = np.sqrt(np.asarray(var_iso, np.float64))[:, None]
    errs = []
    for what, g, w, lim in (("LL", ll_g, ll, tol * abs(ll)),
                            ("N_k", Nk_g, Nk, tol * np.maximum(Nk, 1.0)),
                            ("S1", S1_g, S1, tol * (np.abs(S1) + Nk[:, None] * sd + np.sqrt(ms)[None, :])),
                            ("Q", Q_g, Q, tol * (np.abs(Q) + ms.sum()))):
        bad = np.abs(g - w) > lim
        if np.any(bad):
            errs.append(f"{what}: {int(np.sum(bad))} outside tolerance")
    return errs


def check_params_iso(got, want, Nk_ref, N, tol):
    w_g, mu_g, v_g = (np.asarray(a, np.float64) for a in got)
    w, mu, v = (np.asarray(a, np.float64) for a in want)
    live = np.asarray(Nk_ref) >= 1.0
    errs = []
    if np.any(np.abs(w_g - w) > tol * np.maximum(w, 1.0 / N)):
        errs.append("pi")
    sd = np.sqrt(v)[:, None]
    if np.any((np.abs(mu_g - mu) > tol * (np.abs(mu) + sd))[live]):
        errs.append("mu")
    # Q/N_k - ||mu||^2 in float32 storage: a few ulps of (sigma^2 + ||mu||^2 / D)
    mm = np.sum(mu * mu, axis=1) / mu.shape[1]
    if np.any((np.abs(v_g - v) > tol * v + 1e-6 * (v + mm))[live]):
        errs.append("var")
    return errs


@pytest.mark.parametrize("path", ["fused", "fused_split_logits", "fused_fp32mfma", "two_sweep", "two_sweep_fp64"])
@pytest.mark.parametrize("name", list(CASES))
def test_estep_iso_parity(name, path):
    """fused: the isotropic kernel (split-bfloat16 logits and statistics for
    16 < D <= 128); fused_split_logits: split logits, fp32 statistics;
    fused_fp32mfma: fp32 MFMA for both."""
    from soft_clustering_amd import GMM, MFMA_FP32, MFMA_SPLIT_LOGITS, PATH_FUSED, PATH_TWO_SWEEP, PREC_FP64
    Xn, Xg, params, _ = data(name)
    N, D = Xn.shape
    K = params[1].shape[0]
    log(f"[iso estep] case={name} path={path} N={N} D={D} K={K}")
    g = GMM(K, D)
    try:
        g.set_path(PATH_TWO_SWEEP if path.startswith("two_sweep") else PATH_FUSED)
    except Exception as e:
        pytest.skip(f"fused path unavailable: {e}")
    if path.endswith("fp64"):
        g.set_precision(PREC_FP64)
    if path == "fused_fp32mfma":
        g.set_mfma(MFMA_FP32)
    if path == "fused_split_logits":
        g.set_mfma(MFMA_SPLIT_LOGITS)
    split_ok = path in ("fused", "fused_split_logits") and 16 < D <= 128
    assert g.split_level(1) == ((2 if path == "fused" else 1) if split_ok else 0)
    got = [t.cpu().numpy() for t in g.estep_stats_iso(Xg, *gpu(params))]
    g.check()
    want = OI.estep_stats(Xn, *params, method="gemm" if N * K * D > 3e7 else "direct")
    errs = check_stats_iso((got[0], got[1], got[2], got[3][0]), want, Xn, params[2], 1e-4)
    assert not errs, "\n".join(errs)


@pytest.mark.parametrize("mfma", ["split", "fp32"])
def test_estep_iso_far_from_origin(mfma):
    """Rows and means near 50 in every dimension (x . mu / s^2 and
    ||x||^2 / (2 s^2) cancel terms of about 2500 / s^2 per dimension): the
    float64 refinement carries the result for split-bf16 and fp32 MFMA
    alike.  Parameters after three GPU EM iterations."""
    from soft_clustering_amd import GMM, MFMA_FP32, PATH_FUSED
    N, D, K = 6_007, 32, 24
    mix = datagen.mixture("iso", D, K, seed=3)
    Xc = datagen.sample(mix, N, seed=3) + 50.0
    Xn = Xc.numpy()
    params = tuple(np.asarray(a, np.float32) for a in OI.init(Xn, datagen.init_rows(N, K, seed=4), 1e-6))
    log(f"[iso far] mfma={mfma} N={N} D={D} K={K}")
    g = GMM(K, D)
    g.set_path(PATH_FUSED)
    if mfma == "fp32":
        g.set_mfma(MFMA_FP32)
    assert g.split_level(1) == (2 if mfma == "split" else 0)
    Xg = Xc.to(DEV)
    w, mu, v = gpu(params)
    g.fit_iso(Xg, w, mu, v, 3, 1e-6)
    g.check()
    th = tuple(a.cpu().numpy().copy() for a in (w, mu, v))
    got = [t.cpu().numpy() for t in g.estep_stats_iso(Xg, w, mu, v)]
    g.check()
    want = OI.estep_stats(Xn, *th)
    errs = check_stats_iso((got[0], got[1], got[2], got[3][0]), want, Xn, th[2], 1e-4)
    assert not errs, errs


def test_estep_iso_accumulate_over_chunks():
    from soft_clustering_amd import GMM
    Xn, Xg, params, _ = data("d200_k100")
    K, D = params[1].shape
    g = GMM(K, D)
    p = gpu(params)
    full = [t.cpu().numpy() for t in g.estep_stats_iso(Xg, *p)]
    out = g.estep_stats_iso(Xg[:777], *p)
    g.estep_stats_iso(Xg[777:], *p, out=out, accumulate=True)
    g.check()
    part = [t.cpu().numpy() for t in out]
    errs = check_stats_iso((part[0], part[1], part[2], part[3][0]), (full[0], full[1], full[2], full[3][0]),
                           Xn, params[2], 1e-6)
    assert not errs, "\n".join(errs)


def test_mstep_iso_parity():
    from soft_clustering_amd import GMM
    Xn, Xg, params, _ = data("iso_prefix")
    N = Xn.shape[0]
    K, D = params[1].shape
    Nk, S1, Q, _ = OI.estep_stats(Xn, *params, method="gemm")
    Nk = Nk.copy()
    Nk[:3] = [0.0, 5e-7, 2e-6]  # empty-rule edge: below / above 1e-6
    want = OI.mstep(Nk, S1, Q, N, 1e-6, params[1], params[2])
    g = GMM(K, D)
    w, mu, v = gpu(params)
    g.mstep_iso(*(torch.as_tensor(a).to(DEV) for a in (Nk, S1, Q)), N, 1e-6, w, mu, v)
    g.check()
    np.testing.assert_array_equal(w.cpu().numpy(), want[0].astype(np.float32))
    np.testing.assert_array_equal(mu.cpu().numpy(), want[1].astype(np.float32))
    np.testing.assert_allclose(v.cpu().numpy(), want[2].astype(np.float32), rtol=2e-7)


def test_init_iso_parity():
    from soft_clustering_amd import GMM
    for name in ("tiny", "odd_d5_k7", "iso_prefix"):
        Xn, Xg, params, rows = data(name)
        K, D = params[1].shape
        g = GMM(K, D)
        w, mu, v = g.init_iso(Xg, rows, 1e-6)
        np.testing.assert_array_equal(w.cpu().numpy(), params[0])
        np.testing.assert_array_equal(mu.cpu().numpy(), params[1])
        np.testing.assert_allclose(v.cpu().numpy(), params[2], rtol=2e-7)


@pytest.mark.parametrize("path", ["fused", "two_sweep"])
def test_fit_iso_tiny_per_iteration_and_end_to_end(path):
    from soft_clustering_amd import GMM, PATH_FUSED, PATH_TWO_SWEEP
    Xn, Xg, params, _ = data("tiny")
    N = Xn.shape[0]
    K, D = params[1].shape
    T = 10
    g = GMM(K, D)
    g.set_path(PATH_FUSED if path == "fused" else PATH_TWO_SWEEP)
    w, mu, v = gpu(params)
    for t in range(T):
        th = tuple(a.cpu().numpy().copy() for a in (w, mu, v))
        Nk, S1, Q, ll = OI.estep_stats(Xn, *th)
        want = OI.mstep(Nk, S1, Q, N, 1e-6, th[1], th[2])
        hist = torch.zeros(1, dtype=torch.float64, device=DEV)
        g.fit_iso(Xg, w, mu, v, 1, 1e-6, hist)
        g.check()
        assert abs(hist.item() - ll) <= 1e-4 * abs(ll), (t, hist.item(), ll)
        errs = check_params_iso((w.cpu(), mu.cpu(), v.cpu()), want, Nk, N, 1e-4)
        assert not errs, f"iteration {t}: {errs}"
    w2, mu2, v2 = gpu(params)
    _, _, _, hist = g.fit_iso(Xg, w2, mu2, v2, T, 1e-6)
    g.check()
    rw, rmu, rv, rhist = OI.fit(Xn, *params, T, 1e-6)
    np.testing.assert_allclose(hist.cpu().numpy(), rhist, rtol=1e-3)
    errs = check_params_iso((w2.cpu(), mu2.cpu(), v2.cpu()), (rw, rmu, rv), np.full(K, 2.0), N, 1e-3)
    assert not errs, errs
    h = hist.cpu().numpy()
    assert np.all(np.diff(h) >= -1e-6 * np.abs(h[1:]))


def test_fit_iso_mid_1e6_rows_one_iteration():
    """The isotropic law at 1e6 x 128, K=1024: from parameters after two GPU
    iterations, one full EM iteration on both sides."""
    from soft_clustering_amd import GMM
    wl = datagen.WORKLOADS["iso"]
    N = 1_000_000
    log(f"iso mid: N={N} D={wl.D} K={wl.K}")
    mix = datagen.mixture(wl.law, wl.D, wl.K, seed=wl.seed)
    X = torch.empty(N, wl.D, dtype=torch.float32, device=DEV)
    datagen.sample_into(X, mix, 0, seed=wl.seed)
    g = GMM(wl.K, wl.D)
    w, mu, v = g.init_iso(X, datagen.init_rows(N, wl.K, seed=wl.init_seed), wl.var_floor)
    g.fit_iso(X, w, mu, v, 2, wl.var_floor)
    th = tuple(a.cpu().numpy().copy() for a in (w, mu, v))
    got = [t.cpu().numpy() for t in g.estep_stats_iso(X, w, mu, v)]
    hist = torch.zeros(1, dtype=torch.float64, device=DEV)
    g.fit_iso(X, w, mu, v, 1, wl.var_floor, hist)
    g.check()
    Xn = X.cpu().numpy()
    want = OI.estep_stats(Xn, *th, method="gemm")
    errs = check_stats_iso((got[0], got[1], got[2], got[3][0]), want, Xn, th[2], 1e-4)
    assert not errs, errs
    assert abs(hist.item() - want[3]) <= 1e-4 * abs(want[3])
    ref = OI.mstep(*want[:3], N, wl.var_floor, th[1], th[2])
    errs = check_params_iso((w.cpu(), mu.cpu(), v.cpu()), ref, want[0], N, 1e-4)
    assert not errs, errs


@pytest.mark.parametrize("precision", ["refined", "fp32"])
@pytest.mark.parametrize("name", ["tiny", "odd_d5_k7", "iso_prefix"])
def test_iso_kernel_matches_broadcast_path(name, precision, monkeypatch):
    """The fused isotropic kernel (D-wide contractions) against the diagonal
    kernels run on the broadcast variances: the same statistics up to
    float32 rounding of the logits (refined logits agree to float64)."""
    from soft_clustering_amd import GMM, PATH_FUSED, PREC_FP32, PREC_REFINED
    Xn, Xg, params, _ = data(name)
    K, D = params[1].shape
    g = GMM(K, D)
    g.set_path(PATH_FUSED)
    g.set_precision(PREC_REFINED if precision == "refined" else PREC_FP32)
    out = {}
    for flag in ("1", "0"):
        monkeypatch.setenv("FLASHGMM_ISO_KERNEL", flag)
        out[flag] = [t.cpu().numpy() for t in g.estep_stats_iso(Xg, *gpu(params))]
        g.check()
    a, b = out["1"], out["0"]
    tol = 1e-5 if precision == "refined" else 1e-3
    errs = check_stats_iso((a[0], a[1], a[2], a[3][0]), (b[0], b[1], b[2], b[3][0]), Xn, params[2], tol)
    assert not errs, errs
