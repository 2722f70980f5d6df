"""gmm_estep_stats_noalloc (the E-step for callers that cannot allocate device
memory) through the C ABI, against gmm_estep_stats on the same inputs: two
calls in a row, the second on fewer rows, for a shape whose workspace fits
the scratch with every statistics slot (bit-identical) and one that gets
fewer slots (the per-iteration tolerance); and no device memory allocated."""
import ctypes
import sys

import numpy as np
import pytest
import torch

import oracle.gmm_oracle as O
from soft_clustering_amd import GMM, datagen, raw_library
from tests.tolerance import check_stats, data_scales

pytestmark = pytest.mark.gpu
DEV = "cuda"


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _lib():
    lib = raw_library()
    f = lib.gmm_estep_stats_noalloc
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    f.restype = i32
    f.argtypes = [i32, i32, vp, i64, i64, vp, vp, vp, vp, vp, vp, vp, i32, vp]
    lib.gmm_last_error.restype = ctypes.c_char_p
    lib.gmm_last_error.argtypes = [vp]
    return lib


def noalloc(lib, X, w, mu, var, out):
    K, D = mu.shape
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    st = lib.gmm_estep_stats_noalloc(K, D, p(X), X.shape[0], X.stride(0), p(w), p(mu), p(var),
                                     *(p(t) for t in out), 0,
                                     ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, lib.gmm_last_error(None).decode()
    return out


def zeros(K, D):
    return (torch.zeros(K, dtype=torch.float64, device=DEV), torch.zeros(K, D, dtype=torch.float64, device=DEV),
            torch.zeros(K, D, dtype=torch.float64, device=DEV), torch.zeros(1, dtype=torch.float64, device=DEV))


@pytest.mark.parametrize("law,N,D,K,exact", [
    ("mid", 60_013, 128, 1024, True),      # every statistics slot fits: bit-identical
    ("ivf", 30_011, 128, 16_384, False),   # fewer slots than the context: same sums, other order
    ("tiny", 5_003, 8, 16, True),
    ("embed", 9_001, 768, 512, False),     # eight dim-segment waves, 32-row tiles
])
def test_noalloc_matches_estep_stats(law, N, D, K, exact):
    lib = _lib()
    mix = datagen.mixture(law, D, K, seed=0)
    X = datagen.sample(mix, N, seed=0, device=DEV)
    floor = 1.0 / 12.0 if law == "ivf" else 1e-6
    g = GMM(K, D)
    w, mu, var = g.init(X, datagen.init_rows(N, K, seed=1), floor)
    g.fit(X, w, mu, var, 2, floor)
    g.check()
    # the first call on a device takes the scratch's address, which may load
    # the code object that holds it: device memory is compared from then on
    noalloc(lib, X[:64], w, mu, var, zeros(K, D))
    for rows in (N, N // 3 + 7):  # two calls in a row, the second smaller
        log(f"[noalloc] law={law} N={rows} D={D} K={K}")
        Xr = X[:rows]
        ref = [t.clone() for t in g.estep_stats(Xr, w, mu, var)]
        g.check()
        out = zeros(K, D)
        torch.cuda.synchronize()
        free0, _ = torch.cuda.mem_get_info()
        noalloc(lib, Xr, w, mu, var, out)
        torch.cuda.synchronize()
        free1, _ = torch.cuda.mem_get_info()
        if exact:
            for a, b, what in zip(out, ref, ("Nk", "S1", "S2", "LL")):
                assert torch.equal(a, b), f"{what} differs from gmm_estep_stats"
        else:
            ms, rms = data_scales(Xr.cpu().numpy())
            o = [t.cpu().numpy() for t in out]
            r = [t.cpu().numpy() for t in ref]
            errs = check_stats((o[0], o[1], o[2], o[3][0]), (r[0], r[1], r[2], r[3][0]), ms, rms,
                               np.sqrt(var.cpu().numpy().astype(np.float64)), 1e-4)
            assert not errs, "\n".join(errs)
        # and against the float64 oracle on a row sample's statistics
        if rows < N and K <= 1024:
            want = O.estep_stats(Xr.cpu().numpy(), w.cpu().numpy(), mu.cpu().numpy(), var.cpu().numpy(),
                                 method="gemm")
            ms, rms = data_scales(Xr.cpu().numpy())
            o = [t.cpu().numpy() for t in out]
            errs = check_stats((o[0], o[1], o[2], o[3][0]), want, ms, rms,
                               np.sqrt(var.cpu().numpy().astype(np.float64)), 1e-4)
            assert not errs, "\n".join(errs)
        assert free0 - free1 <= (2 << 20), f"device memory fell by {free0 - free1} bytes"
    g.close()


def test_noalloc_rejects_what_does_not_fit():
    lib = _lib()
    K, D = 16_384, 768  # its smallest workspace is above the scratch size
    X = torch.zeros(64, D, device=DEV)
    w = torch.full((K,), 1.0 / K, device=DEV)
    mu = torch.zeros(K, D, device=DEV)
    var = torch.ones(K, D, device=DEV)
    out = zeros(K, D)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    st = lib.gmm_estep_stats_noalloc(K, D, p(X), 64, D, p(w), p(mu), p(var), *(p(t) for t in out), 0, None)
    assert st == 6, "expected GMM_ERR_CAPACITY"
    assert b"scratch" in lib.gmm_last_error(None)
    st = lib.gmm_estep_stats_noalloc(K, D, p(X), 64, D + 1, p(w), p(mu), p(var), *(p(t) for t in out), 0, None)
    assert st == 1, "ldx not a multiple of 4 must be rejected"
