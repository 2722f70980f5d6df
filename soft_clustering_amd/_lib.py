"""ctypes binding of libflashgmm.so (C ABI in include/flashgmm.h).

Argument marshalling only: tensors are checked for dtype, device, layout and
alignment, then their device pointers and the current HIP stream are passed
to the library.  Every computation runs in the library's HIP kernels; there
is no fallback of any kind, and a missing library raises at import.
"""
from __future__ import annotations

import atexit
import ctypes
import os
import sys
import weakref

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("FLASHGMM_LIB") or os.path.join(_HERE, "libflashgmm.so")

GMM_OK = 0
_STATUS = {0: "GMM_OK", 1: "GMM_ERR_INVALID_ARG", 2: "GMM_ERR_UNSUPPORTED", 3: "GMM_ERR_OOM",
           4: "GMM_ERR_HIP", 5: "GMM_ERR_NUMERIC", 6: "GMM_ERR_CAPACITY"}
PATH_AUTO, PATH_TWO_SWEEP, PATH_FUSED = 0, 1, 2
PREC_REFINED, PREC_FP32, PREC_FP64 = 0, 1, 2
MFMA_SPLIT_BF16, MFMA_SPLIT_LOGITS, MFMA_FP32 = 0, 1, 2

EXPORTS = ["gmm_create", "gmm_destroy", "gmm_last_error", "gmm_workspace_bytes", "gmm_set_path", "gmm_set_precision",
           "gmm_set_mfma", "gmm_split_level", "gmm_set_assign_limit",
           "gmm_init", "gmm_estep_stats", "gmm_mstep", "gmm_fit", "gmm_soft_assign", "gmm_check",
           "gmm_init_iso", "gmm_estep_stats_iso", "gmm_mstep_iso", "gmm_fit_iso", "gmm_kmeans", "gmm_init_kmeans",
           "gmm_estep_stats_host", "gmm_fit_host",
           "gmm_profile", "gmm_profile_read", "gmm_refine_stats", "gmm_estep_stats_noalloc"]


class GMMError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python soft_clustering_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32, f64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_double
    sig = {
        "gmm_create": (i32, [ctypes.POINTER(vp), i32, i32, vp]),
        "gmm_destroy": (None, [vp]),
        "gmm_last_error": (ctypes.c_char_p, [vp]),
        "gmm_workspace_bytes": (ctypes.c_size_t, [i32, i32]),
        "gmm_set_path": (i32, [vp, i32]),
        "gmm_set_precision": (i32, [vp, i32]),
        "gmm_set_mfma": (i32, [vp, i32]),
        "gmm_set_assign_limit": (i32, [vp, i64]),
        "gmm_split_level": (i32, [vp, i32]),
        "gmm_init": (i32, [vp, vp, i64, i64, vp, f32, vp, vp, vp]),
        "gmm_estep_stats": (i32, [vp, vp, i64, i64, vp, vp, vp, vp, vp, vp, vp, i32]),
        "gmm_mstep": (i32, [vp, vp, vp, vp, f64, f32, vp, vp, vp]),
        "gmm_fit": (i32, [vp, vp, i64, i64, i32, f32, vp, vp, vp, vp]),
        "gmm_init_iso": (i32, [vp, vp, i64, i64, vp, f32, vp, vp, vp]),
        "gmm_estep_stats_iso": (i32, [vp, vp, i64, i64, vp, vp, vp, vp, vp, vp, vp, i32]),
        "gmm_mstep_iso": (i32, [vp, vp, vp, vp, f64, f32, vp, vp, vp]),
        "gmm_fit_iso": (i32, [vp, vp, i64, i64, i32, f32, vp, vp, vp, vp]),
        "gmm_kmeans": (i32, [vp, vp, i64, i64, i32, vp, vp, vp, vp]),
        "gmm_estep_stats_host": (i32, [vp, vp, i64, i64, vp, vp, vp, vp, vp, vp, vp, i32, i64]),
        "gmm_fit_host": (i32, [vp, vp, i64, i64, i32, f32, vp, vp, vp, vp, i64]),
        "gmm_init_kmeans": (i32, [vp, vp, i64, i64, vp, f32, i32, vp, vp, vp, vp, vp]),
        "gmm_soft_assign": (i32, [vp, vp, i64, i64, vp, vp, vp, f32, i32, vp, vp, i64, vp]),
        "gmm_check": (i32, [vp]),
        "gmm_profile": (i32, [vp, i32]),
        "gmm_refine_stats": (i32, [vp, ctypes.POINTER(i64), ctypes.POINTER(f64)]),
        "gmm_profile_read": (i32, [vp, ctypes.POINTER(f64), ctypes.POINTER(i64), ctypes.POINTER(f64),
                                   ctypes.POINTER(i64)]),
        "gmm_estep_stats_noalloc": (i32, [i32, i32, vp, i64, i64, vp, vp, vp, vp, vp, vp, vp, i32, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t, dtype, shape, name, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _rows(X, D, device):
    """(N, ldx) of a row-major fp32 matrix that may have a row stride > D."""
    if not isinstance(X, torch.Tensor) or X.dtype != torch.float32 or X.dim() != 2:
        raise TypeError("X must be a 2-D float32 tensor")
    if X.device != device:
        raise ValueError(f"X must be on {device}")
    if X.shape[1] != D:
        raise ValueError(f"X has {X.shape[1]} columns, the model has D={D}")
    if X.stride(1) != 1:
        raise ValueError("X rows must be contiguous (stride(1) == 1)")
    return X.shape[0], X.stride(0) if X.shape[0] > 1 else ((D + 3) // 4) * 4


_LIVE: "weakref.WeakSet[GMM]" = weakref.WeakSet()


@atexit.register
def _close_all():
    """Destroy every live context while the HIP runtime is still up: torch
    registers its own exit handlers when it is imported, before this module,
    and exit handlers run last-registered first, so this runs ahead of them.
    Afterwards no library call is left for a finaliser to make during
    interpreter teardown."""
    for g in list(_LIVE):
        try:
            g.close()
        except Exception:
            pass


class GMM:
    """A context for K components of dimension D on the current HIP device.

    Release it with close() (or use it as a context manager); contexts still
    open when the interpreter exits are closed by an exit handler."""

    def __init__(self, K: int, D: int, device=None):
        if not torch.cuda.is_available():
            raise RuntimeError("the HIP library needs a GPU")
        dev = torch.device(device) if device is not None else torch.device("cuda")
        if dev.type != "cuda":
            raise ValueError("device must be a GPU device")
        self.device = dev if dev.index is not None else torch.device("cuda", torch.cuda.current_device())
        self.K, self.D = int(K), int(D)
        with torch.cuda.device(self.device):
            h = ctypes.c_void_p()
            st = _lib.gmm_create(ctypes.byref(h), self.K, self.D, _stream())
            if st != GMM_OK:
                raise GMMError(st, _lib.gmm_last_error(None).decode())
        self._h = h
        _LIVE.add(self)

    def close(self):
        """Synchronise the context's stream and release its workspace."""
        h = getattr(self, "_h", None)
        self._h = None
        if h:
            with torch.cuda.device(self.device):
                _lib.gmm_destroy(h)
        _LIVE.discard(self)

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()
        return False

    def __del__(self):
        # never call into the library while the interpreter is finalising
        # (the exit handler above has closed every context by then)
        if sys.is_finalizing():
            return
        try:
            self.close()
        except Exception:
            pass

    def _check(self, st):
        if st != GMM_OK:
            raise GMMError(st, _lib.gmm_last_error(self._h).decode())

    @staticmethod
    def workspace_bytes(K: int, D: int) -> int:
        return int(_lib.gmm_workspace_bytes(int(K), int(D)))

    def set_path(self, path: int):
        self._check(_lib.gmm_set_path(self._h, int(path)))

    def set_precision(self, mode: int):
        self._check(_lib.gmm_set_precision(self._h, int(mode)))

    def set_mfma(self, kind: int):
        self._check(_lib.gmm_set_mfma(self._h, int(kind)))

    def set_assign_limit(self, nbytes: int):
        """Device memory soft_assign may hold beyond the workspace (kept
        selections, list-sort buffer); 0 = none (chunked list building)."""
        self._check(_lib.gmm_set_assign_limit(self._h, int(nbytes)))

    def split_level(self, model: int = 0) -> int:
        """0 fp32 MFMA, 1 split-bf16 logits, 2 split-bf16 logits and
        statistics; model: 0 diagonal, 1 isotropic, 2 k-means hard
        assignment."""
        return int(_lib.gmm_split_level(self._h, int(model)))

    def params(self):
        """Fresh fp32 (weights, means, vars) buffers on the device."""
        K, D = self.K, self.D
        return (torch.empty(K, dtype=torch.float32, device=self.device),
                torch.empty(K, D, dtype=torch.float32, device=self.device),
                torch.empty(K, D, dtype=torch.float32, device=self.device))

    def _params(self, w, mu, var):
        _need(w, torch.float32, (self.K,), "weights", self.device)
        _need(mu, torch.float32, (self.K, self.D), "means", self.device)
        _need(var, torch.float32, (self.K, self.D), "vars", self.device)

    def init(self, X, rows, var_floor, out=None):
        N, ldx = _rows(X, self.D, self.device)
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        if rows.shape != (self.K,):
            raise ValueError(f"rows must have shape ({self.K},)")
        w, mu, var = out if out is not None else self.params()
        self._params(w, mu, var)
        with torch.cuda.device(self.device):
            self._check(_lib.gmm_init(self._h, _ptr(X), N, ldx, rows.ctypes.data_as(ctypes.c_void_p),
                                      float(var_floor), _ptr(w), _ptr(mu), _ptr(var)))
        return w, mu, var

    def estep_stats(self, X, w, mu, var, out=None, accumulate=False):
        N, ldx = _rows(X, self.D, self.device)
        self._params(w, mu, var)
        K, D = self.K, self.D
        if out is None:
            out = (torch.zeros(K, dtype=torch.float64, device=self.device),
                   torch.zeros(K, D, dtype=torch.float64, device=self.device),
                   torch.zeros(K, D, dtype=torch.float64, device=self.device),
                   torch.zeros(1, dtype=torch.float64, device=self.device))
        Nk, S1, S2, ll = out
        _need(Nk, torch.float64, (K,), "Nk", self.device)
        _need(S1, torch.float64, (K, D), "S1", self.device)
        _need(S2, torch.float64, (K, D), "S2", self.device)
        _need(ll, torch.float64, (1,), "loglik", self.device)
        with torch.cuda.device(self.device):
            self._check(_lib.gmm_estep_stats(self._h, _ptr(X), N, ldx, _ptr(w), _ptr(mu), _ptr(var),
                                             _ptr(Nk), _ptr(S1), _ptr(S2), _ptr(ll), int(bool(accumulate))))
        return Nk, S1, S2, ll

    def mstep(self, Nk, S1, S2, n_total, var_floor, w, mu, var):
        K, D = self.K, self.D
        _need(Nk, torch.float64, (K,), "Nk", self.device)
        _need(S1, torch.float64, (K, D), "S1", self.device)
        _need(S2, torch.float64, (K, D), "S2", self.device)
        self._params(w, mu, var)
        with torch.cuda.device(self.device):
            self._check(_lib.gmm_mstep(self._h, _ptr(Nk), _ptr(S1), _ptr(S2), float(n_total), float(var_floor),
                                       _ptr(w), _ptr(mu), _ptr(var)))
        return w, mu, var

    def fit(self, X, w, mu, var, T, var_floor, ll_hist=None):
        N, ldx = _rows(X, self.D, self.device)
        self._params(w, mu, var)
        if ll_hist is None:
            ll_hist = torch.zeros(int(T), dtype=torch.float64, device=self.device)
        _need(ll_hist, torch.float64, (int(T),), "loglik_hist", self.device)
        with torch.cuda.device(self.device):
            self._check(_lib.gmm_fit(self._h, _ptr(X), N, ldx, int(T), float(var_floor), _ptr(w), _ptr(mu),
                                     _ptr(var), _ptr(ll_hist)))
        return w, mu, var, ll_hist

    # ---- isotropic model (var_iso: K variances)
    def _params_iso(self, w, mu, var_iso):
        _need(w, torch.float32, (self.K,), "weights", self.device)
        _need(mu, torch.float32, (self.K, self.D), "means", self.device)
        _need(var_iso, torch.float32, (self.K,), "var_iso", self.device)

    def init_iso(self, X, rows, var_floor):
        N, ldx = _rows(X, self.D, self.device)
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        if rows.shape != (self.K,):
            raise ValueError(f"rows must have shape ({self.K},)")
        w, mu, _ = self.params()
        var_iso = torch.empty(self.K, dtype=torch.float32, device=self.device)
        with torch.cuda.device(self.device):
            self._check(_lib.gmm_init_iso(self._h, _ptr(X), N, ldx, rows.ctypes.data_as(ctypes.c_void_p),
                                          float(var_floor), _ptr(w), _ptr(mu), _ptr(var_iso)))
        return w, mu, var_iso

    def estep_stats_iso(self, X, w, mu, var_iso, out=None, accumulate=False):
        N, ldx = _rows(X, self.D, self.device)
        self._params_iso(w, mu, var_iso)
        K, D = self.K, self.D
        if out is None:
            out = (torch.zeros(K, dtype=torch.float64, device=self.device),
                   torch.zeros(K, D, dtype=torch.float64, device=self.device),
                   torch.zeros(K, dtype=torch.float64, device=self.device),
                   torch.zeros(1, dtype=torch.float64, device=self.device))
        Nk, S1, Q, ll = out
        _need(Nk, torch.float64, (K,), "Nk", self.device)
        _need(S1, torch.float64, (K, D), "S1", self.device)
        _need(Q, torch.float64, (K,), "Q", self.device)
        _need(ll, torch.float64, (1,), "loglik", self.device)
        with torch.cuda.device(self.device):
            self._check(_lib.gmm_estep_stats_iso(self._h, _ptr(X), N, ldx, _ptr(w), _ptr(mu), _ptr(var_iso),
                                                 _ptr(Nk), _ptr(S1), _ptr(Q), _ptr(ll), int(bool(accumulate))))
        return Nk, S1, Q, ll

    def mstep_iso(self, Nk, S1, Q, n_total, var_floor, w, mu, var_iso):
        K, D = self.K, self.D
        _need(Nk, torch.float64, (K,), "Nk", self.device)
        _need(S1, torch.float64, (K, D), "S1", self.device)
        _need(Q, torch.float64, (K,), "Q", self.device)
        self._params_iso(w, mu, var_iso)
        with torch.cuda.device(self.device):
            self._check(_lib.gmm_mstep_iso(self._h, _ptr(Nk), _ptr(S1), _ptr(Q), float(n_total), float(var_floor),
                                           _ptr(w), _ptr(mu), _ptr(var_iso)))
        return w, mu, var_iso

    def fit_iso(self, X, w, mu, var_iso, T, var_floor, ll_hist=None):
        N, ldx = _rows(X, self.D, self.device)
        self._params_iso(w, mu, var_iso)
        if ll_hist is None:
            ll_hist = torch.zeros(int(T), dtype=torch.float64, device=self.device)
        _need(ll_hist, torch.float64, (int(T),), "loglik_hist", self.device)
        with torch.cuda.device(self.device):
            self._check(_lib.gmm_fit_iso(self._h, _ptr(X), N, ldx, int(T), float(var_floor), _ptr(w), _ptr(mu),
                                         _ptr(var_iso), _ptr(ll_hist)))
        return w, mu, var_iso, ll_hist

    # ---- out-of-core: X in host memory (a CPU tensor, pinned for overlap)
    def _host_rows(self, X):
        if not isinstance(X, torch.Tensor) or X.device.type != "cpu" or X.dtype != torch.float32:
            raise TypeError("X must be a float32 CPU tensor")
        if X.dim() != 2 or X.shape[1] != self.D or X.stride(1) != 1:
            raise ValueError(f"X must be N x {self.D} with unit column stride")
        return X.shape[0], X.stride(0)

    def estep_stats_host(self, X, w, mu, var, chunk_rows, out=None, accumulate=False):
        N, ldx = self._host_rows(X)
        self._params(w, mu, var)
        K, D = self.K, self.D
        if out is None:
            out = (torch.zeros(K, dtype=torch.float64, device=self.device),
                   torch.zeros(K, D, dtype=torch.float64, device=self.device),
                   torch.zeros(K, D, dtype=torch.float64, device=self.device),
                   torch.zeros(1, dtype=torch.float64, device=self.device))
        Nk, S1, S2, ll = out
        with torch.cuda.device(self.device):
            self._check(_lib.gmm_estep_stats_host(self._h, ctypes.c_void_p(X.data_ptr()), N, ldx, _ptr(w), _ptr(mu),
                                                  _ptr(var), _ptr(Nk), _ptr(S1), _ptr(S2), _ptr(ll),
                                                  int(bool(accumulate)), int(chunk_rows)))
        return Nk, S1, S2, ll

    def fit_host(self, X, w, mu, var, T, var_floor, chunk_rows, ll_hist=None):
        N, ldx = self._host_rows(X)
        self._params(w, mu, var)
        if ll_hist is None:
            ll_hist = torch.zeros(int(T), dtype=torch.float64, device=self.device)
        with torch.cuda.device(self.device):
            self._check(_lib.gmm_fit_host(self._h, ctypes.c_void_p(X.data_ptr()), N, ldx, int(T), float(var_floor),
                                          _ptr(w), _ptr(mu), _ptr(var), _ptr(ll_hist), int(chunk_rows)))
        return w, mu, var, ll_hist

    # ---- k-means warm start
    def _list_scratch(self, N):
        return (torch.empty(self.K + 1, dtype=torch.int64, device=self.device),
                torch.empty(max(N, 1), dtype=torch.int32, device=self.device))

    def kmeans(self, X, centres, iters, lists=True):
        """Lloyd iterations in place on centres (K x D float32); returns
        (centres, counts float64[K], offsets, ids).  With lists the CSR lists
        of the rows' nearest returned centres come back (one more assignment
        sweep); without them offsets and ids are None, which only the fused
        path accepts."""
        N, ldx = _rows(X, self.D, self.device)
        _need(centres, torch.float32, (self.K, self.D), "centres", self.device)
        counts = torch.zeros(self.K, dtype=torch.float64, device=self.device)
        offsets, ids = self._list_scratch(N) if lists else (None, None)
        with torch.cuda.device(self.device):
            self._check(_lib.gmm_kmeans(self._h, _ptr(X), N, ldx, int(iters), _ptr(centres), _ptr(counts),
                                        _ptr(offsets), _ptr(ids)))
        return centres, counts, offsets, (ids[:N] if lists else None)

    def init_kmeans(self, X, centres, var_floor, isotropic=False):
        """(weights, means, vars) of the mixture seeded from the clustering."""
        N, ldx = _rows(X, self.D, self.device)
        _need(centres, torch.float32, (self.K, self.D), "centres", self.device)
        w, mu, var = self.params()
        if isotropic:
            var = torch.empty(self.K, dtype=torch.float32, device=self.device)
        offsets, ids = self._list_scratch(N)
        with torch.cuda.device(self.device):
            self._check(_lib.gmm_init_kmeans(self._h, _ptr(X), N, ldx, _ptr(centres), float(var_floor),
                                             int(bool(isotropic)), _ptr(w), _ptr(mu), _ptr(var), _ptr(offsets),
                                             _ptr(ids)))
        return w, mu, var

    def soft_assign(self, X, w, mu, var, threshold=0.1, max_extra=3, ids_capacity=None):
        """CSR inverted lists: (offsets int64[K+1], ids int32[nnz])."""
        N, ldx = _rows(X, self.D, self.device)
        self._params(w, mu, var)
        offsets = torch.empty(self.K + 1, dtype=torch.int64, device=self.device)
        cap = int(ids_capacity) if ids_capacity is not None else N * (1 + int(max_extra))
        ids = torch.empty(max(cap, 1), dtype=torch.int32, device=self.device)
        nnz = ctypes.c_int64(0)
        with torch.cuda.device(self.device):
            st = _lib.gmm_soft_assign(self._h, _ptr(X), N, ldx, _ptr(w), _ptr(mu), _ptr(var), float(threshold),
                                      int(max_extra), _ptr(offsets), _ptr(ids), cap, ctypes.byref(nnz))
        if st == 6:
            raise GMMError(st, f"{_lib.gmm_last_error(self._h).decode()} (nnz={nnz.value})")
        self._check(st)
        return offsets, ids[: nnz.value]

    def profile(self, enable: bool):
        self._check(_lib.gmm_profile(self._h, int(bool(enable))))

    def profile_read(self):
        """(stats_ms, stats_launches, logz_ms, logz_launches) since the last read."""
        a, b, c, d = ctypes.c_double(), ctypes.c_int64(), ctypes.c_double(), ctypes.c_int64()
        with torch.cuda.device(self.device):
            self._check(_lib.gmm_profile_read(self._h, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c),
                                              ctypes.byref(d)))
        return a.value, b.value, c.value, d.value

    def refine_stats(self):
        """(refined logits, evaluated logits) since the last call."""
        a, b = ctypes.c_int64(), ctypes.c_double()
        with torch.cuda.device(self.device):
            self._check(_lib.gmm_refine_stats(self._h, ctypes.byref(a), ctypes.byref(b)))
        return a.value, b.value

    def check(self):
        with torch.cuda.device(self.device):
            self._check(_lib.gmm_check(self._h))


def estep_stats_noalloc(X, w, mu, var, out, accumulate=False):
    """gmm_estep_stats_noalloc: the E-step statistics without a context, into
    the caller's out = (Nk, S1, S2, loglik) on torch's current stream; the
    library allocates nothing (its workspace is a fixed device array)."""
    K, D = mu.shape
    N, ldx = _rows(X, D, X.device)
    for t, dt, shape, name in ((w, torch.float32, (K,), "weights"), (mu, torch.float32, (K, D), "means"),
                               (var, torch.float32, (K, D), "vars")):
        _need(t, dt, shape, name, X.device)
    Nk, S1, S2, ll = out
    for t, shape, name in ((Nk, (K,), "Nk"), (S1, (K, D), "S1"), (S2, (K, D), "S2"), (ll, (1,), "loglik")):
        _need(t, torch.float64, shape, name, X.device)
    with torch.cuda.device(X.device):
        st = _lib.gmm_estep_stats_noalloc(int(K), int(D), _ptr(X), N, ldx, _ptr(w), _ptr(mu), _ptr(var), _ptr(Nk),
                                          _ptr(S1), _ptr(S2), _ptr(ll), int(bool(accumulate)), _stream())
    if st != GMM_OK:
        raise GMMError(st, _lib.gmm_last_error(None).decode())
    return out


def raw_library():
    """The ctypes handle (for ABI tests)."""
    return _lib
