"""Writes the end-to-end EM fixtures fit_<name>.npz from the float64 oracle alone.

Each fixture is T EM iterations of ``oracle.gmm_oracle.fit`` (Section 2 of the
Flash-GMM pages: E-step, then the M-step Eqs. (1)-(3), repeated) on rows
drawn by ``datagen.sample_portable`` from one of the configured workloads'
laws, from the initialisation ``oracle.gmm_oracle.init`` on seeded rows.
Stored: the SHA-256 of the data bytes (the GPU test regenerates the rows on
its own host and checks this first), the initial rows, the log-likelihood
history of all T iterations and the parameters after the checkpoint
iteration (all components, or a seeded sample of them where all would make
the file large).  Nothing here runs the HIP library.

Usage: python tests/golden/make_fit_goldens.py [name ...]
"""
import hashlib
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
from oracle import gmm_oracle as o  # noqa: E402
from soft_clustering_amd import datagen  # noqa: E402

# name: (law, N rows, D, K, T iterations, checkpoint iteration, variance floor,
#        stored components or None for all)
# Parameters are stored after the checkpoint iteration (T unless stated);
# the log-likelihood history always covers all T iterations.
FIXTURES = {
    # the mid workload in full: N=1e6, D=128, K=1024, 30 iterations
    "mid": ("mid", 1_000_000, 128, 1024, 30, 30, 1e-6, None),
    # the embedding-like workload on a 262,144-row prefix (64 rows per
    # component), 20 iterations; parameters after 5 (its trajectory is
    # chaotic past that: one float32 ulp of the start moves a sixth of the
    # components by more than 1e-4 by iteration 20)
    "embed": ("embed", 262_144, 768, 4096, 20, 5, 1e-5, 256),
    # the IVF training on a 131,072-row prefix of the sample, 10 iterations
    "ivf": ("ivf", 131_072, 128, 16_384, 10, 10, 1.0 / 12.0, 1024),
}


def make(name):
    law, N, D, K, T, tc, floor, keep = FIXTURES[name]
    mix = datagen.mixture(law, D, K, seed=0)
    X = datagen.sample_portable(mix, N, seed=0)
    digest = hashlib.sha256(X.tobytes()).hexdigest()
    rows = datagen.init_rows(N, K, seed=1)
    w0, mu0, v0 = (a.astype(np.float32) for a in o.init(X, rows, floor))
    t0 = time.time()
    chunk = max(1024, (1 << 28) // (K * 8))  # bounds the per-chunk log-density block to 256 MiB
    # the oracle stores its parameters in float32 after every iteration, so
    # tc iterations and then T - tc more are the same run as T in one go
    w, mu, v, hist = o.fit(X, w0, mu0, v0, tc, floor, method="gemm", chunk_rows=chunk)
    if tc < T:
        _, _, _, hist2 = o.fit(X, w.astype(np.float32), mu.astype(np.float32), v.astype(np.float32), T - tc, floor,
                               method="gemm", chunk_rows=chunk)
        hist = np.concatenate([hist, hist2])
    comps = np.arange(K) if keep is None else np.sort(np.random.default_rng(7).choice(K, keep, replace=False))
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), f"fit_{name}.npz")
    np.savez_compressed(out, sha256=np.array(digest), law=np.array(law), N=N, D=D, K=K, T=T, checkpoint=tc,
                        var_floor=floor, init_rows=rows, loglik=hist, weights=w.astype(np.float32), comps=comps,
                        means=mu[comps].astype(np.float32), vars=v[comps].astype(np.float32))
    print(f"{name}: {T} iterations in {time.time() - t0:.0f} s, LL {hist[0]:.6e} -> {hist[-1]:.6e}, "
          f"{os.path.getsize(out)} bytes", flush=True)


if __name__ == "__main__":
    for n in (sys.argv[1:] or list(FIXTURES)):
        make(n)
