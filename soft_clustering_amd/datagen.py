"""Seeded synthetic inputs for the five GMM workloads.

This module draws mixture laws and sample rows. It holds none of the EM
arithmetic: both the HIP path and the float64 oracle take their inputs from
here, and nothing here depends on either of them.

Mixture laws (parameters of the *generating* distribution, float64 numpy):
  tiny   N=10,000   D=8    K=16     means U[-10,10], std U[0.5,2], weights Dirichlet(1)
  mid    N=1e6      D=128  K=1024   means N(0, 4^2), std U[0.5,1.5], weights Dirichlet(2)
  large  N=1e8      D=128  K=1024   the mid law (same parameter seed), more rows
  embed  N=1e7      D=768  K=4096   unit-sphere centres, noise variance 1/(1+d/64),
                                    rows L2-normalised, weights Zipf(1.1)
  ivf    N=1e7 base D=128  K=16384  integer values 0..255 stored as fp32: clipped,
                                    rounded Gaussians around 1024 super-centres with
                                    16 sub-centres each
  iso    N=1e8      D=128  K=1024   the mid law with one std per component (isotropic)
Parameters are drawn from numpy ``default_rng(seed)`` in the order
means -> stds -> weights.  Rows are drawn in fixed chunks of ``CHUNK`` rows;
chunk ``c`` uses a torch generator seeded from ``(seed, stream, c)``, so any
row range can be regenerated on its own and a prefix of a large workload is a
prefix of the same data.  On one device the draw is deterministic; the CPU and
GPU generators give different (equally valid) samples.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

CHUNK = 1 << 16  # rows per independently seeded chunk


@dataclass(frozen=True)
class Workload:
    name: str
    N: int
    D: int
    K: int
    iters: int
    var_floor: float
    law: str
    seed: int = 0
    init_seed: int = 1
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    "tiny": Workload("tiny", 10_000, 8, 16, 10, 1e-6, "tiny"),
    "mid": Workload("mid", 1_000_000, 128, 1024, 30, 1e-6, "mid"),
    "large": Workload("large", 100_000_000, 128, 1024, 30, 1e-6, "mid"),
    "embed": Workload("embed", 10_000_000, 768, 4096, 20, 1e-5, "embed"),
    # the pages' isotropic model at the large size
    "iso": Workload("iso", 100_000_000, 128, 1024, 30, 1e-6, "iso"),
    # ivf: EM on a 1e6-row sample, then soft assignment of the 1e7-row base.
    "ivf": Workload("ivf", 10_000_000, 128, 16384, 10, 1.0 / 12.0, "ivf",
                    extra={"train_rows": 1_000_000, "queries": 10_000,
                           "threshold": 0.1, "max_extra": 3,
                           "nprobe": (8, 16, 32, 64)}),
}


@dataclass
class Mixture:
    """Generating law: weights (K,), means (K,D), stds (K,D), plus a row transform."""
    weights: np.ndarray
    means: np.ndarray
    stds: np.ndarray
    law: str

    @property
    def K(self):
        return self.means.shape[0]

    @property
    def D(self):
        return self.means.shape[1]


def mixture(law: str, D: int, K: int, seed: int = 0) -> Mixture:
    """Draw the generating mixture of a law (means, then stds, then weights)."""
    rng = np.random.default_rng(seed)
    if law == "tiny":
        means = rng.uniform(-10.0, 10.0, (K, D))
        stds = rng.uniform(0.5, 2.0, (K, D))
        weights = rng.dirichlet(np.ones(K))
    elif law == "mid":
        means = rng.normal(0.0, 4.0, (K, D))
        stds = rng.uniform(0.5, 1.5, (K, D))
        weights = rng.dirichlet(2.0 * np.ones(K))
    elif law == "iso":
        # the mid law with one standard deviation per component (the pages'
        # isotropic model, Sigma_k = sigma_k^2 I)
        means = rng.normal(0.0, 4.0, (K, D))
        stds = np.repeat(rng.uniform(0.5, 1.5, (K, 1)), D, axis=1)
        weights = rng.dirichlet(2.0 * np.ones(K))
    elif law == "embed":
        c = rng.normal(size=(K, D))
        means = c / np.linalg.norm(c, axis=1, keepdims=True)
        var_d = 1.0 / (1.0 + np.arange(D) / 64.0)
        stds = np.broadcast_to(np.sqrt(var_d), (K, D)).copy()
        weights = (np.arange(K) + 1.0) ** -1.1
        weights = weights / weights.sum()
    elif law == "ivf":
        n_super = max(1, K // 16)
        sup = rng.uniform(40.0, 216.0, (n_super, D))
        means = np.repeat(sup, K // n_super + 1, axis=0)[:K] + rng.normal(0.0, 1.5, (K, D))
        stds = rng.uniform(6.0, 10.0, (K, D))
        weights = np.full(K, 1.0 / K)
    elif law == "separated":
        # well separated components, for recovery tests: means 40 std apart
        means = rng.normal(0.0, 40.0, (K, D))
        stds = rng.uniform(0.5, 1.5, (K, D))
        weights = rng.dirichlet(5.0 * np.ones(K))
    else:
        raise ValueError(f"unknown law {law!r}")
    return Mixture(weights, means, stds, law)


def _chunk_seed(seed: int, stream: int, chunk: int) -> int:
    return (seed * 1_000_003 + stream * 7_919 + chunk * 104_729 + 12_345) % (2**62)


def _draw_chunk(mix: Mixture, chunk: int, seed: int, stream: int, device) -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(_chunk_seed(seed, stream, chunk))
    cdf = torch.as_tensor(np.cumsum(mix.weights), dtype=torch.float64, device=device)
    cdf[-1] = 1.0
    u = torch.rand(CHUNK, generator=g, device=device, dtype=torch.float64)
    labels = torch.searchsorted(cdf, u, right=True).clamp_(max=mix.K - 1)
    noise = torch.randn(CHUNK, mix.D, generator=g, device=device, dtype=torch.float32)
    means = torch.as_tensor(mix.means, dtype=torch.float32, device=device)
    stds = torch.as_tensor(mix.stds, dtype=torch.float32, device=device)
    x = means[labels] + stds[labels] * noise
    if mix.law == "embed":
        x = x / torch.linalg.vector_norm(x, dim=1, keepdim=True)
    elif mix.law == "ivf":
        x = torch.clamp(torch.round(x), 0.0, 255.0)
    return x, labels


def sample_into(out: torch.Tensor, mix: Mixture, start: int = 0, seed: int = 0,
                stream: int = 0, labels_out: torch.Tensor | None = None) -> torch.Tensor:
    """Fill ``out`` (rows x D, fp32, any device, row stride may exceed D) with
    rows [start, start+rows) of the seeded sample of ``mix``."""
    rows = out.shape[0]
    device = out.device
    done = 0
    while done < rows:
        r = start + done
        c, off = divmod(r, CHUNK)
        take = min(CHUNK - off, rows - done)
        x, lab = _draw_chunk(mix, c, seed, stream, device)
        out[done:done + take, : mix.D].copy_(x[off:off + take])
        if labels_out is not None:
            labels_out[done:done + take].copy_(lab[off:off + take])
        done += take
    return out


def sample(mix: Mixture, rows: int, start: int = 0, seed: int = 0, stream: int = 0,
           device="cpu", ldx: int | None = None) -> torch.Tensor:
    """Rows [start, start+rows) as a new fp32 tensor of shape (rows, D).  With
    ``ldx`` > D the tensor is a view into a (rows, ldx) buffer whose padding
    columns hold NaN, so code that reads past column D is caught."""
    D = mix.D
    if ldx is None or ldx == D:
        out = torch.empty(rows, D, dtype=torch.float32, device=device)
        return sample_into(out, mix, start, seed, stream)
    buf = torch.full((rows, ldx), float("nan"), dtype=torch.float32, device=device)
    sample_into(buf, mix, start, seed, stream)
    return buf[:, :D]


def sample_portable(mix: Mixture, rows: int, seed: int = 0) -> np.ndarray:
    """Rows of the law drawn with numpy's PCG64 stream alone (labels by
    inverse CDF of uniforms, then standard normals; elementwise float64
    arithmetic, one rounding to float32).  Unlike ``sample`` (torch
    generators, whose CPU kernels differ between instruction sets), the
    result is the same bytes on any x86-64 host running the same numpy, so
    expected values computed once from it can be stored and checked later
    on another machine.  Returns a (rows, D) float32 array."""
    rng = np.random.default_rng([seed, 0x5EED])
    cdf = np.cumsum(mix.weights)
    cdf[-1] = 1.0
    labels = np.minimum(np.searchsorted(cdf, rng.random(rows), side="right"), mix.K - 1)
    noise = rng.standard_normal((rows, mix.D))
    x = mix.means[labels] + mix.stds[labels] * noise
    if mix.law == "embed":
        # squared norms summed column by column: elementwise operations only,
        # so the order of the additions cannot depend on the host's SIMD width
        ss = x[:, 0] * x[:, 0]
        for d in range(1, mix.D):
            ss = ss + x[:, d] * x[:, d]
        x = x / np.sqrt(ss)[:, None]
    elif mix.law == "ivf":
        x = np.clip(np.round(x), 0.0, 255.0)
    return x.astype(np.float32)


def init_rows(N: int, K: int, seed: int = 1) -> np.ndarray:
    """K distinct row indices drawn without replacement (int64, host)."""
    if K > N:
        raise ValueError("need K <= N distinct rows")
    return np.random.default_rng(seed).choice(N, size=K, replace=False).astype(np.int64)


def query_rows(mix: Mixture, n: int, seed: int = 0, device="cpu") -> torch.Tensor:
    """Held-out queries from the same law on a separate seed stream."""
    return sample(mix, n, 0, seed, stream=2, device=device)


def random_params(K: int, D: int, seed: int, scale: float = 1.0, var_lo: float = 0.3,
                  var_hi: float = 3.0, zero_weights: int = 0):
    """Arbitrary valid fp32 parameters (weights sum to one) for unit tests."""
    rng = np.random.default_rng(seed)
    w = rng.uniform(0.2, 1.0, K)
    if zero_weights:
        w[rng.choice(K, zero_weights, replace=False)] = 0.0
    w = (w / w.sum()).astype(np.float32)
    mu = (scale * rng.normal(size=(K, D))).astype(np.float32)
    var = rng.uniform(var_lo, var_hi, (K, D)).astype(np.float32)
    return w, mu, var


__all__ = ["CHUNK", "WORKLOADS", "Workload", "Mixture", "mixture", "sample", "sample_into", "sample_portable",
           "init_rows", "query_rows", "random_params"]
