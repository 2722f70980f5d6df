"""Benchmark of the fused diagonal-GMM EM step on one MI355X.

A step is one EM iteration (log-densities, log-sum-exp, responsibilities,
sufficient statistics, deterministic reduction, M-step) over the whole data
set, which is resident in HBM before timing starts.  The default workload is
N=100M rows, D=128, K=1024 fp32 (51.2 GB of X), 30 iterations; data and the
mixture law are seeded synthetic (see soft_clustering_amd/datagen.py).

Prints one JSON line with the throughput (useful GFLOP/s: N*K*(8D+2) per
iteration), ms per iteration, the roofline of the dominant kernel measured
with HIP events around each of its launches, and the float64 oracle timed on
a bounded row sample on this host.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

MFMA_FP32_PEAK_TFLOPS = 157.3  # MI355X dense fp32 matrix, AMD published figure
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix, AMD published figure
MFMA_FP64_PEAK_TFLOPS = 78.6  # MI355X dense fp64 matrix, AMD published figure
HBM_PEAK_GBS = 8000.0

# The configured workloads; the timed iterations are --steps (after --warmup
# untimed ones), and the line reports what 30 iterations (the configured run
# of the large and mid workloads) take at the measured rate.
WORKLOAD_TEXT = {
    "large": "large EM: N=100,000,000, D=128, K=1024, fp32, diagonal covariance (configured run: 30 EM iterations)",
    "mid": "mid EM: N=1,000,000, D=128, K=1024, fp32, diagonal covariance (configured run: 30 EM iterations)",
    "tiny": "tiny EM: N=10,000, D=8, K=16, fp32, diagonal covariance (configured run: 10 EM iterations)",
    "embed": "embedding-like EM: N=10,000,000, D=768, K=4096, fp32, diagonal covariance "
             "(configured run: 20 EM iterations)",
    "iso": "isotropic EM (sigma_k^2 I): N=100,000,000, D=128, K=1024, fp32 (30 EM iterations as the large run)",
    "stream": "out-of-core EM: the large data (N=100,000,000, D=128, K=1024) in pinned host memory, streamed in "
              "2^24-row chunks",
    "kmeans": "k-means warm start: Lloyd iterations at N=100,000,000, D=128, K=1024 (the large data), fp32",
    "ivf": "IVF: EM on a 1,000,000-row sample, D=128, K=16384, integer values 0..255 (configured run: 10 EM "
           "iterations); soft assignment (argmax + up to 3 with r >= 0.1) of 10,000,000 base rows into CSR lists; "
           "10,000 queries probed at nprobe 8, 16, 32, 64 with recall@10 against exact search",
}
CONFIGURED_ITERS = {"large": 30, "mid": 30, "tiny": 10, "embed": 20, "iso": 30, "ivf": 10}


def useful_flops(N, K, D, iso=False):
    """Diagonal: [x^2, x] logit contraction (4D per pair) + r^T[1, x, x^2]
    statistics (2(2D+1)).  Isotropic: x.mu/s^2 plus the ||x||^2 term (2D+2)
    + r^T[1, x, ||x||^2] (2(D+2)); run on the diagonal kernels, which issue
    the diagonal count."""
    return float(N) * K * ((4 * D + 6) if iso else (8 * D + 2))


def mfma_roofline(N, K, D, split, iso=False, f64=False, sweeps=1):
    """Peak for the E-step: the rate at which the matrix pipes, fully busy
    with its MFMA instruction mix, would deliver its useful flops.  The
    logit and statistics contractions take 2*N*K*F flops each over F
    features (F = 2D diagonal, D isotropic); the two-sweep path (sweeps = 2)
    contracts the logits twice.  split 0: every contraction fp32 MFMA.
    split 1: the logits are three bf16 passes at the bf16 peak, the
    statistics fp32 at the fp32 peak.  split 2: the statistics are six bf16
    passes too.  f64: float64 MFMA logits at the fp64 peak, fp32 statistics.
    The peak is the useful count over that busy time."""
    F = D if iso else 2 * D
    if f64 or not split:
        lpeak = MFMA_FP64_PEAK_TFLOPS if f64 else MFMA_FP32_PEAK_TFLOPS
        t_busy = (sweeps * 2.0 * N * K * F / (lpeak * 1e12)
                  + 2.0 * N * K * F / (MFMA_FP32_PEAK_TFLOPS * 1e12))
        peak = useful_flops(N, K, D, iso) / t_busy / 1e12
        return peak, (f"matrix pipes busy with this mix: logits {sweeps} time(s) over F={'D' if iso else '2D'} "
                      f"features in {'fp64' if f64 else 'fp32'} (2*N*K*F flops each at {lpeak} TFLOP/s) + "
                      f"statistics in fp32 (2*N*K*F at 157.3 TFLOP/s); useful N*K*({'4D+6' if iso else '8D+2'}) "
                      f"over that time")
    bf16_passes = 3 + (6 if split == 2 else 0)
    t_busy = bf16_passes * 2.0 * N * K * F / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    if split == 1:
        t_busy += 2.0 * N * K * F / (MFMA_FP32_PEAK_TFLOPS * 1e12)
    peak = useful_flops(N, K, D, iso) / t_busy / 1e12
    f = "D" if iso else "2D"
    stats = ("statistics as 6 bf16 passes (12*N*K*F at 2500 TFLOP/s)" if split == 2 else
             "statistics in fp32 (2*N*K*F at 157.3 TFLOP/s)")
    return peak, (f"matrix pipes busy with this kernel's mix: logits over F={f} features as 3 bf16 passes "
                  f"(6*N*K*F flops at 2500 TFLOP/s) + {stats}; useful N*K*({'4D+6' if iso else '8D+2'}) over "
                  f"that time")


TRAFFIC_PROFILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                               "k_stats_fused_large_traffic.md")
COUNTER_PROFILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                               "k_stats_fused_large_counters.md")
SIMDS = 1024          # 256 CUs x 4 SIMDs
CLOCK_HZ = 2.4e9      # MI355X peak engine clock


def kernel_source_hash(root=None):
    """sha256 prefix of the fused E-step's source: the text of k_stats (from its
    heading comment to the next kernel's) and the device code it includes."""
    import hashlib
    base = os.path.join(root or os.path.dirname(os.path.abspath(__file__)), "soft_clustering_amd", "csrc")
    src = open(os.path.join(base, "gmm_kernels.hip")).read()
    i = src.index("// E-step statistics sweep.")
    j = src.index("// First sweep of the two-sweep path", i)
    h = hashlib.sha256()
    h.update(src[i:j].encode())
    with open(os.path.join(base, "gmm_device.h"), "rb") as fh:
        h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch of the fused E-step on the large workload, from the
    committed FETCH_SIZE + WRITE_SIZE counter summary (each counter scaled by
    what it reads for a copy of known size), or None when the kernel sources
    have changed since those counters were taken."""
    return profile_field(TRAFFIC_PROFILE, "traffic_bytes_per_launch")


def profile_field(path, name):
    """A numeric field ("name: value" line) of a committed profile summary,
    or None when the file is missing or the fused E-step's source has changed
    since the counters in it were taken (its source_hash no longer matches)."""
    try:
        with open(path) as fh:
            text = fh.read()
    except OSError:
        return None
    fields = {}
    for ln in text.splitlines():
        if ":" in ln and ln.split(":", 1)[0] in (name, "source_hash"):
            k, v = ln.split(":", 1)
            fields[k] = v.strip()
    if fields.get("source_hash") != kernel_source_hash() or name not in fields:
        return None
    return float(fields[name])


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_rate(O, X, w, mu, var, n, floor, budget_s, max_iters):
    """Seconds per EM iteration of the oracle on X (at least one iteration)."""
    t0 = time.perf_counter()
    iters = 0
    while True:
        Nk, S1, S2, ll = O.estep_stats(X, w, mu, var, method="gemm")  # S2: Q for the isotropic model
        w, mu, var = O.mstep(Nk, S1, S2, n, floor, mu, var)
        iters += 1
        if time.perf_counter() - t0 > budget_s or iters >= max_iters:
            break
    return (time.perf_counter() - t0) / iters, iters


def cpu_baseline(workload, sample_rows, budget_s):
    """Time the oracle as it stands on a prefix of the same data with every
    host core, then once more on one thread on a tenth of that prefix,
    each scaled to ms per EM iteration at the full N (EM cost is linear in N)."""
    import torch
    from threadpoolctl import threadpool_limits
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    from soft_clustering_amd import datagen
    iso = workload == "iso"
    if iso:
        import oracle.gmm_oracle_iso as O
    else:
        import oracle.gmm_oracle as O
    wl = datagen.WORKLOADS[workload]
    mix = datagen.mixture(wl.law, wl.D, wl.K, seed=wl.seed)
    n = min(sample_rows, wl.N)
    X = datagen.sample(mix, n, seed=wl.seed).numpy()
    rows = datagen.init_rows(n, wl.K, seed=wl.init_seed)
    w, mu, var = O.init(X, rows, wl.var_floor)
    from threadpoolctl import threadpool_info
    blas = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
    cores = max(blas) if blas else 1  # the threads the oracle's BLAS calls use
    dt, iters = _oracle_rate(O, X, w, mu, var, n, wl.var_floor, budget_s, 3)
    n1 = max(wl.K, n // 10)
    with threadpool_limits(limits=1):
        dt1, iters1 = _oracle_rate(O, X[:n1], w, mu, var, n1, wl.var_floor, budget_s / 2, 1)
    n_full = wl.extra.get("train_rows", wl.N)  # EM runs on the training sample for ivf
    ms_full = dt * 1e3 * (n_full / n)
    return {"value": ms_full, "unit": "ms per EM iteration (extrapolated linearly in N)", "cores": cores,
            "kind": "oracle",
            "sample": f"{iters} EM iteration(s) of the float64 numpy oracle on the first {n} rows of the "
                      f"{workload} workload ({dt:.2f} s each, BLAS on {cores} threads of "
                      f"{len(os.sched_getaffinity(0))} host CPUs), scaled by {n_full}/{n}",
            "gflops": useful_flops(n, wl.K, wl.D, iso) / dt / 1e9,
            "cpu_model": cpu_model(),
            "torch_threads": torch.get_num_threads(),
            "one_thread": {"value": dt1 * 1e3 * (n_full / n1), "unit": "ms per EM iteration (extrapolated)",
                           "cores": 1, "sample": f"{iters1} EM iteration(s) on the first {n1} rows "
                                                 f"({dt1:.2f} s each) on one BLAS thread",
                           "gflops": useful_flops(n1, wl.K, wl.D, iso) / dt1 / 1e9}}


def bench_stream(args):
    """EM with X in pinned host memory: every iteration copies all of X over
    PCIe in chunks (a copy stream, two device staging buffers) while the
    E-step of the previous chunk runs.  The value is PCIe-inclusive."""
    import torch
    from soft_clustering_amd import GMM, datagen
    wl = datagen.WORKLOADS["large"]
    N = args.rows or wl.N
    K, D = wl.K, wl.D
    chunk = 1 << 24
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    mix = datagen.mixture(wl.law, D, K, seed=wl.seed)
    t0 = time.perf_counter()
    Xh = torch.empty(N, D, dtype=torch.float32, pin_memory=True)
    tmp = torch.empty(min(chunk, N), D, dtype=torch.float32, device=dev)
    for r0 in range(0, N, chunk):
        rows = min(chunk, N - r0)
        datagen.sample_into(tmp[:rows], mix, r0, seed=wl.seed)
        Xh[r0:r0 + rows].copy_(tmp[:rows])
    torch.cuda.synchronize()
    print(f"# {N}x{D} in pinned host memory in {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)
    g = GMM(K, D, dev)
    n0 = min(N, 1_000_000)  # initialisation from the first rows (the same rule)
    Xd = Xh[:n0].to(dev)
    w, mu, var = g.init(Xd, datagen.init_rows(n0, K, seed=wl.init_seed), wl.var_floor)
    del Xd, tmp
    if args.warmup > 0:
        g.fit_host(Xh, w, mu, var, args.warmup, wl.var_floor, chunk)
    g.check()
    torch.cuda.synchronize()
    hist = torch.zeros(args.steps, dtype=torch.float64, device=dev)
    t0 = time.perf_counter()
    g.fit_host(Xh, w, mu, var, args.steps, wl.var_floor, chunk, hist)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    g.check()
    g.close()
    ms = dt * 1e3 / args.steps
    F = useful_flops(N, K, D)
    line = {"metric": "ms per EM iteration with X streamed from pinned host memory (PCIe-inclusive)",
            "value": round(F / (dt / args.steps) / 1e9, 1), "unit": "GFLOP/s (useful: N*K*(8D+2) per EM iteration)",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 3),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
            "data": "synthetic (seeded mixture, generated on the GPU, held in pinned host memory)",
            "config": {"workload": WORKLOAD_TEXT["stream"], "N": N, "K": K, "D": D, "chunk_rows": chunk},
            "h2d_gbs": round(N * D * 4 / (dt / args.steps) / 1e9, 1),
            "loglik_first_last": [float(hist[0]), float(hist[-1])]}
    print(json.dumps(line), flush=True)


def bench_kmeans(args):
    """Lloyd iterations of the k-means warm start on the large data set.  Each
    is one sweep of the fused isotropic E-step kernel in its hard mode
    (nearest centre per row, one-hot statistics) and a centre update from the
    sums; FLASHGMM_KMEANS_FUSED=0 selects the list path instead (two logit
    sweeps of the soft-assignment kernels into CSR lists, then a gather pass
    over X), which needs the lists as scratch."""
    import torch
    from soft_clustering_amd import GMM, datagen
    wl = datagen.WORKLOADS["large"]
    N = args.rows or wl.N
    K, D = wl.K, wl.D
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    mix = datagen.mixture(wl.law, D, K, seed=wl.seed)
    X = torch.empty(N, D, dtype=torch.float32, device=dev)
    datagen.sample_into(X, mix, 0, seed=wl.seed)
    rows = torch.as_tensor(datagen.init_rows(N, K, seed=wl.init_seed), device=dev)
    c = X[rows].contiguous()
    g = GMM(K, D, dev)
    lists = os.environ.get("FLASHGMM_KMEANS_FUSED", "1").strip() == "0"
    split = 0 if lists else g.split_level(2)
    if args.warmup > 0:
        g.kmeans(X, c, args.warmup, lists=lists)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    _, counts, _, _ = g.kmeans(X, c, args.steps, lists=lists)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    g.close()
    ms = dt * 1e3 / args.steps
    useful = 2.0 * N * K * D  # the x.c products of the distances
    line = {"metric": "ms per Lloyd iteration (k-means warm start)", "value": round(ms, 3), "unit": "ms",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 3),
            "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
            "data": "synthetic (seeded mixture, generated on the GPU)",
            "config": {"workload": WORKLOAD_TEXT["kmeans"], "N": N, "K": K, "D": D,
                       "path": "lists" if lists else "fused",
                       "mfma": ["fp32", "split-bf16 logits", "split-bf16 logits and statistics"][split]},
            "distance_tflops": round(useful / (dt / args.steps) / 1e12, 2),
            # MFMA work issued per iteration: the list path runs two logit sweeps
            # over the 2D expanded features; the fused sweep runs the logits over
            # D features (three bf16 passes when split) and the one-hot
            # statistics product over D (three bf16 passes when split: r is
            # exact in bf16)
            "issued_mfma_tflops": round((8.0 if lists else {0: 4.0, 1: 8.0, 2: 12.0}[split]) * N * K * D
                                        / (dt / args.steps) / 1e12, 2),
            "empty_clusters": int((counts == 0).sum().item())}
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="large", choices=sorted(WORKLOAD_TEXT))
    ap.add_argument("--path", default="auto", choices=["auto", "fused", "two_sweep"])
    ap.add_argument("--precision", default=None, choices=["refined", "fp32", "fp64"],
                    help="logit precision (default: refined; fp64 for the embed workload, whose diffuse "
                         "responsibilities would have a large share of the logits refined)")
    ap.add_argument("--mfma", default="split", choices=["split", "split-logits", "fp32"],
                    help="matrix instructions of the fused refined E-step: split-bf16 logits and statistics, "
                         "split-bf16 logits only, or fp32")
    ap.add_argument("--rows", type=int, default=0, help="override N (testing only)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-recall", action="store_true", help="ivf: skip the probe / recall@10 evaluation")
    ap.add_argument("--cpu-sample-rows", type=int, default=250_000)
    ap.add_argument("--cpu-budget-s", type=float, default=20.0)
    ap.add_argument("--copy-calibration", type=float, default=0.0, metavar="GIB",
                    help="only copy GIB GiB device-to-device three times (a known-size kernel that scales "
                         "the FETCH_SIZE / WRITE_SIZE counters) and exit")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the EM step here is built and measured "
              "on a single MI355X, with no multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.workload == "kmeans":
        return bench_kmeans(args)
    if args.workload == "stream":
        return bench_stream(args)
    if args.copy_calibration > 0:
        n = int(args.copy_calibration * (1 << 30)) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": n * 4, "launches": 3}), flush=True)
        return
    from soft_clustering_amd import (GMM, MFMA_FP32, MFMA_SPLIT_BF16, MFMA_SPLIT_LOGITS, PATH_AUTO, PATH_FUSED,
                                     PATH_TWO_SWEEP, PREC_FP32, PREC_FP64, PREC_REFINED, datagen)

    wl = datagen.WORKLOADS[args.workload]
    if args.precision is None:
        args.precision = "fp64" if args.workload == "embed" else "refined"
    ivf = args.workload == "ivf"
    iso = args.workload == "iso"
    N = args.rows or (wl.extra["train_rows"] if ivf else wl.N)
    K, D = wl.K, wl.D
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    mix = datagen.mixture(wl.law, D, K, seed=wl.seed)
    t0 = time.perf_counter()
    X = torch.empty(N, D, dtype=torch.float32, device=dev)
    datagen.sample_into(X, mix, 0, seed=wl.seed, stream=1 if ivf else 0)
    torch.cuda.synchronize()
    print(f"# generated {N}x{D} in {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)

    g = GMM(K, D, dev)
    g.set_path({"auto": PATH_AUTO, "fused": PATH_FUSED, "two_sweep": PATH_TWO_SWEEP}[args.path])
    g.set_precision({"refined": PREC_REFINED, "fp32": PREC_FP32, "fp64": PREC_FP64}[args.precision])
    g.set_mfma({"split": MFMA_SPLIT_BF16, "split-logits": MFMA_SPLIT_LOGITS, "fp32": MFMA_FP32}[args.mfma])
    split = g.split_level(1 if iso else 0)
    init = g.init_iso if iso else g.init
    fit = g.fit_iso if iso else g.fit
    w, mu, var = init(X, datagen.init_rows(N, K, seed=wl.init_seed), wl.var_floor)
    hist_w = torch.zeros(max(args.warmup, 1), dtype=torch.float64, device=dev)
    if args.warmup > 0:
        fit(X, w, mu, var, args.warmup, wl.var_floor, hist_w)
    g.check()
    torch.cuda.synchronize()

    hist = torch.zeros(args.steps, dtype=torch.float64, device=dev)
    g.profile(True)
    g.profile_read()
    g.refine_stats()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    fit(X, w, mu, var, args.steps, wl.var_floor, hist)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    stats_ms, stats_n, logz_ms, logz_n = g.profile_read()
    n_ref, n_logits = g.refine_stats()
    g.profile(False)
    g.check()

    ms_step = dt * 1e3 / args.steps
    F = useful_flops(N, K, D, iso)
    gflops = F / (dt / args.steps) / 1e9
    fused = logz_n == 0
    # dominant kernel: fused path, the one E-step launch per iteration
    # (algorithmic flops per launch N*K*(8D+2)); two-sweep path, the pair of
    # sweeps (log Z sweep + statistics sweep, launched per row chunk), charged
    # with the same useful flops per iteration (the logit recomputation of the
    # second sweep is not counted)
    kern_ms = (stats_ms + logz_ms) / args.steps  # per iteration
    avg_ms = stats_ms / max(stats_n, 1)
    achieved = F / (kern_ms * 1e-3) / 1e12
    hl = hist.cpu().numpy()
    peak, peak_basis = mfma_roofline(N, K, D, split, iso, f64=args.precision == "fp64", sweeps=1 if fused else 2)
    traffic = None
    busy_cycles = None
    if fused and split == 2 and args.workload == "large" and args.precision == "refined" and not args.rows:
        # taken on the default kernel (split-bf16 logits and statistics)
        traffic = measured_traffic()
        busy_cycles = profile_field(COUNTER_PROFILE, "mfma_busy_cycles_per_launch")
    line = {
        "metric": "ms per EM iteration and GFLOP/s at N=100M,K=1024,D=128 fp32; % MFMA peak",
        "value": round(gflops, 1),
        "unit": "GFLOP/s (useful: N*K*(" + ("4D+6" if iso else "8D+2") + ") per EM iteration)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic (seeded mixture, generated on the GPU)",
        "config": {"workload": WORKLOAD_TEXT[args.workload] if not args.rows else
                   f"{args.workload} law with N={N}", "N": N, "K": K, "D": D,
                   "path": "fused" if fused else "two_sweep", "logit_precision": args.precision,
                   "mfma": ["fp32", "split-bf16 logits", "split-bf16 logits and statistics"][split],
                   "covariance": "isotropic" if iso else "diagonal"},
        "pct_fp32_mfma_peak": round(100 * gflops / (MFMA_FP32_PEAK_TFLOPS * 1e3), 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": round(peak, 1),
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "peak_basis": peak_basis,
                     "fp32_peak_frac": round(achieved / MFMA_FP32_PEAK_TFLOPS, 4),
                     "traffic": traffic,
                     # matrix-pipe busy cycles per launch from the committed
                     # counter summary (SQ_VALU_MFMA_BUSY_CYCLES) over this
                     # run's launch time x 1024 SIMDs x 2.4 GHz
                     "mfma_busy_from_counters": (round(busy_cycles / (avg_ms * 1e-3 * CLOCK_HZ * SIMDS), 4)
                                                 if busy_cycles else None),
                     "traffic_unit": "HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                     "kernel": ("k_stats (fused E-step" + ["", ", split-bf16 logits", ", split-bf16 logits and statistics"][split]
                                + ")") if fused
                     else "k_logz + k_stats (two-sweep E-step)",
                     "kernel_ms_per_iteration": round(kern_ms, 3),
                     "avg_launch_ms": round(avg_ms, 3), "launches": stats_n + logz_n},
        "loglik_first_last": [float(hl[0]), float(hl[-1])],
        "configured_iterations": CONFIGURED_ITERS.get(args.workload),
        "configured_run_ms": (round(ms_step * CONFIGURED_ITERS[args.workload], 1)
                              if args.workload in CONFIGURED_ITERS else None),
        "configured_run_ms_basis": "configured iterations x the measured ms per timed iteration",
        "refined_logit_fraction": n_ref / max(n_logits, 1.0),
        "x_hbm_gbs_once": round(N * D * 4 / (avg_ms * 1e-3) / 1e9, 1),
    }
    if not fused:
        line["logz_sweep_avg_ms"] = round(logz_ms / max(logz_n, 1), 3)
    del X
    torch.cuda.empty_cache()
    if ivf:
        # soft assignment of the base rows with the trained parameters
        nb = wl.N
        Xb = torch.empty(nb, D, dtype=torch.float32, device=dev)
        datagen.sample_into(Xb, mix, 0, seed=wl.seed)
        thr, m = wl.extra["threshold"], wl.extra["max_extra"]
        g.soft_assign(Xb, w, mu, var, thr, m)  # warm-up
        torch.cuda.synchronize()
        g.refine_stats()
        t0 = time.perf_counter()
        offsets, ids = g.soft_assign(Xb, w, mu, var, thr, m)
        torch.cuda.synchronize()
        dt_a = time.perf_counter() - t0
        n_ref_a, _ = g.refine_stats()
        # one logit sweep over the base (the selections of the counting pass
        # are kept for the scatter): 4*N*K*D flops of the expanded quadratic
        line["soft_assign"] = {"rows": nb, "ms": round(dt_a * 1e3, 1), "lists_per_row": round(ids.shape[0] / nb, 4),
                               "logit_sweeps": 1,
                               "logit_tflops": round(4.0 * nb * K * D / dt_a / 1e12, 2),
                               "refined_logit_fraction": n_ref_a / (nb * K)}
        del offsets, ids
        # the pages' own rule: argmax plus the second-best component when its
        # responsibility exceeds tau, tau in {0.5, 1, 2} / K
        top2 = []
        for f in (0.5, 1.0, 2.0):
            tau = f / K
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            offsets, ids = g.soft_assign(Xb, w, mu, var, tau, 1)
            torch.cuda.synchronize()
            dt_t = time.perf_counter() - t0
            top2.append({"tau_times_K": f, "ms": round(dt_t * 1e3, 1), "lists_per_row": round(ids.shape[0] / nb, 4)})
            del offsets, ids
        line["soft_assign_top2"] = top2
        if not args.no_recall:
            line["ivf_search"] = ivf_recall(g, Xb, w, mu, var, mix, wl, dev)
        del Xb
        torch.cuda.empty_cache()
    g.close()
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(args.workload, args.cpu_sample_rows, args.cpu_budget_s)
    print(json.dumps(line), flush=True)


def ivf_recall(g, Xb, w, mu, var, mix, wl, dev):
    """Recall@10 and distance computations of IVF search over the lists of
    each assignment rule: argmax only, the configured multi-assignment
    (argmax + up to 3 with r >= 0.1) and the pages' top-2 rule at tau in
    {0.5, 1, 2}/K; queries probe nprobe in {8, 16, 32, 64} nearest means."""
    import torch
    from soft_clustering_amd import datagen, ivf_probe
    K = wl.K
    Q = datagen.query_rows(mix, wl.extra["queries"], seed=wl.seed, device=dev)
    t0 = time.perf_counter()
    truth, _ = ivf_probe.exact_topk(Q, Xb, 10)
    torch.cuda.synchronize()
    out = {"queries": int(Q.shape[0]), "exact_topk_s": round(time.perf_counter() - t0, 2), "rules": []}
    rules = [("argmax", 1.0, 0), (f"argmax+{wl.extra['max_extra']}@r>={wl.extra['threshold']}",
                                  wl.extra["threshold"], wl.extra["max_extra"])]
    rules += [(f"top2@tau={f}/K", f / K, 1) for f in (0.5, 1.0, 2.0)]
    nb = Xb.shape[0]
    for name, thr, m in rules:
        offsets, ids = g.soft_assign(Xb, w, mu, var, thr, m)
        mbar = ids.shape[0] / nb
        pts = []
        for nprobe in wl.extra["nprobe"]:
            t0 = time.perf_counter()
            found, _, dco = ivf_probe.search(Q, Xb, offsets, ids, mu, nprobe)
            torch.cuda.synchronize()
            r10, r1 = ivf_probe.recall(found, truth)
            pts.append({"nprobe": nprobe, "recall@10": round(r10, 4), "1-recall@10": round(r1, 4),
                        "dco_mean": round(float(dco.to(torch.float64).mean()), 1),
                        "dco_identity": round(ivf_probe.dco_identity(offsets, nb, nprobe), 1),
                        "search_s": round(time.perf_counter() - t0, 2)})
        out["rules"].append({"rule": name, "lists_per_row": round(mbar, 4), "points": pts})
        del offsets, ids
    return out


if __name__ == "__main__":
    main()
