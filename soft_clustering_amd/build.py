"""Builds libflashgmm.so (gfx950) in-tree with hipcc.

Usage: python soft_clustering_amd/build.py [--verbose] [--resource-usage] [--incremental]
(loaded by path, so a stale library is never imported while building).
--incremental recompiles only objects older than their source or a header;
the default recompiles everything.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libflashgmm.so")
BUILD = os.path.join(HERE, "_build")
SOURCES = ["gmm_kernels.hip", "gmm_assign.hip", "gmm_lists.hip", "gmm_api.hip"]
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    "-Wall", "-Wno-unused-variable", "-Wno-unused-function",
    # no packed-fp32 instructions in any kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found")
    return p


HEADERS = [os.path.join(CSRC, "gmm_device.h"), os.path.join(CSRC, "gmm_internal.h"),
           os.path.join(ROOT, "include", "flashgmm.h")]


def _stale(src: str, obj: str) -> bool:
    if not os.path.exists(obj):
        return True
    newest = max(os.path.getmtime(p) for p in [os.path.join(CSRC, src), *HEADERS] if os.path.exists(p))
    return os.path.getmtime(obj) < newest


def _compile(src: str, verbose: bool, resource: bool, incremental: bool = False) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    if incremental and not resource and not _stale(src, obj):
        return obj
    cmd = [hipcc(), *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if resource:
        cmd += ["-Rpass-analysis=kernel-resource-usage"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msgs}")
    if msgs.strip() and (verbose or resource):
        print(msgs, flush=True)
    return obj


def build(verbose: bool = False, resource: bool = False, incremental: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    with ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, resource, incremental), srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv, resource="--resource-usage" in sys.argv,
                incremental="--incremental" in sys.argv))
