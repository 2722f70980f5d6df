"""C-ABI contract checks that need no GPU: the library loads, exports every
symbol the header declares, and rejects bad arguments before touching a
device; the product package never reaches into the oracle."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flashgmm.h")


def header_symbols():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gmm_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    from soft_clustering_amd import LIB_PATH, EXPORTS
    syms = header_symbols()
    assert set(syms) == set(EXPORTS), "binding and header disagree"
    out = subprocess.run(["nm", "-D", "--defined-only", LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (gmm_[a-z_]+)$", out, flags=re.M))
    missing = set(syms) - exported
    assert not missing, f"not exported: {missing}"


def test_create_rejects_bad_sizes_without_gpu():
    from soft_clustering_amd import raw_library
    lib = raw_library()
    h = ctypes.c_void_p()
    for K, D in [(0, 8), (65537, 8), (16, 0), (16, 1025), (-1, 4)]:
        st = lib.gmm_create(ctypes.byref(h), K, D, None)
        assert st == 1, (K, D, st)
        assert b"must be in" in lib.gmm_last_error(None)
    assert lib.gmm_create(None, 4, 4, None) == 1
    assert lib.gmm_workspace_bytes(0, 8) == 0
    lib.gmm_destroy(None)  # NULL-safe


def test_null_context_is_invalid_arg():
    from soft_clustering_amd import raw_library
    lib = raw_library()
    assert lib.gmm_check(None) == 1
    assert lib.gmm_set_path(None, 0) == 1
    assert lib.gmm_fit(None, None, 1, 8, 1, 1e-6, None, None, None, None) == 1


def test_product_path_does_not_use_the_oracle():
    pkg = os.path.join(ROOT, "soft_clustering_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                src = open(os.path.join(dirpath, f)).read()
                code = re.sub(r"#.*|//.*", "", src)
                assert "import oracle" not in code and "from oracle" not in code, f"{f} imports the oracle"


def test_gpu_required_without_device():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    from soft_clustering_amd import GMM
    with pytest.raises(RuntimeError):
        GMM(4, 4)


def test_sanitizer_exercise_calls_every_entry_point():
    """tests/native/abi_exercise.cpp, the host program run under AddressSanitizer
    and UndefinedBehaviorSanitizer, reaches every function the header declares."""
    src = open(os.path.join(ROOT, "tests", "native", "abi_exercise.cpp")).read()
    called = set(re.findall(r"\b(gmm_[a-z_]+)\s*\(", src))
    missing = set(header_symbols()) - called
    assert not missing, f"not exercised: {sorted(missing)}"
    build = open(os.path.join(ROOT, "tests", "native", "build_sanitized.sh")).read()
    for line in build.splitlines():
        # sanitizers on host code only: outside the host link of objects, each
        # -fsanitize= sits behind -Xarch_host
        code = line.split("#")[0]
        if code.strip().startswith('"$CLANG"'):
            assert ".hip" not in code, line
            continue
        for m in re.finditer(r"(\S+)\s+-fsanitize=", code):
            assert m.group(1).endswith("-Xarch_host"), line
