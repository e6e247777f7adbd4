"""The CPU tests of the host code under AddressSanitizer + UndefinedBehaviorSanitizer.

Two builds of the same sources, each run in a child pytest with its sanitizer runtime preloaded
(gcc's and clang's runtimes cannot share a process):
  * the oracle (g++ -fsanitize=address,undefined) under the oracle pin tests;
  * libkvarn with sanitized host code (hipcc -Xarch_host -fsanitize=...; device code unchanged) under
    the C-ABI boundary tests and the page-pool tests (argument checks, sizes, the host page pool).
Any sanitizer report ends the child with a non-zero status (UBSan set not to recover)."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def _clang_asan():
    base = "/opt/rocm/lib/llvm/lib/clang"
    if not os.path.isdir(base):
        return None
    for ver in sorted(os.listdir(base), reverse=True):
        p = os.path.join(base, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(p):
            return p
    return None


def _gcc_asan():
    try:
        p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    except OSError:
        return None
    return p if os.path.isabs(p) and os.path.exists(p) else None


def _child(env_extra, tests, log):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0:exitcode=97"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu"]
                         + tests, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, f"{log}: exit {res.returncode}\n{res.stdout[-3000:]}\n{res.stderr[-3000:]}"
    assert " passed" in res.stdout, res.stdout[-2000:]


def test_oracle_under_asan_ubsan():
    if shutil.which("g++") is None or _gcc_asan() is None:
        pytest.skip("g++ or its libasan not available")
    from oracle import build as obuild
    lib = obuild.build(sanitize=True)
    _child({"LD_PRELOAD": _gcc_asan(), "KVARN_ORACLE_LIB": lib}, ["tests/test_oracle_pins.py"], "oracle pins")


def test_host_layer_under_asan_ubsan():
    if shutil.which("hipcc") is None or _clang_asan() is None:
        pytest.skip("hipcc or clang's ASan runtime not available")
    from kv_cache_quantization_pipeline_amd import build as kbuild
    lib = kbuild.build(sanitize=True)
    _child({"LD_PRELOAD": _clang_asan(), "KVARN_LIB": lib}, ["tests/test_boundary.py", "tests/test_page_pool.py"],
           "C-ABI boundary and page pool")
