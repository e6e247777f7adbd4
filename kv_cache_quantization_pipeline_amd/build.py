"""Compile the HIP sources of libkvarn for gfx950 into an in-tree shared library.

hipcc, -O3, packed fp32 instructions disabled for device code.  Each translation unit is compiled
to an object in parallel (decode.hip once per number of quantisation groups per token), then the
objects are linked.  The library is written next to this file as libkvarn.so and loaded by the
binding.
"""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkvarn.so")
ARCH = "gfx950"
# (source, extra defines, object name)
UNITS = [
    ("libkvarn.hip", [], "libkvarn.o"),
    ("quantize.hip", [], "quantize.o"),
    ("decode.hip", ["-DKVARN_DECODE_NG=1"], "decode_ng1.o"),
    ("decode.hip", ["-DKVARN_DECODE_NG=2"], "decode_ng2.o"),
    ("decode.hip", ["-DKVARN_DECODE_NG=4"], "decode_ng4.o"),
    ("prefill.hip", ["-DKVARN_PREFILL_NG=1"], "prefill_ng1.o"),
    ("prefill.hip", ["-DKVARN_PREFILL_NG=2"], "prefill_ng2.o"),
    ("prefill.hip", ["-DKVARN_PREFILL_NG=4"], "prefill_ng4.o"),
    ("page_pool.cpp", [], "page_pool.o"),
]
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include")]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed: " + " ".join(cmd[-3:]))


SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]


def build(verbose: bool = False, extra=(), sanitize: bool = False) -> str:
    """Build libkvarn.so; with sanitize=True, a copy whose host code carries AddressSanitizer and
    UndefinedBehaviorSanitizer (device code unchanged) into <repo>/_build/libkvarn_san.so, for the CPU
    tests of the host layer (load it with clang's ASan runtime preloaded)."""
    lib = os.path.join(ROOT, "_build", "libkvarn_san.so") if sanitize else LIB
    flags = FLAGS + (SAN_FLAGS if sanitize else [])
    os.makedirs(os.path.dirname(lib), exist_ok=True)
    with tempfile.TemporaryDirectory(prefix="kvarn_build_") as tmp:
        jobs = []
        for src, defs, obj in UNITS:
            jobs.append(["hipcc", "-c"] + flags + list(extra) + defs +
                        ["-o", os.path.join(tmp, obj), os.path.join(CSRC, src)])
        workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
        with ThreadPoolExecutor(max_workers=workers) as ex:
            for f in [ex.submit(_run, j, verbose) for j in jobs]:
                f.result()
        link = ["hipcc", "-shared", f"--offload-arch={ARCH}", "-o", lib + ".tmp"]
        if sanitize:
            link += ["-shared-libsan", "-fsanitize=address,undefined"]
        _run(link + [os.path.join(tmp, obj) for _, _, obj in UNITS], verbose)
    os.replace(lib + ".tmp", lib)
    return lib


# stand-alone timing programs (not part of the library), built into <repo>/_build/
PROBES = [("probes/rotation_probe.hip", "rotation_probe")]


def build_probes(verbose: bool = False) -> list:
    out_dir = os.path.join(ROOT, "_build")
    os.makedirs(out_dir, exist_ok=True)
    outs = []
    for src, name in PROBES:
        out = os.path.join(out_dir, name)
        _run(["hipcc", "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
              "-packed-fp32-ops", "-o", out, os.path.join(HERE, src)], verbose)
        outs.append(out)
    return outs


if __name__ == "__main__":
    build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv)
    if "--probes" in sys.argv:
        build_probes(verbose="-v" in sys.argv)
