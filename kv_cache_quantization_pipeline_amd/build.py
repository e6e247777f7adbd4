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


def _short_name(mangled: str) -> str:
    """kernel<template ints> from an Itanium-mangled kernel name of this library."""
    import re
    m = re.match(r"_ZN5kvarn(?:12_GLOBAL__N_1)?(\d+)", mangled)
    if not m:
        return mangled
    n = int(m.group(1))
    name = mangled[m.end():m.end() + n]
    rest = mangled[m.end() + n:]
    args = re.match(r"I((?:Li-?\d+E)+)E", rest)
    return name + ("<" + ", ".join(re.findall(r"Li(-?\d+)E", args.group(1))) + ">" if args else "")


def resource_usage(verbose: bool = False) -> str:
    """Compile every unit with -Rpass-analysis=kernel-resource-usage (objects discarded) and return a
    markdown table of each kernel's VGPRs, AGPRs, scratch bytes per lane, occupancy and LDS bytes."""
    import re

    def one(unit, tmp):
        src, defs, obj = unit
        cmd = ["hipcc", "-c"] + FLAGS + defs + ["-Rpass-analysis=kernel-resource-usage", "-o",
                                                os.path.join(tmp, obj), os.path.join(CSRC, src)]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            sys.stderr.write(res.stderr)
            raise RuntimeError("hipcc failed: " + src)
        out = []
        for block in re.split(r"remark: [^\n]*Function Name: ", res.stderr)[1:]:
            def get(key):
                m = re.search(key + r": (\d+)", block)
                return int(m.group(1)) if m else -1
            out.append((block.split()[0], get("VGPRs"), get("AGPRs"), get(r"ScratchSize \[bytes/lane\]"),
                        get(r"Occupancy \[waves/SIMD\]"), get(r"LDS Size \[bytes/block\]")))
        return out

    units = [u for u in UNITS if u[0].endswith(".hip")]
    with tempfile.TemporaryDirectory(prefix="kvarn_ru_") as tmp:
        workers = max(1, min(len(units), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
        with ThreadPoolExecutor(max_workers=workers) as ex:
            results = list(ex.map(lambda u: one(u, tmp), units))
    seen = {}
    for rows in results:
        for r in rows:
            seen[_short_name(r[0])] = r  # a kernel compiled in several units appears once
    lines = ["| kernel | VGPRs | AGPRs | scratch B/lane | waves/SIMD | LDS B |", "|---|---:|---:|---:|---:|---:|"]
    for nm in sorted(seen):
        r = seen[nm]
        lines.append(f"| `{nm}` | {r[1]} | {r[2]} | {r[3]} | {r[4]} | {r[5]} |")
    spill = sum(1 for r in seen.values() if r[3] > 0)
    lines.append("")
    lines.append(f"{len(seen)} kernels, {spill} with scratch.")
    return "\n".join(lines)


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
    if "--resource-usage" in sys.argv:
        print(resource_usage(verbose="-v" in sys.argv))
        sys.exit(0)
    build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv)
    if "--probes" in sys.argv:
        build_probes(verbose="-v" in sys.argv)
