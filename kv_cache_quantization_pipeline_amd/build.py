"""Compile the HIP sources of libkvarn for gfx950 into an in-tree shared library.

hipcc, -O3, packed fp32 instructions disabled for device code.  The library is
written next to this file as libkvarn.so and loaded by the binding.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkvarn.so")
SOURCES = ["libkvarn.hip", "quantize.hip", "decode.hip"]
ARCH = "gfx950"


def build(verbose: bool = False, extra=()) -> str:
    cmd = ["hipcc", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"),
           "-o", LIB + ".tmp"] + list(extra) + [os.path.join(CSRC, s) for s in SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libkvarn")
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
