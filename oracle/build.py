"""Compile the CPU oracle (test infrastructure) into oracle/liboracle.so.

Plain g++, -O2, no fast-math and no intrinsics, so the oracle's arithmetic is
IEEE fp64 in program order.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kvarn_oracle.cpp")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """Build liboracle.so; with sanitize=True, an AddressSanitizer + UndefinedBehaviorSanitizer copy
    at <repo>/_build/liboracle_san.so (load it with gcc's libasan preloaded)."""
    lib = os.path.join(os.path.dirname(HERE), "_build", "liboracle_san.so") if sanitize else LIB
    cmd = ["g++", "-std=c++17", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared", "-pthread"]
    if sanitize:
        os.makedirs(os.path.dirname(lib), exist_ok=True)
        cmd += ["-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=undefined"]
    cmd += [SRC, "-o", lib + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(lib + ".tmp", lib)
    return lib


if __name__ == "__main__":
    build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv)
