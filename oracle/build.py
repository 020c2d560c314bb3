"""Compile the C oracle into oracle/libptgq_oracle.so with gcc.

Test infrastructure: the oracle is the slow, plain CPU implementation the GPU
library is checked against.  Flags keep IEEE binary32 semantics: no fast-math,
no floating-point contraction, SSE arithmetic (the x86-64 default).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ptgq_oracle.c")
LIB = os.path.join(HERE, "libptgq_oracle.so")

CFLAGS = ["-std=c11", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared",
          "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    """Compile the oracle unconditionally; return the path of the library."""
    tmp = LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, "-o", tmp, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def ensure_built() -> str:
    """Build only when the library is missing or older than its source."""
    if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        return build()
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
