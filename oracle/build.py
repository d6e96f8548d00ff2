"""Builds the oracle's shared library, oracle/liboracle.so, with gcc.

Test infrastructure: the checker, not the product.  Strict IEEE binary32:
no fast-math and no implicit FMA contraction (-ffp-contract=off), so the
library computes exactly the operations its source writes.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "mhcb_oracle.c")
LIBRARY = os.path.join(HERE, "liboracle.so")

FLAGS = [
    "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
    "-ffp-contract=off", "-fno-fast-math", "-fexcess-precision=standard",
    "-Wall", "-Wextra", "-Wno-unused-parameter",
]


def build(verbose: bool = False) -> str:
    """Compiles the oracle; returns the library path."""
    tmp = LIBRARY + ".tmp"
    cmd = ["gcc", *FLAGS, SOURCE, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
