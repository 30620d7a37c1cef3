"""Compile the fp64 CPU oracle (``kda_ref.c``) into ``oracle/libkda_oracle.so``.

Test infrastructure only: the oracle is what the GPU path is checked against,
and nothing in the GPU library depends on it.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "kda_ref.c")
LIBRARY = os.path.join(HERE, "libkda_oracle.so")


def build(verbose: bool = False) -> str:
    """Compile the oracle with gcc (plain C99, -O2, pthreads); return the path."""
    tmp = LIBRARY + f".tmp{os.getpid()}"
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-fPIC", "-shared",
           "-pthread", SOURCE, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
