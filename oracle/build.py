"""Compile the fp64 oracle (oracle.c) into oracle/liboracle.so with gcc.

Test infrastructure: building the checker is not using it.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False, src: str = SRC, out: str = LIB) -> str:
    """Compile ``src`` (default oracle.c) into the shared library ``out``."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-fPIC", "-shared",
           "-pthread", "-fno-fast-math", "-ffp-contract=off", src, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
