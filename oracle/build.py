"""Build the CPU oracle library (``oracle/libkvc_oracle.so``) with gcc.

Test infrastructure: the oracle is the checker of the HIP path, never part
of it.  ``-ffp-contract=off`` keeps every fp64/fp32 operation a separately
rounded IEEE operation, as written in the source.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libkvc_oracle.so")


def build(verbose: bool = False) -> str:
    src = os.path.join(HERE, "kvc_oracle.c")
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared",
           "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
           src, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
