"""Build ``libkvc.so`` (the HIP library behind include/kvc.h) and
``libkvc_ceiling.so`` (the benchmark's streaming yardstick,
include/kvc_ceiling.h) for gfx950.

Every HIP source is compiled with hipcc for ``--offload-arch=gfx950`` and
linked into shared libraries next to this file.  Packed fp32 VALU forms are
switched off (``-packed-fp32-ops``): the kernels' float arithmetic stays on
the scalar-per-lane instructions.
"""
from __future__ import annotations

import os
import subprocess
import sys
import concurrent.futures as cf

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkvc.so")
SOURCES = ["kvc_api.cpp", "store_gather.hip", "compress.hip"]
CEILING_LIB = os.path.join(HERE, "libkvc_ceiling.so")
CEILING_SOURCES = ["ceiling.hip"]
ARCH = "gfx950"

FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function"]


def _compile(src: str, obj: str, verbose: bool) -> None:
    cmd = ["hipcc", *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)


def _link(objs, lib: str, verbose: bool) -> None:
    tmp = lib + ".tmp"
    cmd = ["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    every = SOURCES + CEILING_SOURCES
    objs = {s: os.path.join(objdir, s.rsplit(".", 1)[0] + ".o") for s in every}
    with cf.ThreadPoolExecutor(max_workers=len(every)) as ex:
        list(ex.map(lambda s: _compile(s, objs[s], verbose), every))
    _link([objs[s] for s in SOURCES], LIB, verbose)
    _link([objs[s] for s in CEILING_SOURCES], CEILING_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
