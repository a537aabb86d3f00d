"""AddressSanitizer + UBSan run of the host code on the CPU.

Builds, with gcc / g++ and -fsanitize=address,undefined (errors fatal):
  - the oracle (oracle/kvc_oracle.c), with the flags of oracle/build.py;
  - the C ABI's host code (fp8_fp4_quantized_amd/csrc/kvc_api.cpp) with the
    stub launchers of launch_stub.cpp (no device code: a call that gets past
    its host-side checks returns KVC_ELAUNCH).
Then copies the Python packages and the tests into a scratch tree with those
two libraries in place of libkvc_oracle.so and libkvc.so, and runs the CPU
test suite there (``-m "not gpu"``) with the sanitizer runtime preloaded.
The exhaustive ue8m0 pin over every positive fp32 (about 2 minutes
unsanitized) is left out; every other CPU test runs.

Usage: python tests/sanitize/run.py [scratch_dir]   (exit status = pytest's)
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
       "-fno-omit-frame-pointer", "-g", "-O1"]
SKIP = "not every_positive_fp32"


def _run(cmd):
    print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build(out_dir: str) -> tuple[str, str]:
    oracle_so = os.path.join(out_dir, "libkvc_oracle.so")
    _run(["gcc", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-Wextra", *SAN, os.path.join(ROOT, "oracle", "kvc_oracle.c"),
          "-o", oracle_so, "-lm"])
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    kvc_so = os.path.join(out_dir, "libkvc.so")
    _run(["g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", f"-I{rocm}/include", "-fPIC", "-shared",
          "-Wall", *SAN, os.path.join(ROOT, "fp8_fp4_quantized_amd", "csrc", "kvc_api.cpp"),
          os.path.join(ROOT, "tests", "sanitize", "launch_stub.cpp"), f"-L{rocm}/lib",
          "-lamdhip64", f"-Wl,-rpath,{rocm}/lib", "-o", kvc_so])
    return oracle_so, kvc_so


def tree(work: str, oracle_so: str, kvc_so: str) -> str:
    """the Python side of the repository with the sanitized libraries"""
    dst = os.path.join(work, "tree")
    ign = shutil.ignore_patterns("*.so", "__pycache__", "_build", "*.o", "sanitize")
    for d in ("oracle", "fp8_fp4_quantized_amd", "workloads", "tests", "include"):
        shutil.copytree(os.path.join(ROOT, d), os.path.join(dst, d), ignore=ign)
    for f in ("bench.py", "__graft_entry__.py"):
        shutil.copy(os.path.join(ROOT, f), dst)
    shutil.copy(oracle_so, os.path.join(dst, "oracle", "libkvc_oracle.so"))
    shutil.copy(kvc_so, os.path.join(dst, "fp8_fp4_quantized_amd", "libkvc.so"))
    # the ceiling library carries device code only; the ABI test loads it
    shutil.copy(os.path.join(ROOT, "fp8_fp4_quantized_amd", "libkvc_ceiling.so"),
                os.path.join(dst, "fp8_fp4_quantized_amd", "libkvc_ceiling.so"))
    return dst


CANARY = r"""
#include <stdlib.h>
int kvc_canary_heap(const int* i) {
  int* a = (int*)malloc(4 * sizeof(int));
  for (int k = 0; k < 4; ++k) a[k] = k;
  const int* p = a;
  int v = p[*i];
  free(a);
  return v;
}
int kvc_canary_index(const int* i) { int a[4] = {1, 2, 3, 4}; return a[*i]; }
"""


def sanitizer_env(dst: str) -> dict:
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True, check=True).stdout.strip()
    ubsan = subprocess.run(["gcc", "-print-file-name=libubsan.so"], capture_output=True,
                           text=True, check=True).stdout.strip()
    return dict(os.environ, LD_PRELOAD=f"{asan}:{ubsan}", PYTHONPATH=dst,
                ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:verify_asan_link_order=0",
                UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="4")


def canary_is_caught(work: str, env: dict) -> bool:
    """the harness itself: a read one past a malloc'd block (AddressSanitizer)
    and an index one past an array's bound (UBSan), built with the same flags
    and loaded the same way, must each stop the process with its report"""
    src = os.path.join(work, "canary.c")
    with open(src, "w") as fh:
        fh.write(CANARY)
    ok = True
    # each canary built with its own sanitizer alone, so that the other one
    # cannot report it first
    for fn, flag, report in (("kvc_canary_heap", "address", "heap-buffer-overflow"),
                             ("kvc_canary_index", "undefined", "out of bounds")):
        so = os.path.join(work, f"lib{fn}.so")
        _run(["gcc", "-std=c11", "-fPIC", "-shared", f"-fsanitize={flag}",
              "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g", "-O1", src,
              "-o", so])
        code = ("import ctypes; L = ctypes.CDLL(%r); i = ctypes.c_int(4); "
                "print(L.%s(ctypes.byref(i)))" % (so, fn))
        r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True)
        ok &= r.returncode != 0 and report in r.stderr
    return ok


def main(argv) -> int:
    work = argv[1] if len(argv) > 1 else tempfile.mkdtemp(prefix="kvc_san_")
    os.makedirs(work, exist_ok=True)
    oracle_so, kvc_so = build(work)
    dst = tree(work, oracle_so, kvc_so)
    env = sanitizer_env(dst)
    if not canary_is_caught(work, env):
        print("sanitizer harness did not catch the planted out-of-bounds reads", flush=True)
        return 3
    print("sanitizer harness catches the planted out-of-bounds reads", flush=True)
    cmd = [sys.executable, "-m", "pytest", os.path.join(dst, "tests"), "-m", "not gpu", "-k", SKIP,
           "-q", "-p", "no:cacheprovider", "--ignore", os.path.join(dst, "tests", "test_sanitize.py")]
    print(" ".join(cmd), flush=True)
    return subprocess.run(cmd, cwd=dst, env=env).returncode


if __name__ == "__main__":
    sys.exit(main(sys.argv))
