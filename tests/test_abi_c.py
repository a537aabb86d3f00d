"""The public headers as a C99 program sees them: tests/abi_c/consumer.c is
compiled with gcc -std=c99 -pedantic and every warning an error, linked
against the built libraries and run.  It calls only what answers on the host
(version, layout geometry, argument checks), so it needs no GPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "fp8_fp4_quantized_amd")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_headers_compile_and_link_as_c99(tmp_path):
    for lib in ("libkvc.so", "libkvc_ceiling.so"):
        if not os.path.exists(os.path.join(PKG, lib)):
            pytest.skip(f"{lib} not built")
    exe = str(tmp_path / "consumer")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cmd = ["gcc", "-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror",
           f"-I{os.path.join(ROOT, 'include')}", os.path.join(ROOT, "tests", "abi_c", "consumer.c"),
           f"-L{PKG}", "-lkvc", "-lkvc_ceiling", f"-Wl,-rpath,{PKG}", f"-Wl,-rpath,{rocm}/lib",
           "-Wl,--allow-shlib-undefined",
           "-o", exe]
    subprocess.run(cmd, check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks passed" in r.stdout
