"""The host code -- the CPU oracle and the C ABI's argument checks and reuse
head (kvc_api.cpp, with stub launchers: no device code) -- built with
AddressSanitizer and UBSan, and the CPU test suite run against those builds
(tests/sanitize/run.py).  CPU only: nothing here touches a GPU."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None,
                    reason="needs gcc and g++")
def test_cpu_suite_under_asan_and_ubsan(tmp_path):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "sanitize", "run.py"),
                        str(tmp_path)], capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-3000:]
    assert "catches the planted out-of-bounds reads" in r.stdout, tail
    assert r.returncode == 0, tail
    assert " passed" in r.stdout and " failed" not in r.stdout, tail
