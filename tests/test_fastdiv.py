"""The kernels decode their work items with divisions by launch-fixed divisors done as a
multiply-high, an add and a shift (csrc/fa_internal.h).  This compiles a host program over
that header and checks it against plain integer division (CPU only)."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_fast_division_matches_integer_division(tmp_path):
    exe = tmp_path / "fastdiv_check"
    src = os.path.join(ROOT, "tests", "fastdiv_check.cpp")
    inc = os.path.join(ROOT, "exact_attention_17_amd", "csrc")
    subprocess.run([HIPCC, "-O2", "-std=c++17", "-I", inc, src, "-o", str(exe)], check=True,
                   capture_output=True, timeout=300)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stdout + out.stderr
    assert out.stdout.startswith("ok "), out.stdout
