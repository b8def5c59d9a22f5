"""The workgroup decomposition divides by launch-time sizes with the
Granlund-Montgomery multiply-high method (csrc/fastdiv.h); this compiles a
host checker against that header and compares it with ordinary division."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "exact_attention_forward_attn_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs a host C++ compiler")
def test_fastdiv_matches_division(tmp_path):
    exe = tmp_path / "fastdiv_check"
    subprocess.run(["g++", "-O2", "-std=c++17", f"-I{CSRC}", os.path.join(HERE, "fastdiv_check.cpp"), "-o", str(exe)],
                   check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stdout
    assert out.stdout.startswith("OK"), out.stdout
