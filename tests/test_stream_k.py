"""Host check of the skinny kernel's unit split (range_begin / range_of in stream_k.h).

The kernel computes its Stream-K range bounds (spark-kernels post, "stream-k proper": balanced,
contiguous ranges of a flat unit list) with 32-bit and float arithmetic instead of a 64-bit
division; `stream_k_check.cpp` compiles the same header with the host compiler and compares it
with the exact 64-bit definitions, exhaustively on small sizes and on every range boundary up to
U = 2^31 - 1 units and 2^15 ranges."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "gemv_layers_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="no host C++ compiler")
def test_unit_split_matches_exact_division(tmp_path):
    exe = tmp_path / "stream_k_check"
    subprocess.run(["g++", "-O2", "-std=c++17", "-Wall", "-Werror", f"-I{CSRC}",
                    os.path.join(HERE, "stream_k_check.cpp"), "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok")
