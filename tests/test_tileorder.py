"""The packed GEMM's work order (csrc/kq_tileorder.hpp) on the CPU: a host-only
build of the header with a checker (tests/native/tileorder_check.cpp) that every
order covers each tile once (whole or as two halves), that the staggered order
finishes no later than the plain one in a model of the dispatcher, and that it
starts each XCD with both halves and whole tiles."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not found")
def test_tile_order_cover_and_makespan(tmp_path):
    exe = str(tmp_path / "tileorder_check")
    p = subprocess.run(["g++", "-std=c++17", "-O2", "-Wall", "-Werror", "-I",
                        os.path.join(ROOT, "mxfp4_activation_quantizer_amd", "csrc"),
                        os.path.join(ROOT, "tests", "native", "tileorder_check.cpp"), "-o", exe],
                       capture_output=True, text=True)
    assert p.returncode == 0, p.stderr
    p = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert p.returncode == 0, p.stdout + p.stderr
    assert p.stdout.startswith("ok")
