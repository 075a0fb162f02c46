"""Host check of the kernels' lane / LDS index maps (no GPU): compiles
tests/layout_check.cpp against csrc/layout.hpp with g++ and runs it."""

import os
import shutil
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_layout_maps():
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "layout_check")
        subprocess.run(["g++", "-std=c++17", "-O1", os.path.join(HERE, "layout_check.cpp"), "-o", exe], check=True)
        res = subprocess.run([exe], capture_output=True, text=True)
        assert res.returncode == 0 and res.stdout.strip() == "ok", res.stdout + res.stderr
