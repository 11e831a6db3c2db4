"""Host check of the bf16 kernels' K/V tile addressing (no GPU).

Compiles tests/tile_addr_check.cpp against the kernels' own addressing header
(exact_blockwise_long_amd/csrc/tile_addr.h) with g++ and runs it: for every
tile shape the kernels launch and ragged key counts over several tiles, every
lane's load either lies inside the key range or has a per-lane offset the
buffer range check rejects (so keys past a range read as zeros and touch no
memory).
"""

from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_blockwise_long_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not installed")
def test_tile_addressing_stays_in_range(tmp_path):
    exe = str(tmp_path / "tile_addr_check")
    src = os.path.join(ROOT, "tests", "tile_addr_check.cpp")
    subprocess.run(["g++", "-std=c++17", "-O2", "-Wall", f"-I{CSRC}", src, "-o", exe], check=True)
    res = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.startswith("ok "), res.stdout
