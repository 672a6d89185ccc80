"""The work-group -> tile map's division by invariant divisors (FastDiv and
TileMap in csrc/common.hpp), checked on the host: tests/fast_div_check.cpp
includes the header, compiled for the host only, and compares every
quotient with exact division and every mapped tile with the same raster
computed with plain divisions."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "dense_fp32_matrix_03_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_fast_division_and_tile_map_match_plain_division(tmp_path):
    exe = tmp_path / "fast_div_check"
    subprocess.run([HIPCC, "-std=c++17", "-O2", "--cuda-host-only", "-x", "hip",
                    "-I", CSRC, os.path.join(HERE, "fast_div_check.cpp"), "-o", str(exe)],
                   check=True, capture_output=True, timeout=300)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "failures 0" in r.stdout
