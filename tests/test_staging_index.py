"""Host check of the staged kernels' copy addressing (no GPU).

Builds tests/staging_index_check.cpp against the kernels' own index header
(gated_delta_rule_03_amd/csrc/tile_index.hpp) and runs it on the CPU: every
global offset an LDS staging copy reads must stay inside its chunk's rows and
columns, and the LDS tiles and output pieces must be covered exactly once.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gated_delta_rule_03_amd", "csrc")


def test_staging_copies_stay_in_bounds(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = tmp_path / "staging_index_check"
    src = os.path.join(ROOT, "tests", "staging_index_check.cpp")
    subprocess.run([hipcc, "-x", "hip", "--offload-arch=gfx950", "-std=c++17", "-O1", "-I", CSRC,
                    src, "-o", str(exe)], check=True, capture_output=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 0 and out.stdout.strip().endswith("OK"), out.stdout
