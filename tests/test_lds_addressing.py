"""The kernels' fast LDS addressing equals the reference swizzled layout.

Compiles tests/native/lds_addressing_check.cpp (which includes the kernels'
device header) for the host and runs it; no GPU is needed."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_fast_lds_addressing_matches_swizzle(tmp_path):
    exe = tmp_path / "lds_check"
    cmd = [HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O1", "-std=c++17",
           "-I", os.path.join(ROOT, "variable_length_flash_jfa_amd", "csrc"),
           os.path.join(ROOT, "tests", "native", "lds_addressing_check.cpp"), "-o", str(exe)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    run = subprocess.run([str(exe)], capture_output=True, text=True)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "mismatches=0" in run.stdout
