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


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
@pytest.mark.parametrize("src", ["fwd.hip", "bwd.hip"])
def test_m0_only_written_by_lds_load_asm(tmp_path, src):
    """The direct-to-LDS loads set M0 in inline assembly; that is only sound while
    no compiler-generated instruction of the kernels reads or writes M0."""
    csrc = os.path.join(ROOT, "variable_length_flash_jfa_amd", "csrc")
    out = tmp_path / (src + ".s")
    cmd = [HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O3", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-I", csrc, "-S", "--cuda-device-only",
           os.path.join(csrc, src), "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    code = [ln.strip() for ln in out.read_text().splitlines()
            if ln.strip() and not ln.strip().startswith((";", "."))]
    uses = [i for i, ln in enumerate(code) if "m0" in ln.replace(",", " ").split()]
    assert uses, "expected the LDS-load assembly to set M0"
    for i in uses:
        # the only M0 writer is the inline pair "s_mov_b32 m0, <sgpr>" followed at
        # once by the LDS-direct buffer load that consumes it
        assert code[i].startswith("s_mov_b32 m0, "), f"unexpected M0 use: {code[i]}"
        assert i + 1 < len(code) and code[i + 1].startswith("buffer_load_dword") \
            and code[i + 1].endswith(" lds"), f"M0 write not followed by an LDS load: {code[i:i + 2]}"
