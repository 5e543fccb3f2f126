"""(CPU) The quantizer kernels' input loads stay inside their tensors.

tests/index_bounds_check.cpp compiles csrc/quant_index.h -- the functions the
kernels call to address every input load -- with g++ on the host and walks
every lane of the launch grids for ragged, strided and full-size shapes,
including 32-token V blocks that lie wholly in the token padding."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mxfp4_microscaled_bit_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="g++ or the ROCm headers not available")
def test_quantizer_loads_stay_inside_the_input(tmp_path):
    exe = str(tmp_path / "index_check")
    cmd = ["g++", "-O2", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include", "-I", CSRC,
           os.path.join(ROOT, "tests", "index_bounds_check.cpp"), "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stderr[-3000:]
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert run.returncode == 0, (run.stdout + run.stderr)[-3000:]
    assert "all quantizer loads inside their tensors" in run.stdout
