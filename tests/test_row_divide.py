"""(CPU) The forward's epilogue divides O~ by l through the row's correctly
rounded reciprocal and one fused correction (Markstein's theorem), falling
back to a true division for rows the theorem does not cover.

tests/row_divide_check.cpp compiles csrc/row_divide.h -- the functions the
kernels call -- with g++ on the host and checks, over random and boundary
operands, that every quotient the fast route produces equals the correctly
rounded a / l bit for bit, and that the guard refuses zero, subnormal,
non-finite and out-of-range rows."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mxfp4_microscaled_bit_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="g++ or the ROCm headers not available")
def test_epilogue_division_is_correctly_rounded(tmp_path):
    exe = str(tmp_path / "row_divide_check")
    cmd = ["g++", "-O2", "-std=c++17", "-ffp-contract=off", "-fno-fast-math", "-D__HIP_PLATFORM_AMD__",
           "-I", "/opt/rocm/include", "-I", CSRC, os.path.join(ROOT, "tests", "row_divide_check.cpp"), "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stderr[-3000:]
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert run.returncode == 0, (run.stdout + run.stderr)[-3000:]
    assert "epilogue division correctly rounded" in run.stdout
