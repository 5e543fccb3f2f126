"""(CPU) Host code under the sanitizers.  The oracle: oracle/sanitize_check.c drives
every oracle entry point on small inputs; built with gcc together with
oracle.c under AddressSanitizer + UndefinedBehaviorSanitizer, and under
ThreadSanitizer (the oracle splits rows and heads over a pthread pool), it
must run clean."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE = os.path.join(ROOT, "oracle")

SANITIZERS = {
    "address_undefined": ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"],
    "thread": ["-fsanitize=thread"],
}


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
@pytest.mark.parametrize("name", sorted(SANITIZERS))
def test_oracle_runs_clean_under_sanitizers(name, tmp_path):
    exe = str(tmp_path / f"oracle_{name}")
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-fno-omit-frame-pointer", "-ffp-contract=off", *SANITIZERS[name],
           "-I", ORACLE, os.path.join(ORACLE, "oracle.c"), os.path.join(ORACLE, "sanitize_check.c"), "-o", exe,
           "-lm", "-pthread"]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stderr[-3000:]
    # verify_asan_link_order=0: the sanitizer runtime need not come first when
    # the environment preloads a library of its own
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0", TSAN_OPTIONS="halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert run.returncode == 0 and "oracle sanitizer run: ok" in run.stdout, (run.stdout + run.stderr)[-3000:]
    assert "runtime error" not in run.stderr and "Sanitizer" not in run.stderr, run.stderr[-3000:]


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="g++ or the ROCm headers not available")
def test_abi_validation_runs_clean_under_sanitizers(tmp_path):
    """(CPU) The C-ABI layer's validation under AddressSanitizer +
    UndefinedBehaviorSanitizer: tests/abi_sanitize_check.cpp links api.cpp
    against launchers that abort if reached and feeds every entry point
    arguments it must reject, and the size helpers extreme shapes."""
    csrc = os.path.join(ROOT, "mxfp4_microscaled_bit_amd", "csrc")
    exe = str(tmp_path / "abi_check")
    cmd = ["g++", "-O1", "-g", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-fno-omit-frame-pointer",
           *SANITIZERS["address_undefined"], "-I", "/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
           "-I", csrc, os.path.join(csrc, "api.cpp"), os.path.join(ROOT, "tests", "abi_sanitize_check.cpp"), "-o",
           exe]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert run.returncode == 0 and "ABI sanitizer run: ok" in run.stdout, (run.stdout + run.stderr)[-3000:]
    assert "runtime error" not in run.stderr, run.stderr[-3000:]
