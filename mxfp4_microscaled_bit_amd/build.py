"""Build libmxattn.so in-tree with hipcc for gfx950.

Every HIP source is compiled with packed-FP32 instructions disabled (the
compiler otherwise forms v_pk_* FP32 ops on its own) and linked into one
shared library next to this file.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmxattn.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = {
    # the quantizers are bit-exact: no contraction of separate multiplies/adds
    "quantize.hip": ["-ffp-contract=off"],
    "attention.hip": [],
    "api.cpp": [],
}
# in-run throughput probes of the benchmark: a library of their own
PROBE_SOURCES = {"probes.hip": []}
PROBE_LIB = os.path.join(HERE, "libmxprobe.so")

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-function",
]


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD, src + ".o")
    cmd = [HIPCC] + COMMON + list(extra) + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(ln for ln in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msgs}")
    if msgs.strip():
        sys.stderr.write(msgs + "\n")
    return obj


def _link(objs, lib: str, verbose: bool):
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, lib)
    if verbose:
        print("built", lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = list(SOURCES.items()) + list(PROBE_SOURCES.items())
    with ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        objs = dict(zip([k for k, _ in jobs], ex.map(lambda kv: _compile(*kv), jobs)))
    _link([objs[k] for k in SOURCES], LIB, verbose)
    _link([objs[k] for k in PROBE_SOURCES], PROBE_LIB, verbose)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
