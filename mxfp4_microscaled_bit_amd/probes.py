"""In-run throughput probes (libmxprobe.so): the matrix-core FP4 rate, the
fused forward's per-pair vector mix and HBM read+write bandwidth, measured on
the GPU the benchmark runs on.  Each probe runs one untimed launch and then
times `launches` launches with HIP events on the current stream; the best is
reported (the probes have no data-dependent work)."""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmxprobe.so")
_lib = None

FLOPS_PER_FP4_PRODUCT = 2 * 32 * 32 * 64  # one 32x32x64 matrix product
PAIRS_PER_MIX_ROUND = 32                    # per lane: 16 chains x 2 pairs


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with mxfp4_microscaled_bit_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        i32, vp = ctypes.c_int, ctypes.c_void_p
        L.mxprobe_mfma_fp4.restype = i32
        L.mxprobe_mfma_fp4.argtypes = [i32, i32, vp, vp]
        L.mxprobe_pair_mix.restype = i32
        L.mxprobe_pair_mix.argtypes = [i32, i32, vp, vp]
        L.mxprobe_stream.restype = i32
        L.mxprobe_stream.argtypes = [vp, vp, ctypes.c_int64, vp]
        L.mxprobe_read.restype = i32
        L.mxprobe_read.argtypes = [vp, vp, ctypes.c_int64, vp]
        _lib = L
    return _lib


def _best_ms(launch, launches: int) -> float:
    launch()
    torch.cuda.synchronize()
    best = float("inf")
    for _ in range(launches):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        launch()
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1))
    return best


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def mfma_fp4_tflops(groups: int = 512, iters: int = 4000, launches: int = 3) -> float:
    """Dense scaled-FP4 32x32x64 products, four independent accumulators per
    wave, `groups` workgroups of four waves."""
    out = torch.empty(groups * 256, dtype=torch.float32, device="cuda")

    def launch():
        st = lib().mxprobe_mfma_fp4(groups, iters, ctypes.c_void_p(out.data_ptr()), _stream())
        if st != 0:
            raise RuntimeError(f"mxprobe_mfma_fp4 failed ({st})")

    ms = _best_ms(launch, launches)
    return groups * 4 * iters * 4 * FLOPS_PER_FP4_PRODUCT / (ms * 1e-3) / 1e12


def pair_mix_gpairs(groups: int = 512, iters: int = 2000, launches: int = 3) -> float:
    """The forward's vector work per (query, key) pair -- one FMA, one
    exponential, half an FP4 convert and half a max3 -- in pairs per second
    (1e9), at two waves per SIMD when groups = 2 x the number of CUs."""
    out = torch.empty(groups * 256, dtype=torch.float32, device="cuda")

    def launch():
        st = lib().mxprobe_pair_mix(groups, iters, ctypes.c_void_p(out.data_ptr()), _stream())
        if st != 0:
            raise RuntimeError(f"mxprobe_pair_mix failed ({st})")

    ms = _best_ms(launch, launches)
    return groups * 256 * iters * PAIRS_PER_MIX_ROUND / (ms * 1e-3) / 1e9


def stream_gbs(nbytes: int = 1 << 30, launches: int = 3) -> float:
    """Read + write bandwidth of a 16-bytes-per-element copy of nbytes (GB/s)."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    n16 = nbytes // 16

    def launch():
        st = lib().mxprobe_stream(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()), n16, _stream())
        if st != 0:
            raise RuntimeError(f"mxprobe_stream failed ({st})")

    ms = _best_ms(launch, launches)
    return 2.0 * n16 * 16 / (ms * 1e-3) / 1e9


def read_gbs(nbytes: int = 1 << 30, launches: int = 3) -> float:
    """Read bandwidth over nbytes (GB/s; the probe's own small writes not counted)."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    n16 = nbytes // 16
    dst = torch.empty(((n16 + 1023) // 1024) * 256, dtype=torch.int32, device="cuda")

    def launch():
        st = lib().mxprobe_read(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()), n16, _stream())
        if st != 0:
            raise RuntimeError(f"mxprobe_read failed ({st})")

    ms = _best_ms(launch, launches)
    return n16 * 16 / (ms * 1e-3) / 1e9
