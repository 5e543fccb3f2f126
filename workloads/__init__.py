"""Seeded synthetic inputs for the five attention workloads.

This module only draws random numbers and rounds them to the input dtype; it
holds none of the method's arithmetic.  Both the CPU oracle and the GPU path
consume the same 16-bit patterns it returns.

Recipe (identical for every workload):
  * every (tensor, batch, head) has its own counter-based Philox stream,
    keyed by (seed, stream id, batch, head), so any subset of heads can be
    regenerated on its own and generation runs in parallel;
  * a value is drawn in binary64, multiplied by its channel scale (and outlier
    factor), rounded to binary32 and then to the input dtype with
    round-to-nearest-even;
  * per-channel scales are drawn once per (tensor, head, channel) and shared
    by all tokens and batches.

Shapes follow the pages' workloads: self-attention of video diffusion
transformers (Wan2.2-like and HunyuanVideo-like token counts), a causal
language-model shape, and a small-head stress case.  The pages also mention
Wan2.2's separate text cross-attention without giving its shape; the cross
workload pairs the Wan-like video queries with 512 text keys/values, a
synthetic choice.  None of the pages'
model activations are available, so lognormal channel scales and sparse x15
outlier channels stand in for the activation outliers the pages describe.
"""
from __future__ import annotations

import os
import threading
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

BF16, FP16 = 0, 1  # same numbering as the library's dtype enum


@dataclass(frozen=True)
class Workload:
    cid: int
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: int
    causal: bool
    seed: int
    kind: str
    params: dict = field(default_factory=dict)
    Nk: int = 0  # key/value tokens of cross-attention; 0: self-attention (N)

    @property
    def shape(self):
        return (self.B, self.H, self.N, self.d)

    @property
    def kv_tokens(self) -> int:
        return self.Nk if self.Nk > 0 else self.N

    def tokens(self, tensor: str) -> int:
        return self.N if tensor == "q" else self.kv_tokens

    def flops(self) -> float:
        """4*d flops per visible (query, key) pair: QK^T and PV each take 2*d."""
        pairs = self.N * (self.N + 1) / 2 if self.causal else float(self.N) * self.kv_tokens
        return 4.0 * self.d * self.B * self.H * pairs

    def describe(self) -> str:
        return (f"B{self.B} H{self.H} N{self.N}{f' Nk{self.Nk}' if self.Nk else ''} d{self.d} "
                f"{'fp16' if self.dtype == FP16 else 'bf16'}{' causal' if self.causal else ''}")


WORKLOADS = {
    1: Workload(1, "tiny_outliers", 1, 2, 256, 128, FP16, False, 1, "outlier_channels",
                {"channels": (3, 40, 77, 114), "factor": 20.0}),
    2: Workload(2, "wan_like", 1, 40, 32760, 128, BF16, False, 2, "lognormal",
                {"sigma": 1.0}),
    3: Workload(3, "hunyuan_like", 1, 24, 118800, 128, BF16, False, 3, "lognormal_outliers",
                {"sigma": 1.5, "p_outlier": 0.01, "factor": 15.0}),
    4: Workload(4, "causal_lm", 4, 32, 8192, 128, BF16, True, 4, "lognormal",
                {"sigma": 1.0}),
    5: Workload(5, "sharp_d64", 16, 16, 4096, 64, BF16, False, 5, "sharp",
                {"qk_scale": 4.0, "v_range": 8.0}),
    6: Workload(6, "wan_like_cross", 1, 40, 32760, 128, BF16, False, 6, "lognormal",
                {"sigma": 1.0}, Nk=512),
}

TENSOR_ID = {"q": 0, "k": 1, "v": 2}


def _rng(seed: int, stream: int, b: int, h: int) -> np.random.Generator:
    key = (seed << 64) | (stream << 48) | (b << 24) | h
    return np.random.Generator(np.random.Philox(key=key))


def to_bits(x: np.ndarray, dtype: int, out=None, scratch=None) -> np.ndarray:
    """Round binary64 values to binary32, then to bf16/fp16 (RNE); return the bits.

    ``out`` (uint16) and ``scratch`` (float32, same shape) may be given to reuse memory.
    """
    f = np.empty(x.shape, np.float32) if scratch is None else scratch
    f[...] = x
    if out is None:
        out = np.empty(x.shape, np.uint16)
    if dtype == FP16:
        out[...] = f.astype(np.float16).view(np.uint16)
        return out
    u = f.view(np.uint32)
    u += np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    u >>= np.uint32(16)
    out[...] = u
    return out


def from_bits(bits: np.ndarray, dtype: int) -> np.ndarray:
    """Exact decode of 16-bit patterns to float32 (for reporting and references)."""
    if dtype == FP16:
        return bits.view(np.float16).astype(np.float32)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def channel_scales(w: Workload, tensor: str) -> np.ndarray:
    """[H, d] binary64 factors applied per channel (shared by batches and tokens)."""
    t = TENSOR_ID[tensor]
    s = np.ones((w.H, w.d))
    if w.kind == "outlier_channels":
        if tensor in ("q", "k"):
            s[:, list(w.params["channels"])] = w.params["factor"]
        return s
    if w.kind in ("lognormal", "lognormal_outliers"):
        for h in range(w.H):
            s[h] = _rng(w.seed, 3 + t, 0, h).lognormal(0.0, w.params["sigma"], w.d)
        if w.kind == "lognormal_outliers":
            for h in range(w.H):
                mask = _rng(w.seed, 6 + t, 0, h).random(w.d) < w.params["p_outlier"]
                s[h, mask] *= w.params["factor"]
        return s
    if w.kind == "sharp":
        return s
    raise ValueError(w.kind)


def head_values(w: Workload, tensor: str, b: int, h: int, scales=None, out=None) -> np.ndarray:
    """[N, d] binary64 values of one head before rounding to the input dtype."""
    t = TENSOR_ID[tensor]
    rng = _rng(w.seed, t, b, h)
    if out is None:
        out = np.empty((w.tokens(tensor), w.d))
    if w.kind == "sharp":
        if tensor == "v":
            r = w.params["v_range"]
            rng.random(out=out)
            out *= 2.0 * r
            out -= r
            return out
        rng.standard_normal(out=out)
        out *= w.params["qk_scale"]
        return out
    if scales is None:
        scales = channel_scales(w, tensor)
    rng.standard_normal(out=out)
    out *= scales[h][None, :]
    return out


def _threads() -> int:
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        return min(int(env), 16)
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:  # pragma: no cover
        return 1


_tls = threading.local()


def _scratch(shape):
    """Per-thread reusable buffers: first-touch page faults dominate otherwise."""
    bufs = getattr(_tls, "bufs", None)
    if bufs is None or bufs[0].shape != shape:
        bufs = (np.empty(shape), np.empty(shape, np.float32))
        _tls.bufs = bufs
    return bufs


def generate(w: Workload, tensor: str, heads=None) -> np.ndarray:
    """16-bit patterns of one input tensor.

    heads=None -> array [B, H, n, d]; heads=[(b, h), ...] -> array [len(heads), n, d],
    with n = w.tokens(tensor).
    """
    scales = channel_scales(w, tensor)
    n = w.tokens(tensor)
    sel = [(b, h) for b in range(w.B) for h in range(w.H)] if heads is None else list(heads)
    out = np.empty((len(sel), n, w.d), np.uint16)

    def one(i):
        b, h = sel[i]
        f64, f32 = _scratch((n, w.d))
        head_values(w, tensor, b, h, scales, out=f64)
        to_bits(f64, w.dtype, out=out[i], scratch=f32)

    with ThreadPoolExecutor(max_workers=_threads()) as ex:
        list(ex.map(one, range(len(sel))))
    if heads is None:
        return out.reshape(w.B, w.H, n, w.d)
    return out


def custom(B, H, N, d, dtype=BF16, seed=0, tensors=("q", "k", "v"), scale=1.0):
    """Standard-normal inputs of any shape (edge-case tests); returns a dict of bit arrays."""
    res = {}
    for name in tensors:
        t = TENSOR_ID[name]
        vals = np.empty((B, H, N, d))
        for b in range(B):
            for h in range(H):
                vals[b, h] = scale * _rng(seed, t, b, h).standard_normal((N, d))
        res[name] = to_bits(vals, dtype)
    return res


def device_normal(B, H, N, d, dtype=BF16, seed=0, tensor="q", scale=1.0, device="cuda"):
    """Standard-normal inputs drawn on the device, for shapes too large to draw
    on the host (billions of elements): torch's seeded Philox generator on
    `device`, keyed by (seed, tensor), rounded to the input dtype.  Returns a
    torch tensor [B, H, N, d]; a test hands the oracle the 16-bit patterns of
    the heads it checks, read back from this tensor."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(1_000_003 * int(seed) + 7919 * TENSOR_ID[tensor] + 17)
    tdt = torch.bfloat16 if dtype == BF16 else torch.float16
    out = torch.empty((B, H, N, d), dtype=tdt, device=device)
    step = max(1, (1 << 28) // (N * d))  # heads per draw: at most 2^28 binary32 values at a time
    flat = out.view(B * H, N, d)
    for h0 in range(0, B * H, step):
        h1 = min(B * H, h0 + step)
        x = torch.randn((h1 - h0, N, d), generator=g, device=device, dtype=torch.float32)
        if scale != 1.0:
            x.mul_(scale)
        flat[h0:h1].copy_(x)
    return out
