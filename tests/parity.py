"""Helpers for the GPU parity tests: upload seeded inputs, run the HIP path
through the C ABI, and compare with the CPU oracle on the same inputs.

Comparison rules:
  * codes and E8M0 scales of the quantizers: bit-exact;
  * attention output: max |o - o_ref| <= ABS_TOL + allowance per element, and
    sum |o - o_ref| / sum |o_ref| <= REL_TOL over the compared elements whose
    result is unique (decision allowance <= ABS_TOL); elements of rows where a
    near-threshold decision can move the output by more than ABS_TOL have two
    correct results and are held to the per-element bound only.
    ABS_TOL = 1e-2 and REL_TOL = 1e-3 are the acceptance bounds of the target.
    The allowance covers two ways the binary32 GPU path may legitimately
    differ from the binary64 oracle:
      - decision allowance: P~ quantization decisions that lie within a
        relative margin DELTA of a rounding midpoint or a scale boundary may
        go the other way (the oracle reports a first-order bound on the
        resulting change of O_i, field ``amb``);
      - accumulation allowance: the binary32 sum over T key tiles of
        beta-weighted P^ V^ terms, bounded by (T + 4) u * absmass with
        u = 2^-24 and absmass = sum beta P^ |v^| / l (field ``absmass``).
DELTA: the GPU evaluates y = exp2(fma(s, c, -(m c + e))) in binary32 from
binary32 scores.  Its relative error against the binary64 oracle is
ln2 * |error of the exponent argument| plus the exp2 error; with scores
|s| <= 2^10, c <= 0.19 and a few ulps of accumulation error in s and m this
stays below 2^-14.  DELTA = 2^-13 leaves a factor of two.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import mxfp4_microscaled_bit_amd as mx
import oracle
import workloads as W

ABS_TOL = 1e-2
REL_TOL = 1e-3
DELTA = 2.0 ** -13
U32 = 2.0 ** -24


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_device(bits: np.ndarray, dtype: int) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    t = t.view(torch.bfloat16 if dtype == W.BF16 else torch.float16)
    return t.cuda()


def compare_headdim(x_bits, dtype, B, H, N, d, rotate, rule, rows=None, dev=None, strides=None):
    """Bit-exact comparison of the head-dim quantizer with the oracle on `rows`
    (global row indices (b*H+h)*N+n; None = all)."""
    if dev is None:
        dev = to_device(x_bits, dtype)
    mxt = mx.rotate_quantize(dev, mx.AXIS_HEAD_DIM, rotate=rotate, rule=rule)
    torch.cuda.synchronize()
    codes, scales, pad_c, pad_s = mx.unpack_headdim(mxt)
    assert (pad_c == 0).all() and (pad_s == 127).all(), "padding rows must be zeros with scale 127"
    oc, os_ = oracle.quantize_rows(x_bits if strides is None else x_bits, dtype, B, H, N, d, rotate=rotate,
                                   rule=rule, rows=rows, strides=strides)
    gc = codes.reshape(-1, d)
    gs = scales.reshape(-1, d // 32)
    if rows is not None:
        gc, gs = gc[rows], gs[rows]
    bad_c = int((gc != oc).sum())
    bad_s = int((gs != os_).sum())
    return bad_c, bad_s, gc.size


def compare_tokens(x_bits, dtype, B, H, N, d, rule, blocks=None, dev=None):
    if dev is None:
        dev = to_device(x_bits, dtype)
    mxt = mx.rotate_quantize(dev, mx.AXIS_TOKEN, rotate=False, rule=rule)
    torch.cuda.synchronize()
    codes, scales = mx.unpack_tokens(mxt)
    NB = (N + 31) // 32
    assert (codes[:, :, NB:] == 0).all() and (scales[:, :, NB:] == 127).all()
    oc, os_ = oracle.quantize_token_blocks(x_bits, dtype, B, H, N, d, rule=rule, blocks=blocks)
    gc = codes[:, :, :NB].reshape(-1, d, 32)
    gs = scales[:, :, :NB].reshape(-1, d)
    if blocks is not None:
        gc, gs = gc[blocks], gs[blocks]
    return int((gc != oc).sum()), int((gs != os_).sum()), gc.size


def run_forward(dq, dk, dv, causal, rotate=True, with_stats=True):
    qm = mx.rotate_quantize(dq, mx.AXIS_HEAD_DIM, rotate=rotate)
    km = mx.rotate_quantize(dk, mx.AXIS_HEAD_DIM, rotate=rotate)
    vm = mx.rotate_quantize(dv, mx.AXIS_TOKEN, rotate=False)
    B, H, N, d = dq.shape
    stats = torch.empty((B, H, N, 2), dtype=torch.float32, device=dq.device) if with_stats else None
    out = mx.forward(qm, km, vm, causal=causal, row_stats=stats)
    torch.cuda.synchronize()
    return out, stats


def check_output(gpu, ref, label, n_tiles):
    """gpu: float array; ref: oracle dict sliced to the same elements."""
    o_ref = ref["out"]
    diff = np.abs(gpu.astype(np.float64) - o_ref)
    allowance = ref["amb"] + (n_tiles + 4) * U32 * ref["absmass"] * 4.0
    excess = diff - (ABS_TOL + allowance)
    # mean-relative error over the elements whose result is unique: rows where a
    # near-threshold decision could move the output by more than ABS_TOL have
    # two correct results, and are held to the allowance bound only
    unique = ref["amb"] <= ABS_TOL
    rel = float(diff[unique].sum() / max(np.abs(o_ref[unique]).sum(), 1e-300))
    rel_all = float(diff.sum() / max(np.abs(o_ref).sum(), 1e-300))
    raw_max = float(diff.max())
    n_need = int((diff > ABS_TOL).sum())
    say(f"[{label}] max|diff|={raw_max:.3e} mean-rel={rel:.3e} (all elements {rel_all:.3e}) "
        f"elements>1e-2={n_need} ambiguous={int((~unique).sum())}/{diff.size} "
        f"within allowance={bool((excess <= 0).all())} max amb={float(ref['amb'].max()):.3e}")
    assert np.isfinite(gpu).all(), f"{label}: non-finite GPU output"
    assert (excess <= 0).all(), f"{label}: max excess {float(excess.max()):.3e}"
    assert rel <= REL_TOL, f"{label}: mean-relative error {rel:.3e}"
    return raw_max, rel
