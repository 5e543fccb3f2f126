"""Helpers for the GPU parity tests: upload seeded inputs, run the HIP path
through the C ABI, and compare with the CPU oracle on the same inputs.

Comparison rules:
  * codes and E8M0 scales of the quantizers: bit-exact;
  * attention output, over every compared element:
      max |o - o_ref| <= ABS_TOL (+ the accumulation allowance below), and
      sum |o - o_ref| / sum |o_ref| <= REL_TOL.
    ABS_TOL = 1e-2 and REL_TOL = 1e-3 are the acceptance bounds of the target.
    Elements may exceed ABS_TOL only where a quantization decision of P~ (or
    P) lies within the relative margin DELTA of its threshold, so that the
    binary32 GPU path and the binary64 oracle may legitimately take it
    differently: such an element must stay within ABS_TOL + amb, where amb is
    the oracle's bound on the output change when every such decision flips,
    and such elements may sit in at most MAX_AMBIGUOUS_ROW_FRACTION of the
    compared rows (never more than a couple of rows on small cases: one flipped
    scale decision moves all d channels of its row).  The counts are printed.
    The accumulation allowance covers the binary32 sum over T key tiles of
    beta-weighted P^ V^ terms: (T + 4) u * absmass with u = 2^-24 and
    absmass = sum beta P^ |v^| / l (field ``absmass``); it is ~1e-7 here.
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
MAX_AMBIGUOUS_ROW_FRACTION = 0.005  # rows that may hold elements beyond ABS_TOL (within their allowance)
MIN_AMBIGUOUS_ROW_CAP = 2           # ... a couple of rows on small cases


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
    acc = (n_tiles + 4) * U32 * ref["absmass"] * 4.0
    beyond = diff > ABS_TOL + acc            # beyond the plain bar
    excess = diff - (ABS_TOL + acc + ref["amb"])
    n_beyond = int(beyond.sum())
    rows_beyond = int(beyond.any(axis=-1).sum())
    n_rows = int(np.prod(diff.shape[:-1]))
    cap = max(MIN_AMBIGUOUS_ROW_CAP, int(MAX_AMBIGUOUS_ROW_FRACTION * n_rows))
    rel = float(diff.sum() / max(np.abs(o_ref).sum(), 1e-300))
    n_flagged = int((ref["amb"] > ABS_TOL).sum())
    say(f"[{label}] max|diff|={float(diff.max()):.3e} mean-rel={rel:.3e} over {diff.size} elements; "
        f"beyond 1e-2: {n_beyond} elements in {rows_beyond} of {n_rows} rows (cap {cap} rows); "
        f"elements with a close decision worth >1e-2: {n_flagged}; "
        f"max amb={float(ref['amb'].max()):.3e}")
    assert np.isfinite(gpu).all(), f"{label}: non-finite GPU output"
    assert (excess <= 0).all(), f"{label}: max excess over the decision allowance {float(excess.max()):.3e}"
    assert rows_beyond <= cap, f"{label}: {n_beyond} elements beyond 1e-2 in {rows_beyond} rows (cap {cap})"
    assert rel <= REL_TOL, f"{label}: mean-relative error {rel:.3e}"
    return float(diff.max()), rel


def check_row_sums(gpu_rs, ref, label, rtol=2e-4, atol=2e-4):
    """Induced row sums of the reference modes against the oracle, on every
    row: each may differ by rtol / atol (binary32 evaluation and sums) plus
    the oracle's amb_rowsum, the exact change of that row sum when the
    quantizer decisions within the margin go the other way (zero on rows
    without such a decision)."""
    gpu_rs = np.asarray(gpu_rs, dtype=np.float64)
    ref_rs, allow = ref["rowsum"], ref["amb_rowsum"]
    diff = np.abs(gpu_rs - ref_rs)
    plain = atol + rtol * np.abs(ref_rs)
    n_allow = int((allow > 0).sum())
    say(f"  [{label}] row sums on all {diff.size} rows: max diff {float(diff.max()):.3e}; "
        f"{n_allow} rows hold a close decision (max allowance {float(allow.max()):.3e}), "
        f"{int((diff > plain).sum())} beyond the plain bar")
    assert np.isfinite(gpu_rs).all(), f"{label}: non-finite row sums"
    assert (diff <= plain + allow).all(), \
        f"{label}: max row-sum excess over the allowance {float((diff - plain - allow).max()):.3e}"
