"""GPU parity of the scale-rule family (Sec. 2 Eqs. 12-14; Sec. 4.1; App. G)
and of the Q_max sweep (Sec. 5.5.1, Table 4) with the CPU oracle.

  * rotate_quantize_q: codes and E8M0 scales bit-exact for boundaries across
    the allowed range, both block axes, rotation on and off, ragged shapes;
    q = 7.25 reproduces the UOS codes.
  * scale_sweep: per-head sums of squared errors.  The GPU forms every block's
    sum exactly as the oracle does (same per-element rounding, same order
    inside a block) and adds blocks in another fixed order, so the totals
    agree to a relative 1e-12 (binary64 reassociation over at most 2^22
    blocks per head); boundaries whose block decisions coincide give
    bit-identical sums on both sides.
"""
import numpy as np
import pytest
import torch

import mxfp4_microscaled_bit_amd as mx
import oracle
import workloads as W
from parity import say, to_device

pytestmark = pytest.mark.gpu

SWEEP = [round(6.0 + 0.05 * i, 2) for i in range(41)]  # 6.00 .. 8.00, the page's grid
RTOL = 1e-12


def _codes_headdim(dev, q, rotate):
    m = mx.rotate_quantize_q(dev, q, mx.AXIS_HEAD_DIM, rotate=rotate)
    torch.cuda.synchronize()
    codes, scales, pad_c, pad_s = mx.unpack_headdim(m)
    assert (pad_c == 0).all() and (pad_s == 127).all()
    assert m.rule == mx.SCALE_CEIL_Q
    d = dev.shape[-1]
    return codes.reshape(-1, d), scales.reshape(-1, d // 32)


def _codes_tokens(dev, q):
    m = mx.rotate_quantize_q(dev, q, mx.AXIS_TOKEN, rotate=False)
    torch.cuda.synchronize()
    codes, scales = mx.unpack_tokens(m)
    B, H, N, d = dev.shape
    NB = (N + 31) // 32
    return codes[:, :, :NB].reshape(-1, d, 32), scales[:, :, :NB].reshape(-1, d)


@pytest.mark.parametrize("q", [2.0, 3.3, 6.0, 6.05, 7.0, 7.2, 7.25, 7.3, 8.0, 13.7, 64.0])
def test_ceiling_rule_quantizers_bit_exact(q):
    say(f"ceiling rule q={q}")
    for (B, H, N, d, dtype, seed) in ((1, 3, 200, 128, W.BF16, 1), (2, 2, 129, 64, W.FP16, 2)):
        x = W.custom(B, H, N, d, dtype=dtype, seed=seed, scale=3.0)
        for t in ("q", "v"):
            dev = to_device(x[t], dtype)
            if t == "q":
                for rotate in (True, False):
                    gc, gs = _codes_headdim(dev, q, rotate)
                    oc, os_ = oracle.quantize_rows(x[t], dtype, B, H, N, d, rotate=rotate,
                                                   rule=oracle.RULE_CEIL_Q, q=q)
                    assert np.array_equal(gc, oc) and np.array_equal(gs, os_), (q, rotate, d)
            else:
                gc, gs = _codes_tokens(dev, q)
                oc, os_ = oracle.quantize_token_blocks(x[t], dtype, B, H, N, d, rule=oracle.RULE_CEIL_Q, q=q)
                assert np.array_equal(gc, oc) and np.array_equal(gs, os_), (q, d)


def test_boundary_7_25_is_uos_and_boundaries_between_binary32_numbers():
    """q = 7.25 reproduces the UOS quantizer bit for bit.  A boundary that is
    not a binary32 number decides exactly like the binary32 number just below
    it (the decision M <= q 2^e involves a binary32 M)."""
    B, H, N, d = 1, 4, 300, 128
    x = W.custom(B, H, N, d, seed=5, scale=4.0)
    dev = to_device(x["k"], W.BF16)
    u = mx.rotate_quantize(dev, mx.AXIS_HEAD_DIM, rotate=True, rule=mx.SCALE_UOS)
    c = mx.rotate_quantize_q(dev, 7.25, mx.AXIS_HEAD_DIM, rotate=True)
    torch.cuda.synchronize()
    assert torch.equal(u.codes, c.codes) and torch.equal(u.scales, c.scales)
    q = 7.1 + 2 ** -40  # between two binary32 numbers
    f32_below = float(np.nextafter(np.float32(q), np.float32(0)) if float(np.float32(q)) > q else np.float32(q))
    a = mx.rotate_quantize_q(dev, q, mx.AXIS_HEAD_DIM, rotate=True)
    b = mx.rotate_quantize_q(dev, f32_below, mx.AXIS_HEAD_DIM, rotate=True)
    torch.cuda.synchronize()
    assert torch.equal(a.codes, b.codes) and torch.equal(a.scales, b.scales)
    oc, os_ = oracle.quantize_rows(x["k"], W.BF16, B, H, N, d, rotate=True, rule=oracle.RULE_CEIL_Q, q=q)
    gc, gs = _codes_headdim(dev, q, True)
    assert np.array_equal(gc, oc) and np.array_equal(gs, os_)


def _check_sweep(gpu, ref, label):
    rel = np.abs(gpu - ref) / np.maximum(np.abs(ref), 1e-300)
    say(f"  [{label}] max rel diff {rel.max():.2e}")
    assert (rel <= RTOL).all(), label
    # ties: equal oracle sums for two boundaries -> equal GPU sums
    for h in range(ref.shape[0]):
        for j in range(1, ref.shape[1]):
            if ref[h, j] == ref[h, j - 1]:
                assert gpu[h, j] == gpu[h, j - 1], (label, h, j)


@pytest.mark.parametrize("axis,rotate", [(mx.AXIS_HEAD_DIM, True), (mx.AXIS_HEAD_DIM, False), (mx.AXIS_TOKEN, False)])
@pytest.mark.parametrize("shape", [(1, 3, 300, 128), (2, 2, 33, 64), (1, 1, 1, 128), (1, 2, 4100, 128)])
def test_sweep_matches_oracle(axis, rotate, shape):
    B, H, N, d = shape
    say(f"sweep {shape} axis={axis} rotate={rotate}")
    x = W.custom(B, H, N, d, seed=N + d, scale=3.0)["q"]
    dev = to_device(x, W.BF16)
    gpu = mx.scale_sweep(dev, SWEEP, axis=axis, rotate=rotate).cpu().numpy()
    ref = oracle.scale_sweep(x, W.BF16, B, H, N, d, SWEEP, axis=axis, rotate=rotate)
    _check_sweep(gpu, ref, f"{shape} axis={axis} rotate={rotate}")
    again = mx.scale_sweep(dev, SWEEP, axis=axis, rotate=rotate).cpu().numpy()
    assert np.array_equal(gpu, again), "sweep must be deterministic"


def test_sweep_boundary_order_and_count():
    """Any order of the boundaries, 1..48 of them, TFS (6) and the ceiling
    counterpart of OCP (8) included."""
    B, H, N, d = 1, 2, 257, 128
    x = W.custom(B, H, N, d, seed=77, scale=3.0)["k"]
    dev = to_device(x, W.BF16)
    for qs in ([7.25], [8.0, 6.0, 7.0, 7.25], list(np.linspace(5.0, 10.0, 48))):
        gpu = mx.scale_sweep(dev, qs, axis=mx.AXIS_HEAD_DIM, rotate=True).cpu().numpy()
        ref = oracle.scale_sweep(x, W.BF16, B, H, N, d, qs, rotate=True)
        rel = np.abs(gpu - ref) / ref
        assert (rel <= RTOL).all(), qs


@pytest.mark.parametrize("t", ["q", "k", "v"])
def test_sweep_wan_like_sampled_heads(t):
    """Full Wan-like tensor on the GPU (all 40 heads, 41 boundaries); the
    oracle recomputes three heads."""
    w = W.WORKLOADS[2]
    B, H, N, d = w.shape
    bits = W.generate(w, t)
    dev = to_device(bits, w.dtype)
    axis = mx.AXIS_TOKEN if t == "v" else mx.AXIS_HEAD_DIM
    rotate = t != "v"
    say(f"sweep wan-like {t}")
    gpu = mx.scale_sweep(dev, SWEEP, axis=axis, rotate=rotate).cpu().numpy()
    heads = [0, 17, 39]
    ref = oracle.scale_sweep(bits, w.dtype, B, H, N, d, SWEEP, axis=axis, rotate=rotate, heads=heads)
    _check_sweep(gpu[heads], ref, f"wan-like {t}")
    best = [SWEEP[int(np.argmin(r))] for r in gpu]
    say(f"  per-head argmin q: {dict(zip(*np.unique(best, return_counts=True)))}")


@pytest.mark.parametrize("dtype", [W.BF16, W.FP16])
def test_sweep_strided_layout_and_dtype(dtype):
    """A [B, N, H, d] buffer viewed as [B, H, N, d] (no copy), bf16 and fp16:
    the sweep equals the contiguous tensor's bit for bit, and the oracle's
    sums on both axes."""
    B, H, N, d = 2, 3, 150, 64
    x = W.custom(B, N, H, d, dtype=dtype, seed=91, tensors=("k",), scale=3.0)["k"]  # physical [B, N, H, d]
    dev = to_device(x, dtype).permute(0, 2, 1, 3)
    contig = np.ascontiguousarray(x.transpose(0, 2, 1, 3))
    dc = to_device(contig, dtype)
    say(f"sweep strided dtype={dtype}")
    for axis, rotate in ((mx.AXIS_HEAD_DIM, True), (mx.AXIS_TOKEN, False)):
        a = mx.scale_sweep(dev, SWEEP, axis=axis, rotate=rotate).cpu().numpy()
        b = mx.scale_sweep(dc, SWEEP, axis=axis, rotate=rotate).cpu().numpy()
        assert np.array_equal(a, b), (axis, "strided and contiguous sums differ")
        ref = oracle.scale_sweep(contig, dtype, B, H, N, d, SWEEP, axis=axis, rotate=rotate)
        _check_sweep(a, ref, f"strided dtype={dtype} axis={axis}")
