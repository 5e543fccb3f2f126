"""GPU: the allocation-free sweep entry point (mxattn_scale_sweep_noalloc)
against mxattn_scale_sweep with a caller workspace.

Both run the same kernels in the same fixed order, so the per-head sums must
be bit-identical.  Two calls in a row, the second on a smaller input (the
static scratch keeps the first call's partial sums, and none of them may leak
into the second); then the first input again; and an oversize problem is
refused before anything is enqueued."""
import numpy as np
import pytest
import torch

import mxfp4_microscaled_bit_amd as mx
import workloads as W
from parity import say, to_device

pytestmark = pytest.mark.gpu

SWEEP = [round(6.0 + 0.05 * i, 2) for i in range(41)]  # 6.00 .. 8.00


def _both(x, qs, axis, rotate):
    ref = mx.scale_sweep(x, qs, axis=axis, rotate=rotate)
    got = mx.scale_sweep_noalloc(x, qs, axis=axis, rotate=rotate)
    torch.cuda.synchronize()
    return ref, got


def test_noalloc_sweep_equals_workspace_sweep_on_consecutive_calls():
    w = W.WORKLOADS[2]
    big = to_device(W.generate(w, "q", heads=[(0, h) for h in range(8)])[None], w.dtype)  # B1 H8 N32760 d128
    small = W.custom(2, 3, 1000, 64, seed=77, scale=3.0)
    small_k = to_device(small["k"], W.BF16)
    say(f"noalloc sweep: first call {tuple(big.shape)} head-dim, rotated")
    ref1, got1 = _both(big, SWEEP, mx.AXIS_HEAD_DIM, True)
    assert torch.equal(got1, ref1)
    say(f"noalloc sweep: second call {tuple(small_k.shape)} along tokens (smaller)")
    ref2, got2 = _both(small_k, SWEEP[::3], mx.AXIS_TOKEN, False)
    assert got2.shape == (6, len(SWEEP[::3]))
    assert torch.equal(got2, ref2)
    say("noalloc sweep: the first input again, head-dim without rotation")
    ref3, got3 = _both(big, SWEEP[:7], mx.AXIS_HEAD_DIM, False)
    assert torch.equal(got3, ref3)
    assert np.isfinite(got1.cpu().numpy()).all() and (got1.cpu().numpy() > 0).all()


def test_noalloc_sweep_refuses_a_problem_beyond_its_scratch():
    """B64 H64 N118800 d128 with 48 boundaries needs 731 MB of partial sums:
    refused with MXATTN_ERR_SCRATCH.  The input views one head's buffer for
    every (b, h) (zero batch and head strides), so no memory of that size
    exists; nothing is launched."""
    head = torch.zeros((118800, 128), dtype=torch.bfloat16, device="cuda")
    x = head.as_strided((64, 64, 118800, 128), (0, 0, 128, 1))
    qs = [6.0 + 0.04 * j for j in range(48)]
    out = torch.empty((64 * 64, 48), dtype=torch.float64, device="cuda")
    assert mx.scale_sweep_workspace_bytes(64, 64, 118800, 128, mx.AXIS_HEAD_DIM, 48) > mx.SWEEP_SCRATCH_BYTES
    with pytest.raises(mx.MXAttnError, match="static scratch"):
        mx.scale_sweep_noalloc(x, qs, axis=mx.AXIS_HEAD_DIM, rotate=True, out=out)
