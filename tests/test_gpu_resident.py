"""The resident-key forward returns the streaming kernel's output bit for bit.

A non-causal forward whose keys fit in LDS (at most 4 key tiles of 128 at
d = 128, 8 at d = 64: cross-attention against a short text sequence, the
MXAttention paper's Sec. 5.1 video models) runs a kernel that loads each
head's K^, V^ once and deals the B H ceil(Nq/128) query tiles out in equal
runs, one run per workgroup slot (two per CU), a run crossing head
boundaries where the count demands it.  Every query tile runs the streaming
kernel's own tile code in the same order, and its epilogue divides through
the row's reciprocal with a correctly rounded result, so the outputs must be
identical.  The streaming kernel is reached through the fused-Q forward,
which equals quantize-then-forward bit for bit where both stream
(test_gpu_fused_q).  Inputs are seeded device normals: this is an equality
test of two GPU paths, not a parity test against the oracle."""
import pytest
import torch

import mxfp4_microscaled_bit_amd as mx
from parity import say

pytestmark = pytest.mark.gpu

# (B, H, Nq, Nk, d)
CASES = [
    (2, 20, 4000, 512, 128),   # 1280 query tiles: runs of 3 crossing heads; four full key tiles
    (2, 20, 4000, 77, 128),    # one masked key tile
    (1, 40, 32760, 500, 128),  # the cross-attention query shape: runs of 20, ragged query and key ends
    (3, 7, 9000, 1024, 64),    # d = 64 at its limit, eight key tiles
    (3, 7, 9000, 1000, 64),
    (2, 5, 1000, 129, 128),    # fewer tiles than slots: one tile per workgroup
    (1, 1, 1, 1, 128),         # one query, one key
    (2, 20, 4000, 640, 128),   # past the d = 128 limit: both sides stream
]


def _inputs(B, H, Nq, Nk, d, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    q = (torch.randn(B, H, Nq, d, generator=g, device="cuda") * 1.5).to(torch.bfloat16)
    k = (torch.randn(B, H, Nk, d, generator=g, device="cuda") * 1.5).to(torch.bfloat16)
    v = torch.randn(B, H, Nk, d, generator=g, device="cuda").to(torch.bfloat16)
    return q, k, v


@pytest.mark.parametrize("B,H,Nq,Nk,d", CASES)
def test_resident_keys_equal_streaming(B, H, Nq, Nk, d):
    say(f"resident vs streaming: B={B} H={H} Nq={Nq} Nk={Nk} d={d}")
    q, k, v = _inputs(B, H, Nq, Nk, d, seed=Nq + 7 * Nk + d)
    qm = mx.rotate_quantize(q, mx.AXIS_HEAD_DIM, rotate=True)
    km = mx.rotate_quantize(k, mx.AXIS_HEAD_DIM, rotate=True)
    vm = mx.rotate_quantize(v, mx.AXIS_TOKEN, rotate=False)
    sa = torch.empty((B, H, Nq, 2), dtype=torch.float32, device="cuda")
    sb = torch.empty_like(sa)
    a = mx.forward(qm, km, vm, causal=False, row_stats=sa)
    b = mx.forward_fused_q(q, km, vm, causal=False, row_stats=sb)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32)), f"max |diff| {float((a - b).abs().max()):.3e}"
    assert torch.equal(sa.view(torch.int32), sb.view(torch.int32))
    assert bool(torch.isfinite(a).all())


def test_resident_keys_repeat_and_sparse_values():
    """Two calls in a row give the same bits (the kernel keeps no state), and
    a V^ with many exact zeros -- rows whose O~ holds zeros take the
    reciprocal route, tiny nonzero ones the element-by-element division --
    still matches the streaming kernel."""
    B, H, Nq, Nk, d = 2, 20, 4000, 300, 128
    q, k, v = _inputs(B, H, Nq, Nk, d, seed=11)
    v = torch.where(torch.rand(v.shape, device="cuda") < 0.7, torch.zeros_like(v), v)
    v[..., 0:4] = 0        # whole channels of zeros: O~ holds exact zeros in every row
    v[0, 0, :, 5] = 1e-33  # one channel of head (0, 0) below 2^-100 of its rows' sums
    qm = mx.rotate_quantize(q, mx.AXIS_HEAD_DIM, rotate=True)
    km = mx.rotate_quantize(k, mx.AXIS_HEAD_DIM, rotate=True)
    vm = mx.rotate_quantize(v, mx.AXIS_TOKEN, rotate=False)
    a1 = mx.forward(qm, km, vm, causal=False)
    a2 = mx.forward(qm, km, vm, causal=False)
    b = mx.forward_fused_q(q, km, vm, causal=False)
    torch.cuda.synchronize()
    assert torch.equal(a1.view(torch.int32), a2.view(torch.int32))
    assert torch.equal(a1.view(torch.int32), b.view(torch.int32))
    assert int((a1 == 0).sum()) > 0
