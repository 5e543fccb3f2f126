"""GPU checks of the forward with the Q preprocessing fused into its prologue
(MXAttention, Sec. 4.3: the rotation sits in the Q/K preprocessing stage).

mxattn_forward_fused_q rotates and quantizes Q inside the attention kernel
with the same block arithmetic as mxattn_rotate_quantize, so its output and
row statistics must equal those of rotate_quantize + mxattn_forward bit for
bit, for every shape, dtype, stride, rule and masking case; the workloads are
also compared with the CPU oracle to the forward's bar."""
import numpy as np
import pytest
import torch

import mxfp4_microscaled_bit_amd as mx
import workloads as W
from parity import check_output, say, to_device

pytestmark = pytest.mark.gpu

KV_TILE = 128


def _two_call(dq, km, vm, causal, rotate, rule):
    qm = mx.rotate_quantize(dq, mx.AXIS_HEAD_DIM, rotate=rotate, rule=rule)
    B, H, N, d = dq.shape
    stats = torch.empty((B, H, N, 2), dtype=torch.float32, device=dq.device)
    return mx.forward(qm, km, vm, causal=causal, row_stats=stats), stats


def _fused(dq, km, vm, causal):
    B, H, N, d = dq.shape
    stats = torch.empty((B, H, N, 2), dtype=torch.float32, device=dq.device)
    return mx.forward_fused_q(dq, km, vm, causal=causal, row_stats=stats), stats


def _kv(dk, dv, rotate, rule):
    return (mx.rotate_quantize(dk, mx.AXIS_HEAD_DIM, rotate=rotate, rule=rule),
            mx.rotate_quantize(dv, mx.AXIS_TOKEN, rotate=False, rule=rule))


@pytest.mark.parametrize("N", [1, 31, 127, 128, 129, 300])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fused_q_equals_two_calls(N, d, causal):
    B, H = 2, 3
    for dtype, rotate, rule, seed in ((W.BF16, True, mx.SCALE_UOS, 1), (W.FP16, True, mx.SCALE_UOS, 2),
                                      (W.BF16, False, mx.SCALE_UOS, 3), (W.BF16, True, mx.SCALE_OCP, 4)):
        x = W.custom(B, H, N, d, dtype=dtype, seed=N + d + seed, scale=2.5)
        dq, dk, dv = (to_device(x[t], dtype) for t in "qkv")
        km, vm = _kv(dk, dv, rotate, rule)
        a, sa = _two_call(dq, km, vm, causal, rotate, rule)
        b, sb = _fused(dq, km, vm, causal)
        torch.cuda.synchronize()
        say(f"fused Q N={N} d={d} causal={causal} dtype={dtype} rotate={rotate} rule={rule}")
        assert torch.equal(a, b), f"max |diff| {float((a - b).abs().max()):.3e}"
        assert torch.equal(sa, sb)


@pytest.mark.parametrize("Nq,Nk,d", [(300, 77, 128), (129, 1, 64), (5, 700, 128), (1000, 4100, 64)])
def test_fused_q_cross_attention_and_strided_q(Nq, Nk, d):
    """Cross-attention (Nq != Nk) with Q read through non-contiguous strides:
    a [B, N, H, d] buffer viewed as [B, H, N, d]."""
    B, H = 2, 3
    xq = W.custom(B, H, Nq, d, seed=Nq + 3 * d, scale=2.0)
    xkv = W.custom(B, H, Nk, d, seed=Nk + 5 * d, scale=2.0)
    dq = to_device(xq["q"], W.BF16)
    dq_t = dq.transpose(1, 2).contiguous().transpose(1, 2)  # strides (N H d, d, H d, 1)
    assert not dq_t.is_contiguous() and torch.equal(dq_t, dq)
    km, vm = _kv(to_device(xkv["k"], W.BF16), to_device(xkv["v"], W.BF16), True, mx.SCALE_UOS)
    a, sa = _two_call(dq, km, vm, False, True, mx.SCALE_UOS)
    b, sb = _fused(dq_t, km, vm, False)
    torch.cuda.synchronize()
    say(f"fused Q cross Nq={Nq} Nk={Nk} d={d} strided")
    assert torch.equal(a, b) and torch.equal(sa, sb)


@pytest.mark.parametrize("cid,heads,nrand", [(1, None, None), (5, [(0, 0), (11, 4)], 60),
                                             (4, [(2, 9)], 60), (2, [(0, 0), (0, 27)], 40)])
def test_fused_q_workloads_match_oracle(cid, heads, nrand):
    import oracle
    from parity import DELTA
    w = W.WORKLOADS[cid]
    B, H, N, d = w.shape
    say(f"fused Q parity: workload {cid} {w.describe()}")
    bits = {t: W.generate(w, t) for t in "qkv"}
    dq, dk, dv = (to_device(bits[t], w.dtype) for t in "qkv")
    km, vm = _kv(dk, dv, True, mx.SCALE_UOS)
    out, stats = _fused(dq, km, vm, w.causal)
    ref_out, ref_stats = _two_call(dq, km, vm, w.causal, True, mx.SCALE_UOS)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out) and torch.equal(stats, ref_stats)
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(H)]
        rows = np.arange(N, dtype=np.int32)
    else:
        rng = np.random.default_rng(cid)
        rows = np.unique(np.concatenate([[0, 1, 127, 128, N - 1], rng.integers(0, N, nrand)])).astype(np.int32)
    sel = {t: bits[t][[b for b, _ in heads], [h for _, h in heads]][None] for t in "qkv"}
    ref = oracle.attention(sel["q"], sel["k"], sel["v"], w.dtype, 1, len(heads), N, d, causal=w.causal,
                           kv_tile=KV_TILE, rows=rows, amb_delta=DELTA)
    o = out.cpu().numpy()
    gpu = np.stack([o[b, h][rows] for b, h in heads])[None]
    check_output(gpu, ref, f"fused Q workload {cid}", (N + KV_TILE - 1) // KV_TILE)


def test_fused_q_rejects_bad_arguments():
    x = torch.zeros((1, 2, 64, 128), dtype=torch.bfloat16, device="cuda")
    km, vm = _kv(x, x, True, mx.SCALE_UOS)
    with pytest.raises(TypeError):
        mx.forward_fused_q(x.float(), km, vm)
    with pytest.raises(RuntimeError):  # heads disagree
        mx.forward_fused_q(torch.zeros((1, 3, 64, 128), dtype=torch.bfloat16, device="cuda"), km, vm)
    with pytest.raises(RuntimeError):  # causal cross-attention
        mx.forward_fused_q(torch.zeros((1, 2, 65, 128), dtype=torch.bfloat16, device="cuda"), km, vm, causal=True)
    kq = mx.rotate_quantize_q(x, 7.0, mx.AXIS_HEAD_DIM, rotate=True)
    with pytest.raises(RuntimeError):  # ceiling-rule K^: the fused Q has no boundary to use
        mx.forward_fused_q(x, kq, vm)
