"""Parity past 2^31 elements per tensor.

Twenty thousand heads (B = 4, H = 5000) of 1024 tokens at d = 128 give
2.62e9 elements per tensor (about 50 GB of inputs, quantized tensors and
outputs in all): every element, code, scale and output offset past 2^31 must
be formed in 64 bits.  The inputs are drawn on the device (workloads'
device_normal); the oracle reads back the heads it checks, chosen on both
sides of the 2^31 element boundary (head 16384 starts exactly there) and at
the end.  Checked there, on the benchmark's single Q, K, V launch and on the
forward kernels:
  * every code and scale of those heads bit-exact against the oracle's
    quantizers ([P1] Alg. 1, Alg. 2);
  * sampled output rows of the streaming forward (non-causal and causal) and
    of the resident-key forward (512 keys) against the oracle ([P1] Alg. 2)
    at the plain bar of tests/parity.py;
  * the fused-Q forward equal to the two-call forward bit for bit;
  * the other entry points at the same shape: the Q_max sweep along d and
    along tokens, the materialized-P diagnostics and the POSTNORM reference
    mode, each on the same heads against the oracle at its own test's bar."""
import numpy as np
import pytest
import torch

import mxfp4_microscaled_bit_amd as mx
import oracle
import workloads as W
from parity import DELTA, check_output, check_row_sums, say
from test_gpu_diagnostics import _check as check_diagnostics
from test_gpu_quantize import _pack_rows, _pack_tokens
from test_gpu_sweep import SWEEP, _check_sweep

pytestmark = pytest.mark.gpu

B, H, N, d = 4, 5000, 1024, 128
NK_CROSS = 512
KV_TILE = 128
BH = B * H
# flat head index bh = b H + h; head 16384 starts at element 2^31
HEADS = [(0, 0), (2, 1999), (3, 1383), (3, 1384), (3, 4999)]
ROWS = np.array([0, 1, 127, 128, 511, 512, 700, 1022, 1023], np.int32)


def _host_bits(t, heads):
    """16-bit patterns [1, len(heads), n, d] of the listed heads of a device tensor."""
    sel = torch.stack([t[b, h] for b, h in heads]).view(torch.int16).cpu().numpy().view(np.uint16)
    return sel[None]


def _check_quantizers(qm, km, vm, bits, n_tok):
    Np = (n_tok + 127) // 128 * 128
    NB = (n_tok + 31) // 32
    nh = len(HEADS)
    idx = [b * H + h for b, h in HEADS]
    for t, m in (("q", qm), ("k", km)):
        gc = m.codes.view(BH, Np, d // 2)[idx, :n_tok].cpu().numpy().reshape(-1, d // 2)
        gs = m.scales.view(BH, Np, d // 32)[idx, :n_tok].cpu().numpy().reshape(-1, d // 32)
        oc, os_ = oracle.quantize_rows(bits[t], W.BF16, 1, nh, n_tok, d, rotate=True, rule=oracle.RULE_UOS,
                                       rows=np.arange(nh * n_tok))
        bad = int((gc != _pack_rows(oc)).sum()), int((gs != os_).sum())
        say(f"  {t}: codes/scales of {nh} heads, mismatched {bad}")
        assert bad == (0, 0)
    gc = vm.codes.view(BH, Np // 32, d, 16)[idx, :NB].cpu().numpy().reshape(-1, d, 16)
    gs = vm.scales.view(BH, Np // 32, d)[idx, :NB].cpu().numpy().reshape(-1, d)
    oc, os_ = oracle.quantize_token_blocks(bits["v"], W.BF16, 1, nh, n_tok, d, rule=oracle.RULE_UOS,
                                           blocks=np.arange(nh * NB))
    bad = int((gc != _pack_tokens(oc)).sum()), int((gs != os_).sum())
    say(f"  v: codes/scales of {nh} heads, mismatched {bad}")
    assert bad == (0, 0)


def _check_rows(out, bits, causal, nk, label):
    ref = oracle.attention(bits["q"], bits["k"], bits["v"], W.BF16, 1, len(HEADS), N, d, causal=causal,
                           kv_tile=KV_TILE, rows=ROWS, amb_delta=DELTA, Nk=nk)
    gpu = torch.stack([out[b, h][torch.from_numpy(ROWS).long().to(out.device)] for b, h in HEADS]).cpu().numpy()
    check_output(gpu[None], ref, label, (nk + KV_TILE - 1) // KV_TILE)


@pytest.mark.timeout(600)
def test_past_2_31_elements():
    say(f"large shape B={B} H={H} N={N} d={d}: {B * H * N * d} elements per tensor")
    dev = {t: W.device_normal(B, H, N, d, seed=31, tensor=t) for t in "qkv"}
    torch.cuda.synchronize()
    say("  inputs drawn")
    bits = {t: _host_bits(dev[t], HEADS) for t in "qkv"}
    qm, km, vm = mx.rotate_quantize_qkv(dev["q"], dev["k"], dev["v"], rotate=True)
    torch.cuda.synchronize()
    say("  quantized (one Q, K, V launch)")
    _check_quantizers(qm, km, vm, bits, N)

    out = mx.forward(qm, km, vm, causal=False)
    torch.cuda.synchronize()
    say("  forward (streaming, non-causal) done")
    _check_rows(out, bits, False, N, "large non-causal")
    fused = mx.forward_fused_q(dev["q"], km, vm, causal=False)
    torch.cuda.synchronize()
    assert torch.equal(fused.view(torch.int32), out.view(torch.int32)), "fused-Q and two-call outputs differ"
    del fused
    say("  fused-Q forward equal")

    mx.forward(qm, km, vm, causal=True, out=out)
    torch.cuda.synchronize()
    say("  forward (causal) done")
    _check_rows(out, bits, True, N, "large causal")
    del km, vm, dev["k"], dev["v"]
    torch.cuda.empty_cache()

    kx = W.device_normal(B, H, NK_CROSS, d, seed=32, tensor="k")
    vx = W.device_normal(B, H, NK_CROSS, d, seed=32, tensor="v")
    xb = {"q": bits["q"], "k": _host_bits(kx, HEADS), "v": _host_bits(vx, HEADS)}
    kxm = mx.rotate_quantize(kx, mx.AXIS_HEAD_DIM, rotate=True)
    vxm = mx.rotate_quantize(vx, mx.AXIS_TOKEN, rotate=False)
    mx.forward(qm, kxm, vxm, causal=False, out=out)
    torch.cuda.synchronize()
    say("  forward (resident keys, 512) done")
    _check_rows(out, xb, False, NK_CROSS, "large cross-attention")
    del out, qm, kxm, vxm, kx, vx, dev
    torch.cuda.empty_cache()


@pytest.mark.timeout(600)
def test_other_entry_points_past_2_31_elements():
    say(f"large shape, other entry points: B={B} H={H} N={N} d={d}")
    dev = {t: W.device_normal(B, H, N, d, seed=33, tensor=t) for t in "qkv"}
    torch.cuda.synchronize()
    bits = {t: _host_bits(dev[t], HEADS) for t in "qkv"}
    idx = [b * H + h for b, h in HEADS]
    for t, axis, rotate in (("q", mx.AXIS_HEAD_DIM, True), ("v", mx.AXIS_TOKEN, False)):
        gpu = mx.scale_sweep(dev[t], SWEEP, axis=axis, rotate=rotate).cpu().numpy()
        ref = oracle.scale_sweep(bits[t], W.BF16, 1, len(HEADS), N, d, SWEEP, axis=axis, rotate=rotate)
        _check_sweep(gpu[idx], ref, f"large sweep {t}")

    g = mx.p_diagnostics(dev["q"], dev["k"], rule=mx.SCALE_UOS, rotate=True, causal=False)
    torch.cuda.synchronize()
    ref, amb = oracle.p_diagnostics(bits["q"], bits["k"], W.BF16, 1, len(HEADS), N, d, causal=False, rows=ROWS,
                                    amb_delta=DELTA)
    gs = torch.stack([g[b, h][torch.from_numpy(ROWS).long().to(g.device)] for b, h in HEADS]).cpu().numpy()
    check_diagnostics(gs[None], ref, amb, "large diagnostics")
    del g

    sums = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    out = mx.quantize_reference_modes(dev["q"], dev["k"], dev["v"], rule=mx.SCALE_UOS, p_mode=mx.P_POSTNORM,
                                      rotate=True, causal=False, row_sums=sums)
    torch.cuda.synchronize()
    ref = oracle.attention(bits["q"], bits["k"], bits["v"], W.BF16, 1, len(HEADS), N, d, causal=False,
                           rotate=True, rule=oracle.RULE_UOS, p_mode=oracle.P_POSTNORM, kv_tile=KV_TILE, rows=ROWS,
                           amb_delta=DELTA)
    sel = torch.from_numpy(ROWS).long().to(out.device)
    o = torch.stack([out[b, h][sel] for b, h in HEADS]).cpu().numpy()
    check_output(o[None], ref, "large POSTNORM/UOS", (N + KV_TILE - 1) // KV_TILE)
    rs = torch.stack([sums[b, h][sel] for b, h in HEADS]).cpu().numpy()
    check_row_sums(rs[None], ref, "large POSTNORM/UOS")
    del out, sums, dev
    torch.cuda.empty_cache()
