"""The ablation and analysis entry points on seeded random shapes, every row
against the oracle.

Sixty cases drawn once from a fixed seed: d in {64, 128}, B and H up to 2
and 3, 1 to 600 tokens, causal or not, bf16 or fp16, standard normals
scaled by 0.5 to 3.  Each case runs one reference mode (cycling through the
vanilla OCP baseline, post-normalization under OCP and UOS, DIRECT/UOS and
PNQ under OCP; [P1] Sec. 4.2 Eq. 42, Sec. 5.5.2) with outputs and induced
row sums at the plain bar of tests/parity.py, the materialized-P
diagnostics under UOS or OCP with a random pre-quantization scale gamma
([P1] Sec. 5.5.2, Fig. 7), and the Q_max sweep along d or along tokens
([P1] Sec. 5.5.1)."""
import numpy as np
import pytest
import torch

import mxfp4_microscaled_bit_amd as mx
import oracle
import workloads as W
from parity import DELTA, check_output, check_row_sums, say, to_device
from test_gpu_diagnostics import _check as check_diagnostics
from test_gpu_sweep import SWEEP, _check_sweep

pytestmark = pytest.mark.gpu

KV_TILE = 128
MODES = [(mx.P_DIRECT, mx.SCALE_OCP, False), (mx.P_POSTNORM, mx.SCALE_OCP, True),
         (mx.P_POSTNORM, mx.SCALE_UOS, True), (mx.P_DIRECT, mx.SCALE_UOS, True), (mx.P_PNQ, mx.SCALE_OCP, True)]


def _cases(n=60, seed=20261203):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        d = int(rng.choice([64, 128]))
        B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
        N = int(rng.integers(1, 601))
        causal = bool(rng.integers(0, 2))
        dtype = int(rng.choice([W.BF16, W.FP16]))
        scale = float(rng.choice([0.5, 1.5, 3.0]))
        gamma = float(rng.choice([1.0, 1.25, 0.7, 3.0]))
        out.append((i, B, H, N, d, causal, dtype, scale, gamma))
    return out


CASES = _cases()


@pytest.mark.parametrize("i,B,H,N,d,causal,dtype,scale,gamma", CASES,
                         ids=[f"{c[0]}-B{c[1]}H{c[2]}n{c[3]}d{c[4]}{'c' if c[5] else ''}" for c in CASES])
def test_random_modes_match_oracle(i, B, H, N, d, causal, dtype, scale, gamma):
    p_mode, rule, rotate = MODES[i % len(MODES)]
    label = f"random modes case {i}: B={B} H={H} N={N} d={d} causal={causal} dtype={dtype} mode {p_mode}/{rule}"
    say(label)
    x = W.custom(B, H, N, d, dtype=dtype, seed=7000 + i, scale=scale)
    dev = {t: to_device(x[t], dtype) for t in "qkv"}
    sums = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    out = mx.quantize_reference_modes(dev["q"], dev["k"], dev["v"], rule=rule, p_mode=p_mode, rotate=rotate,
                                      causal=causal, row_sums=sums)
    torch.cuda.synchronize()
    ref = oracle.attention(x["q"], x["k"], x["v"], dtype, B, H, N, d, causal=causal, rotate=rotate, rule=rule,
                           p_mode=p_mode, kv_tile=KV_TILE, amb_delta=DELTA)
    check_output(out.cpu().numpy(), ref, label, (N + KV_TILE - 1) // KV_TILE)
    check_row_sums(sums.cpu().numpy(), ref, label)

    grule, orule = ((mx.SCALE_UOS, oracle.RULE_UOS), (mx.SCALE_OCP, oracle.RULE_OCP))[i % 2]
    g = mx.p_diagnostics(dev["q"], dev["k"], rule=grule, rotate=True, causal=causal, gamma=gamma)
    torch.cuda.synchronize()
    rd, amb = oracle.p_diagnostics(x["q"], x["k"], dtype, B, H, N, d, causal=causal, rotate=True, rule=orule,
                                   gamma=gamma, amb_delta=DELTA)
    check_diagnostics(g.cpu().numpy(), rd, amb, label + " diagnostics")

    axis = (mx.AXIS_HEAD_DIM, mx.AXIS_TOKEN)[(i // 2) % 2]
    rot = axis == mx.AXIS_HEAD_DIM
    sw = mx.scale_sweep(dev["k"], SWEEP, axis=axis, rotate=rot).cpu().numpy()
    rs = oracle.scale_sweep(x["k"], dtype, B, H, N, d, SWEEP, axis=axis, rotate=rot)
    _check_sweep(sw, rs, label + " sweep")
