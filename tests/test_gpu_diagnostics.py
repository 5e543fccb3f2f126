"""GPU parity of the row-sum diagnostics of materialized-P quantization
(MXAttention, Sec. 5.5.2 and Fig. 7) with the CPU oracle.

mxattn_p_diagnostics evaluates P = softmax(S) in binary32 from the exact row
statistics of a first pass; the oracle does it in binary64.  Per row and per
field the bar is

  |gpu - oracle| <= amb + 2^-12          fields 0..4 (row sum, zeroing,
                                         saturation, down, up)
  |gpu - oracle| <= 2^-12 (1 + H_ref)    field 5 (entropy, nats)

amb is the oracle's sum over the row of the largest change of P^_ij that a
quantizer decision within relative margin DELTA of its threshold can make
(the two sides may legitimately take such a decision differently); 2^-12
covers the binary32 evaluation of P (relative error below 2^-14, summed over
a row whose P sums to 1) and the binary32 sums.  An element whose outcome
class flips with such a decision moves its error term between two fields by
at most its own change of P^, so the same bound holds field by field.

Oracle-free properties on the GPU: the partition identity
row sum - 1 = zeroing + saturation + down + up; a power-of-two gamma leaves
every field bit-identical (gamma only shifts the block exponents).
"""
import numpy as np
import pytest
import torch

import mxfp4_microscaled_bit_amd as mx
import oracle
import workloads as W
from parity import DELTA, say, to_device

pytestmark = pytest.mark.gpu

TOL = 2.0 ** -12
NAMES = ("row sum", "zeroing", "saturation", "down", "up", "entropy")


def _check(gpu, ref, amb, label):
    gpu = gpu.astype(np.float64)
    assert np.isfinite(gpu).all(), f"{label}: non-finite diagnostics"
    diff = np.abs(gpu - ref)
    bound = np.empty_like(ref)
    bound[..., :5] = amb[..., None] + TOL
    bound[..., 5] = TOL * (1.0 + np.abs(ref[..., 5]))
    worst = [float(diff[..., k].max()) for k in range(6)]
    say(f"[{label}] max|diff| " + " ".join(f"{n}={w:.2e}" for n, w in zip(NAMES, worst)) +
        f" max amb={float(amb.max()):.2e} rows={ref.shape[-2]}")
    assert (diff <= bound).all(), f"{label}: field {int(np.argmax((diff - bound).max(axis=tuple(range(diff.ndim - 1)))))}" \
                                  f" exceeds its bound by {float((diff - bound).max()):.3e}"


def _gpu_diag(x, dtype, **kw):
    dq, dk = to_device(x["q"], dtype), to_device(x["k"], dtype)
    out = mx.p_diagnostics(dq, dk, **kw)
    torch.cuda.synchronize()
    return out.cpu().numpy()


RULES = {"uos": (mx.SCALE_UOS, oracle.RULE_UOS), "ocp": (mx.SCALE_OCP, oracle.RULE_OCP)}


@pytest.mark.parametrize("rule", ["uos", "ocp"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_diagnostics_match_oracle_small(rule, d, causal):
    gr, orl = RULES[rule]
    for N, gamma, rotate, seed in ((1, 1.0, True, 1), (31, 1.0, True, 2), (129, 1.25, True, 3),
                                  (300, 1.0, False, 4), (257, 0.375, True, 5)):
        B, H = 2, 2
        x = W.custom(B, H, N, d, dtype=W.BF16, seed=seed, scale=2.0, tensors=("q", "k"))
        g = _gpu_diag(x, W.BF16, rule=gr, rotate=rotate, causal=causal, gamma=gamma)
        ref, amb = oracle.p_diagnostics(x["q"], x["k"], W.BF16, B, H, N, d, causal=causal, rotate=rotate,
                                        rule=orl, gamma=gamma, amb_delta=DELTA)
        _check(g, ref, amb, f"{rule} d={d} N={N} causal={causal} gamma={gamma} rotate={rotate}")


def _heads_bits(w, heads):
    return {t: W.generate(w, t, heads=heads)[None] for t in "qk"}


@pytest.mark.parametrize("cid,heads,nrows", [
    (1, None, None),
    (5, [(0, 0), (7, 3)], 96),
    (4, [(1, 5)], 64),
    (2, [(0, 0), (0, 31)], 48),
])
def test_diagnostics_workloads(cid, heads, nrows):
    """Every field on the workload inputs: all rows of the small workload,
    sampled rows of one or two heads of the larger ones (the GPU runs the
    whole problem at its full size; the oracle computes the sampled rows)."""
    w = W.WORKLOADS[cid]
    B, H, N, d = w.shape
    say(f"diagnostics parity: workload {cid} {w.describe()}")
    if heads is None:
        bits = {t: W.generate(w, t) for t in "qk"}
        g = _gpu_diag(bits, w.dtype, causal=w.causal)
        ref, amb = oracle.p_diagnostics(bits["q"], bits["k"], w.dtype, B, H, N, d, causal=w.causal,
                                        amb_delta=DELTA)
        _check(g, ref, amb, f"workload {cid} all rows")
        return
    full = {t: W.generate(w, t) for t in "qk"}
    g = _gpu_diag(full, w.dtype, causal=w.causal)
    rng = np.random.default_rng(cid)
    rows = np.unique(np.concatenate([[0, 1, 127, 128, N - 1], rng.integers(0, N, nrows)])).astype(np.int32)
    sel = _heads_bits(w, heads)
    ref, amb = oracle.p_diagnostics(sel["q"], sel["k"], w.dtype, 1, len(heads), N, d, causal=w.causal,
                                    rows=rows, amb_delta=DELTA)
    gs = np.stack([g[b, h][rows] for b, h in heads])[None]
    _check(gs, ref, amb, f"workload {cid} sampled rows")
    # the row statistic of the page's figure: mean induced row sum, reported only
    say(f"  mean row sum {float(gs[..., 0].mean()):.4f} (oracle {float(ref[..., 0].mean()):.4f}); "
        f"mean entropy {float(gs[..., 5].mean()):.3f} nats")


def test_partition_identity_and_power_of_two_gamma():
    B, H, N, d = 1, 4, 700, 128
    x = W.custom(B, H, N, d, dtype=W.BF16, seed=11, scale=3.0, tensors=("q", "k"))
    g1 = _gpu_diag(x, W.BF16)
    part = g1[..., 1:5].astype(np.float64).sum(-1)
    assert np.abs((g1[..., 0].astype(np.float64) - 1.0) - part).max() <= 2.0 ** -16
    for gamma in (2.0, 0.25, 2.0 ** 10):
        gg = _gpu_diag(x, W.BF16, gamma=gamma)
        assert np.array_equal(gg, g1), f"gamma={gamma} changed the diagnostics"
    g3 = _gpu_diag(x, W.BF16, gamma=1.5)
    assert not np.array_equal(g3[..., 0], g1[..., 0])


def test_diagnostics_reject_bad_arguments():
    x = torch.zeros((1, 1, 64, 128), dtype=torch.bfloat16, device="cuda")
    for gamma in (0.0, -1.0, float("nan"), 2.0 ** 21):
        with pytest.raises(RuntimeError):
            mx.p_diagnostics(x, x, gamma=gamma)
    with pytest.raises(RuntimeError):
        mx.p_diagnostics(x, x, rule=mx.SCALE_CEIL_Q)


@pytest.mark.parametrize("dtype", [W.BF16, W.FP16])
def test_diagnostics_strided_layout_and_dtype(dtype):
    """Q and K in [B, N, H, d] buffers viewed as [B, H, N, d] (no copy), bf16
    and fp16, causal: every field equals the contiguous call's bit for bit and
    the oracle's at the bar above."""
    B, H, N, d = 2, 3, 200, 128
    x = W.custom(B, N, H, d, dtype=dtype, seed=93, tensors=("q", "k"), scale=2.0)
    dev = {t: to_device(x[t], dtype).permute(0, 2, 1, 3) for t in "qk"}
    contig = {t: np.ascontiguousarray(x[t].transpose(0, 2, 1, 3)) for t in "qk"}
    dc = {t: to_device(contig[t], dtype) for t in "qk"}
    a = mx.p_diagnostics(dev["q"], dev["k"], causal=True)
    b = mx.p_diagnostics(dc["q"], dc["k"], causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32)), "strided and contiguous diagnostics differ"
    ref, amb = oracle.p_diagnostics(contig["q"], contig["k"], dtype, B, H, N, d, causal=True, rotate=True,
                                    amb_delta=DELTA)
    _check(a.cpu().numpy(), ref, amb, f"strided dtype={dtype}")
