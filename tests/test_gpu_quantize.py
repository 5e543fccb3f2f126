"""GPU parity of the MXFP4 quantizers (HIP kernels through the C ABI) with the
CPU oracle: codes and E8M0 scales must match bit for bit."""
import numpy as np
import pytest
import torch

import mxfp4_microscaled_bit_amd as mx
import oracle
import workloads as W
from parity import compare_headdim, compare_tokens, say, to_device

pytestmark = pytest.mark.gpu


def _rows_sample(B, H, N, n_random, seed, full_heads=((0, 0),)):
    rng = np.random.default_rng(seed)
    rows = set()
    for b, h in full_heads:
        rows.update(((b * H + h) * N + np.arange(N)).tolist())
    rows.update(rng.integers(0, B * H * N, n_random).tolist())
    for bh in (0, B * H - 1):  # head boundaries and the ragged tail
        rows.update([bh * N, bh * N + N - 1])
    return np.array(sorted(rows), np.int64)


def _blocks_sample(B, H, N, n_random, seed):
    NB = (N + 31) // 32
    rng = np.random.default_rng(seed)
    blocks = set(rng.integers(0, B * H * NB, n_random).tolist())
    blocks.update([0, NB - 1, B * H * NB - 1, (B * H - 1) * NB])
    return np.array(sorted(blocks), np.int64)


@pytest.mark.parametrize("cid", [1, 5])
def test_workload_quantizers_bit_exact(cid):
    """Every code and scale of the small workloads, for both rules (and, on
    workload 1, with the rotation off), one tensor per launch."""
    w = W.WORKLOADS[cid]
    B, H, N, d = w.shape
    say(f"quantizer parity: workload {cid} {w.describe()}")
    full = True
    for t in ("q", "k", "v"):
        bits = W.generate(w, t)
        dev = to_device(bits, w.dtype)
        if t in ("q", "k"):
            rows = None if full else _rows_sample(B, H, N, 20000, cid)
            rules = (mx.SCALE_UOS, mx.SCALE_OCP) if cid in (1, 5) else (mx.SCALE_UOS,)
            for rule in rules:
                for rotate in ((True, False) if cid == 1 else (True,)):
                    bc, bs, n = compare_headdim(bits, w.dtype, B, H, N, d, rotate, rule, rows=rows, dev=dev)
                    say(f"  {t} rotate={rotate} rule={rule}: {n} codes, mismatched codes {bc}, scales {bs}")
                    assert bc == 0 and bs == 0
        else:
            blocks = None if full else _blocks_sample(B, H, N, 4000, cid)
            for rule in ((mx.SCALE_UOS, mx.SCALE_OCP) if cid in (1, 5) else (mx.SCALE_UOS,)):
                bc, bs, n = compare_tokens(bits, w.dtype, B, H, N, d, rule, blocks=blocks, dev=dev)
                say(f"  v rule={rule}: {n} codes, mismatched codes {bc}, scales {bs}")
                assert bc == 0 and bs == 0
        del dev
        torch.cuda.empty_cache()


def _pack_rows(codes):
    """[n, d] one 4-bit code per byte -> [n, d/2] bytes, element 2k in the low nibble."""
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def _pack_tokens(codes):
    """[n_blocks, d, 32] one code per byte (token-minor) -> [n_blocks, d, 16] bytes."""
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cid", [2, 4, 3])
def test_whole_tensors_bit_exact_in_the_benchmark_launch(cid):
    """Every code and scale of Q, K and V at the full size of the Wan-like,
    causal-LM and Hunyuan-like workloads, from the single Q, K, V launch the
    benchmark times (rotation, UOS), against the oracle's quantizers
    ([P1] Alg. 1; Alg. 2), compared in chunks of heads as packed bytes."""
    w = W.WORKLOADS[cid]
    B, H, N, d = w.shape
    say(f"whole-tensor quantizer parity: workload {cid} {w.describe()}")
    bits = {}
    for t in "qkv":
        bits[t] = W.generate(w, t)
        say(f"  generated {t}")
    dev = {t: to_device(bits[t], w.dtype) for t in "qkv"}
    qm, km, vm = mx.rotate_quantize_qkv(dev["q"], dev["k"], dev["v"], rotate=True)
    torch.cuda.synchronize()
    del dev
    torch.cuda.empty_cache()
    Np = (N + 127) // 128 * 128
    NB = (N + 31) // 32
    BH = B * H
    chunk = max(1, (1 << 22) // N)  # heads per comparison chunk
    for t, m in (("q", qm), ("k", km)):
        gc = m.codes.view(BH, Np, d // 2)
        gs = m.scales.view(BH, Np, d // 32)
        assert (gc[:, N:] == 0).all() and (gs[:, N:] == 127).all(), "padding rows must be zeros with scale 127"
        bad_c = bad_s = 0
        for h0 in range(0, BH, chunk):
            h1 = min(BH, h0 + chunk)
            rows = (np.arange(h0, h1)[:, None] * N + np.arange(N)[None, :]).reshape(-1)
            oc, os_ = oracle.quantize_rows(bits[t], w.dtype, B, H, N, d, rotate=True, rule=oracle.RULE_UOS,
                                           rows=rows)
            bad_c += int((gc[h0:h1, :N].cpu().numpy().reshape(-1, d // 2) != _pack_rows(oc)).sum())
            bad_s += int((gs[h0:h1, :N].cpu().numpy().reshape(-1, d // 32) != os_).sum())
        say(f"  {t}: {BH * N * d} codes, {BH * N * d // 32} scales compared; mismatched bytes {bad_c}, "
            f"scales {bad_s}")
        assert bad_c == 0 and bad_s == 0
    gc = vm.codes.view(BH, Np // 32, d, 16)
    gs = vm.scales.view(BH, Np // 32, d)
    assert (gc[:, NB:] == 0).all() and (gs[:, NB:] == 127).all(), "padding blocks must be zeros with scale 127"
    bad_c = bad_s = 0
    for h0 in range(0, BH, chunk):
        h1 = min(BH, h0 + chunk)
        blocks = (np.arange(h0, h1)[:, None] * NB + np.arange(NB)[None, :]).reshape(-1)
        oc, os_ = oracle.quantize_token_blocks(bits["v"], w.dtype, B, H, N, d, rule=oracle.RULE_UOS, blocks=blocks)
        bad_c += int((gc[h0:h1, :NB].cpu().numpy().reshape(-1, d, 16) != _pack_tokens(oc)).sum())
        bad_s += int((gs[h0:h1, :NB].cpu().numpy().reshape(-1, d) != os_).sum())
    say(f"  v: {BH * NB * 32 * d} codes, {BH * NB * d} scales compared; mismatched bytes {bad_c}, scales {bad_s}")
    assert bad_c == 0 and bad_s == 0


@pytest.mark.parametrize("N", [1, 31, 33, 127, 129, 200])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", [W.BF16, W.FP16])
def test_ragged_shapes(N, d, dtype):
    say(f"quantizer ragged N={N} d={d} dtype={dtype}")
    x = W.custom(2, 3, N, d, dtype=dtype, seed=N * d, scale=3.0)
    for rotate in (True, False):
        for rule in (mx.SCALE_UOS, mx.SCALE_OCP):
            bc, bs, _ = compare_headdim(x["q"], dtype, 2, 3, N, d, rotate, rule)
            assert bc == 0 and bs == 0, (rotate, rule)
    for rule in (mx.SCALE_UOS, mx.SCALE_OCP):
        bc, bs, _ = compare_tokens(x["v"], dtype, 2, 3, N, d, rule)
        assert bc == 0 and bs == 0, rule


def _special_bits(N, d, dtype, seed):
    """Inputs full of edge values: zeros of both signs, subnormals, exact
    E2M1 ties after scaling, UOS/OCP boundary maxima, huge values."""
    rng = np.random.default_rng(seed)
    specials = np.array([0.0, -0.0, 1.0, -1.0, 14.5, 7.25, 3.625, 2.5, 5.0, 0.75, 1.75, 0.25, 6.0, 7.0,
                         3.5, 1.25, 12.0, -12.0, 1e-38, -1e-39, 6e-8, 3e4, -65000.0, 2.0 ** -126, 2.0 ** -133,
                         1e30, -3e38, 0.5 * 29 / 16 * 2, 29.0, 58.0, 0.453125])
    if dtype == W.FP16:
        specials = specials[np.abs(specials) < 65000]
    vals = rng.choice(specials, size=(1, 2, N, d))
    scale_pow = rng.integers(-20, 20, size=(1, 2, N, 1)).astype(np.float64)
    if dtype == W.FP16:
        scale_pow = np.clip(scale_pow, -4, 4)
    vals = vals * np.exp2(scale_pow)
    lim = 6.0e4 if dtype == W.FP16 else 1.0e37  # keep every input finite
    vals = np.clip(vals, -lim, lim)
    zero_rows = rng.random((1, 2, N)) < 0.1
    vals[zero_rows] = 0.0
    return W.to_bits(vals, dtype)


@pytest.mark.parametrize("dtype", [W.BF16, W.FP16])
@pytest.mark.parametrize("d", [64, 128])
def test_special_values(dtype, d):
    N = 300
    say(f"quantizer special values d={d} dtype={dtype}")
    bits = _special_bits(N, d, dtype, seed=d + dtype)
    for rotate in (True, False):
        for rule in (mx.SCALE_UOS, mx.SCALE_OCP):
            bc, bs, _ = compare_headdim(bits, dtype, 1, 2, N, d, rotate, rule)
            assert bc == 0 and bs == 0, (rotate, rule)
    for rule in (mx.SCALE_UOS, mx.SCALE_OCP):
        bc, bs, _ = compare_tokens(bits, dtype, 1, 2, N, d, rule)
        assert bc == 0 and bs == 0, rule


def test_every_bf16_value_through_the_element_rounding():
    """All finite bf16 values of magnitude <= 4 as V tokens next to a block
    maximum of 4, 8 or 2 (exponent 0, +1, -1 under both rules), so every
    value goes through the E2M1 rounding at three scales."""
    say("quantizer exhaustive bf16 values")
    allbits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):  # signalling-NaN patterns, dropped on the next line
        vals = W.from_bits(allbits, W.BF16).astype(np.float64)
    vals = vals[np.isfinite(vals) & (np.abs(vals) <= 4.0)]
    per_block = 31
    nblk = (vals.size + per_block - 1) // per_block
    flat = np.zeros(nblk * per_block)
    flat[:vals.size] = vals
    base = np.zeros((nblk, 32))
    base[:, :per_block] = flat.reshape(nblk, per_block)
    blocks = []
    for mmax in (4.0, 8.0, 2.0):
        b = base.copy()
        b[:, 31] = mmax
        blocks.append(b)
    blocks = np.concatenate(blocks)                 # [nb, 32]
    d = 128
    nkb = (blocks.shape[0] + d - 1) // d
    grid = np.zeros((nkb * d, 32))
    grid[:blocks.shape[0]] = blocks
    # channel c of token block kb carries block kb*d + c
    v = grid.reshape(nkb, d, 32).transpose(0, 2, 1).reshape(1, 1, nkb * 32, d)
    bits = W.to_bits(v, W.BF16)
    assert (W.from_bits(bits, W.BF16) == v).all()
    for rule in (mx.SCALE_UOS, mx.SCALE_OCP):
        bc, bs, n = compare_tokens(bits, W.BF16, 1, 1, nkb * 32, d, rule)
        say(f"  rule={rule}: {n} codes, mismatched {bc}/{bs}")
        assert bc == 0 and bs == 0


def test_strided_input_layout():
    """A [B, N, H, d] buffer viewed as [B, H, N, d] (no copy) quantizes like the
    contiguous tensor."""
    B, H, N, d = 2, 3, 150, 128
    x = W.custom(B, N, H, d, seed=77, tensors=("q",))["q"]  # physical [B, N, H, d]
    dev = to_device(x, W.BF16).permute(0, 2, 1, 3)              # logical [B, H, N, d]
    contig = np.ascontiguousarray(x.transpose(0, 2, 1, 3))
    say("quantizer strided input")
    for axis in (mx.AXIS_HEAD_DIM, mx.AXIS_TOKEN):
        a = mx.rotate_quantize(dev, axis, rotate=(axis == mx.AXIS_HEAD_DIM))
        b = mx.rotate_quantize(to_device(contig, W.BF16), axis, rotate=(axis == mx.AXIS_HEAD_DIM))
        torch.cuda.synchronize()
        assert torch.equal(a.codes, b.codes) and torch.equal(a.scales, b.scales)
    bc, bs, _ = compare_headdim(contig, W.BF16, B, H, N, d, True, mx.SCALE_UOS)
    assert bc == 0 and bs == 0


def test_quantizer_is_deterministic():
    w = W.WORKLOADS[1]
    dev = to_device(W.generate(w, "q"), w.dtype)
    a = mx.rotate_quantize(dev, mx.AXIS_HEAD_DIM)
    b = mx.rotate_quantize(dev, mx.AXIS_HEAD_DIM)
    torch.cuda.synchronize()
    assert torch.equal(a.codes, b.codes) and torch.equal(a.scales, b.scales)


def test_binding_rejects_short_buffers_before_launch():
    """A caller-provided MXFP4 tensor or output too short for the call is
    refused before any kernel runs."""
    say("binding: short buffers are refused")
    x = torch.zeros(1, 1, 256, 128, dtype=torch.bfloat16, device="cuda")
    short = mx.MXTensor(torch.empty(100, dtype=torch.uint8, device="cuda"),
                        torch.empty(100, dtype=torch.uint8, device="cuda"), (1, 1, 256, 128), mx.AXIS_HEAD_DIM)
    with pytest.raises(ValueError, match="bytes"):
        mx.rotate_quantize(x, out=short)
    good = mx.rotate_quantize(x)
    v = mx.rotate_quantize(x, mx.AXIS_TOKEN, rotate=False)
    with pytest.raises(ValueError, match="bytes"):
        mx.forward(short, good, v)
    with pytest.raises(ValueError, match="bytes"):
        mx.scale_sweep(x, [6.0, 7.25], out=torch.empty(1, dtype=torch.float64, device="cuda"))
    with pytest.raises(ValueError, match="bytes"):
        mx.p_diagnostics(x, x, out=torch.empty(10, dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()


@pytest.mark.parametrize("B,H,Nq,Nk,d,dt,rotate,rule", [
    (1, 3, 300, 300, 128, torch.bfloat16, True, mx.SCALE_UOS),
    (2, 2, 129, 4100, 64, torch.float16, True, mx.SCALE_OCP),
    (1, 2, 1, 33, 128, torch.bfloat16, False, mx.SCALE_UOS),
    (3, 1, 1000, 77, 64, torch.bfloat16, False, mx.SCALE_OCP),
])
def test_qkv_launch_equals_three_calls(B, H, Nq, Nk, d, dt, rotate, rule):
    """The single Q, K, V launch writes exactly what three separate quantizer
    calls write, padding included, for contiguous and strided inputs."""
    say(f"qkv launch: B{B} H{H} Nq{Nq} Nk{Nk} d{d} {dt} rotate={rotate} rule={rule}")
    g = torch.Generator(device="cpu").manual_seed(Nq * 7 + Nk)
    q = (torch.randn(B, H, Nq, d, generator=g) * 3).to(dt).cuda()
    k = (torch.randn(B, H, Nk, d, generator=g) * 0.5).to(dt).cuda()
    # V as a strided view: every other token of a longer tensor
    vbig = (torch.randn(B, H, 2 * Nk, d, generator=g) * 20).to(dt).cuda()
    v = vbig[:, :, ::2]
    refs = (mx.rotate_quantize(q, mx.AXIS_HEAD_DIM, rotate=rotate, rule=rule),
            mx.rotate_quantize(k, mx.AXIS_HEAD_DIM, rotate=rotate, rule=rule),
            mx.rotate_quantize(v, mx.AXIS_TOKEN, rotate=False, rule=rule))
    outs = mx.rotate_quantize_qkv(q, k, v, rotate=rotate, rule=rule)
    torch.cuda.synchronize()
    for name, r, o in zip("qkv", refs, outs):
        assert torch.equal(r.codes, o.codes), name
        assert torch.equal(r.scales, o.scales), name
        assert (o.shape, o.axis, o.rule, o.rotated) == (r.shape, r.axis, r.rule, r.rotated), name


def test_token_blocks_at_the_exponent_clamp_next_to_subnormal_blocks():
    """V token blocks whose maximum is tiny enough for the clamp e = -127,
    beside blocks of the neighbouring channel with e = -126 or -125 that
    hold subnormal values: both channels of a lane pair go through the
    clamp path's rescaling, and every code must match the oracle."""
    say("token quantizer: clamp exponent next to subnormal blocks")
    N, d = 96, 64
    rng = np.random.default_rng(11)
    vals = np.zeros((1, 1, N, d))
    tiny = 2.0 ** -133 * rng.integers(-40, 41, size=(N, d // 2))   # bf16 subnormals, max < 2^-127
    small = 2.0 ** -133 * rng.integers(-900, 901, size=(N, d // 2))  # subnormals up to ~2^-123
    vals[0, 0, :, 0::2] = tiny
    vals[0, 0, :, 1::2] = small
    vals[0, 0, 5, 1::4] = 2.0 ** -126 * 7.0  # some neighbour blocks with a normal maximum
    bits = W.to_bits(vals, W.BF16)
    for rule in (mx.SCALE_UOS, mx.SCALE_OCP):
        bc, bs, n = compare_tokens(bits, W.BF16, 1, 1, N, d, rule)
        assert bc == 0 and bs == 0, rule
    # the same blocks through the single Q, K, V launch
    x = to_device(bits, W.BF16)
    ref = mx.rotate_quantize(x, mx.AXIS_TOKEN, rotate=False)
    _, _, vm = mx.rotate_quantize_qkv(x, x, x, rotate=False)
    torch.cuda.synchronize()
    assert torch.equal(ref.codes, vm.codes) and torch.equal(ref.scales, vm.scales)


def test_qkv_launch_equals_three_calls_at_the_benchmark_shape():
    """The benchmark's quantizer launch (one mxattn_rotate_quantize_qkv over the
    full Wan-like Q, K, V) writes exactly what the three separate calls write;
    the separate calls are compared with the oracle on sampled rows and blocks
    by test_workload_quantizers_bit_exact."""
    w = W.WORKLOADS[2]
    say(f"qkv launch at the benchmark shape: {w.describe()}")
    dev = {t: to_device(W.generate(w, t), w.dtype) for t in "qkv"}
    refs = (mx.rotate_quantize(dev["q"], mx.AXIS_HEAD_DIM, rotate=True),
            mx.rotate_quantize(dev["k"], mx.AXIS_HEAD_DIM, rotate=True),
            mx.rotate_quantize(dev["v"], mx.AXIS_TOKEN, rotate=False))
    outs = mx.rotate_quantize_qkv(dev["q"], dev["k"], dev["v"], rotate=True)
    torch.cuda.synchronize()
    for name, r, o in zip("qkv", refs, outs):
        assert torch.equal(r.codes, o.codes), name
        assert torch.equal(r.scales, o.scales), name
