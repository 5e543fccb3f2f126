"""GPU parity of the fused MXFP4 attention forward (and its reference modes)
with the CPU oracle, plus oracle-free invariants of the method on the GPU."""
import math

import numpy as np
import pytest
import torch

import mxfp4_microscaled_bit_amd as mx
import oracle
import workloads as W
from parity import DELTA, check_output, check_row_sums, run_forward, say, to_device

pytestmark = pytest.mark.gpu

KV_TILE = 128


def _sample_rows(N, n_random, seed, causal=False):
    rng = np.random.default_rng(seed)
    rows = {0, 1, N - 1, N - 2, 127, 128, 129, N // 2}
    rows.update(range(max(0, N - 130), N, 37))
    rows.update(rng.integers(0, N, n_random).tolist())
    return np.array(sorted(r for r in rows if 0 <= r < N), np.int32)


def _oracle_heads(w, heads, rows, p_mode=oracle.P_PNQ, rule=oracle.RULE_UOS, rotate=True, bits=None):
    """Oracle on the listed (b, h) heads only: they are independent, so the
    oracle sees a [1, len(heads), N, d] problem."""
    sel = {t: (bits[t][[b for b, _ in heads], [h for _, h in heads]][None] if bits else
               W.generate(w, t, heads=heads)[None]) for t in "qkv"}
    return oracle.attention(sel["q"], sel["k"], sel["v"], w.dtype, 1, len(heads), w.N, w.d, causal=w.causal,
                            rotate=rotate, rule=rule, p_mode=p_mode, kv_tile=KV_TILE, rows=rows,
                            amb_delta=DELTA, Nk=w.kv_tokens)


def _gpu_rows(out, heads, rows):
    o = out.cpu().numpy() if isinstance(out, torch.Tensor) else out
    return np.stack([o[b, h][rows] for b, h in heads])[None]


WORKLOAD_SAMPLING = {
    # cid: (heads to compare, random rows per head)
    1: (None, None),
    5: ([(0, 0), (3, 7), (9, 2), (15, 15)], 60),
    4: ([(0, 0), (1, 17), (3, 31)], 60),
    2: ([(0, 0), (0, 19), (0, 39)], 40),
    3: ([(0, 0), (0, 23)], 16),
    6: ([(0, 0), (0, 21), (0, 39)], 200),
}


@pytest.mark.parametrize("cid", [1, 5, 4, 2, 3, 6])
def test_forward_matches_oracle(cid):
    w = W.WORKLOADS[cid]
    B, H, N, d = w.shape
    say(f"forward parity: workload {cid} {w.describe()}")
    bits = {t: W.generate(w, t) for t in "qkv"}
    dev = {t: to_device(bits[t], w.dtype) for t in "qkv"}
    out, stats = run_forward(dev["q"], dev["k"], dev["v"], w.causal)
    heads, nrand = WORKLOAD_SAMPLING[cid]
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(H)]
        rows = np.arange(N, dtype=np.int32)
    else:
        rows = _sample_rows(N, nrand, cid, w.causal)
    ref = _oracle_heads(w, heads, rows, bits=bits)
    gpu = _gpu_rows(out, heads, rows)
    n_tiles = (w.kv_tokens + KV_TILE - 1) // KV_TILE
    check_output(gpu, ref, f"workload {cid} PNQ", n_tiles)
    st = _gpu_rows(stats, heads, rows)
    # App. J: l >= 1 for every row; l and m agree with the oracle
    assert (st[..., 1] >= 1.0).all()
    lrel = np.abs(st[..., 1] - ref["l"]) / ref["l"]
    say(f"  l: max rel diff {lrel.max():.2e}; m: max abs diff {np.abs(st[..., 0] - ref['m']).max():.2e}")
    assert ((lrel <= 1e-4) | (ref["amb"].max(axis=-1) > 0)).all()
    assert np.allclose(st[..., 0], ref["m"], rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("p_mode,rule,rotate", [
    (mx.P_PNQ, mx.SCALE_UOS, True),
    (mx.P_PNQ, mx.SCALE_OCP, True),
    (mx.P_DIRECT, mx.SCALE_OCP, False),   # vanilla OCP MXFP4 baseline (Sec. 5.2)
    (mx.P_DIRECT, mx.SCALE_UOS, True),
    (mx.P_POSTNORM, mx.SCALE_UOS, True),  # materialized-P diagnostic (Sec. 5.5.2)
    (mx.P_POSTNORM, mx.SCALE_OCP, False),
    (mx.P_PNQ, mx.SCALE_UOS, False),      # rotation off
])
@pytest.mark.parametrize("cid", [1, 5])
def test_reference_modes_match_oracle(cid, p_mode, rule, rotate):
    w = W.WORKLOADS[cid]
    B, H, N, d = w.shape
    say(f"reference modes: workload {cid} p_mode={p_mode} rule={rule} rotate={rotate}")
    bits = {t: W.generate(w, t) for t in "qkv"}
    dev = {t: to_device(bits[t], w.dtype) for t in "qkv"}
    sums = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    out = mx.quantize_reference_modes(dev["q"], dev["k"], dev["v"], rule=rule, p_mode=p_mode, rotate=rotate,
                                      causal=w.causal, row_sums=sums)
    torch.cuda.synchronize()
    if cid == 1:
        heads = [(0, 0), (0, 1)]
        rows = np.arange(N, dtype=np.int32)
    else:
        heads = [(0, 0), (7, 9)]
        rows = _sample_rows(N, 40, 5)
    ref = _oracle_heads(w, heads, rows, p_mode=p_mode, rule=rule, rotate=rotate, bits=bits)
    check_output(_gpu_rows(out, heads, rows), ref, f"workload {cid} mode {p_mode}/{rule}/{rotate}",
                 (N + KV_TILE - 1) // KV_TILE)
    rs = _gpu_rows(sums, heads, rows)
    if p_mode == mx.P_PNQ:
        assert np.abs(rs - 1).max() < 1e-5  # Prop. 1 on the GPU
    else:
        check_row_sums(rs, ref, f"workload {cid} mode {p_mode}/{rule}/{rotate}")
    say(f"  induced row sums: gpu mean {rs.mean():.5f} [{rs.min():.4f}, {rs.max():.4f}] "
        f"oracle mean {ref['rowsum'].mean():.5f}")
    # the PNQ-through-reference-modes path equals quantize x3 + forward bit for bit
    if p_mode == mx.P_PNQ and rule == mx.SCALE_UOS and rotate:
        direct_out, _ = run_forward(dev["q"], dev["k"], dev["v"], w.causal, with_stats=False)
        assert torch.equal(direct_out, out)


@pytest.mark.parametrize("N", [1, 2, 31, 127, 128, 129, 200, 300])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_ragged_and_tiny_shapes(N, d, causal):
    say(f"forward ragged N={N} d={d} causal={causal}")
    B, H = 2, 2
    x = W.custom(B, H, N, d, seed=N + d, scale=2.0)
    dev = {t: to_device(x[t], W.BF16) for t in "qkv"}
    out, stats = run_forward(dev["q"], dev["k"], dev["v"], causal)
    ref = oracle.attention(x["q"], x["k"], x["v"], W.BF16, B, H, N, d, causal=causal, kv_tile=KV_TILE,
                           amb_delta=DELTA)
    check_output(out.cpu().numpy(), ref, f"N={N} d={d} causal={causal}", (N + KV_TILE - 1) // KV_TILE)
    assert (stats.cpu().numpy()[..., 1] >= 1.0).all()


@pytest.mark.parametrize("Nq,Nk,d", [(300, 77, 128), (1000, 512, 128), (129, 1, 64), (5, 700, 128),
                                     (256, 128, 64), (131, 4100, 128)])
def test_cross_attention_matches_oracle(Nq, Nk, d):
    """Cross-attention: Nq query rows against Nk key/value tokens (ragged on
    both sides, a single key, fewer keys than one tile, many tiles)."""
    say(f"cross-attention Nq={Nq} Nk={Nk} d={d}")
    B, H = 2, 3
    xq = W.custom(B, H, Nq, d, seed=Nq + d, scale=2.0)
    xkv = W.custom(B, H, Nk, d, seed=Nk + 7 * d, scale=2.0)
    out, stats = run_forward(to_device(xq["q"], W.BF16), to_device(xkv["k"], W.BF16), to_device(xkv["v"], W.BF16),
                             False)
    assert tuple(out.shape) == (B, H, Nq, d)
    ref = oracle.attention(xq["q"], xkv["k"], xkv["v"], W.BF16, B, H, Nq, d, kv_tile=KV_TILE, amb_delta=DELTA,
                           Nk=Nk)
    check_output(out.cpu().numpy(), ref, f"cross Nq={Nq} Nk={Nk} d={d}", (Nk + KV_TILE - 1) // KV_TILE)
    st = stats.cpu().numpy()
    assert (st[..., 1] >= 1.0).all()
    assert np.allclose(st[..., 0], ref["m"], rtol=1e-5, atol=1e-5)


def test_cross_attention_rows_equal_self_attention_rows():
    """Every query row is independent of the others: placing the Nq queries
    among the rows of a self-attention problem over the same K^, V^ gives the
    same output rows bit for bit."""
    B, H, Nq, Nk, d = 1, 2, 77, 600, 128
    xq = W.custom(B, H, Nq, d, seed=21, scale=2.0)
    xkv = W.custom(B, H, Nk, d, seed=22, scale=2.0)
    big = W.custom(B, H, Nk, d, seed=23, scale=2.0)["q"].copy()
    pos = np.arange(Nq) * 7 + 5
    big[:, :, pos] = xq["q"]
    dk, dv = to_device(xkv["k"], W.BF16), to_device(xkv["v"], W.BF16)
    cross, _ = run_forward(to_device(xq["q"], W.BF16), dk, dv, False)
    selfo, _ = run_forward(to_device(big, W.BF16), dk, dv, False)
    say("cross rows vs self-attention rows")
    assert torch.equal(cross, selfo[:, :, torch.from_numpy(pos).long().cuda()])


def test_fp16_inputs():
    w = W.WORKLOADS[1]
    assert w.dtype == W.FP16
    x = W.custom(1, 3, 500, 128, dtype=W.FP16, seed=3, scale=2.0)
    dev = {t: to_device(x[t], W.FP16) for t in "qkv"}
    say("forward fp16 inputs")
    out, _ = run_forward(dev["q"], dev["k"], dev["v"], False)
    ref = oracle.attention(x["q"], x["k"], x["v"], W.FP16, 1, 3, 500, 128, amb_delta=DELTA)
    check_output(out.cpu().numpy(), ref, "fp16", 4)


# ----------------------------------------------------------------------------
# invariants that need no oracle


def test_constant_values_give_their_quantized_value_exactly():
    """PNQ normalizes by the same quantized weights it aggregates with (Prop. 1):
    with V constant per channel, O = Q*(c) for any Q and K.  Powers of two
    quantize to themselves, so the output must equal them bit for bit.  The
    logits are kept moderate so that no quantized weight falls into the
    binary32 subnormal range, where the matrix core may flush terms of O~ and
    of l differently."""
    for causal in (False, True):
        B, H, N, d = 2, 3, 700, 128
        x = W.custom(B, H, N, d, seed=9, scale=0.7)
        rng = np.random.default_rng(1)
        c = np.exp2(rng.integers(-6, 6, d)) * rng.choice([-1.0, 1.0], d)
        v = np.broadcast_to(W.to_bits(c, W.BF16), (B, H, N, d)).copy()
        say(f"constant V causal={causal}")
        out, stats = run_forward(to_device(x["q"], W.BF16), to_device(x["k"], W.BF16), to_device(v, W.BF16), causal)
        o = out.cpu().numpy()
        assert (o == c.astype(np.float32)[None, None, None, :]).all()


def test_zero_queries_average_the_values():
    """Q = 0: every score is 0, every P~ = 1 = P^, so O is the mean of V^ over
    the visible keys (computed here from the GPU's own V^ codes)."""
    B, H, N, d = 1, 2, 333, 128
    x = W.custom(B, H, N, d, seed=10)
    zq = np.zeros_like(x["q"])
    dv = to_device(x["v"], W.BF16)
    out, _ = run_forward(to_device(zq, W.BF16), to_device(x["k"], W.BF16), dv, False)
    vm = mx.rotate_quantize(dv, mx.AXIS_TOKEN, rotate=False)
    codes, scales = mx.unpack_tokens(vm)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    vals = grid[codes & 7] * np.where(codes & 8, -1.0, 1.0) * np.exp2(scales.astype(np.float64) - 127)[..., None]
    vhat = vals.transpose(0, 1, 2, 4, 3).reshape(B, H, -1, d)[:, :, :N]
    mean = vhat.mean(axis=2)
    o = out.cpu().numpy().astype(np.float64)
    say("zero queries")
    assert np.allclose(o, mean[:, :, None, :], rtol=1e-5, atol=1e-6)


TIE_MODES = [(mx.P_PNQ, mx.SCALE_UOS, True), (mx.P_PNQ, mx.SCALE_OCP, True), (mx.P_DIRECT, mx.SCALE_OCP, False),
             (mx.P_POSTNORM, mx.SCALE_OCP, True), (mx.P_POSTNORM, mx.SCALE_UOS, True)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("p_mode,rule,rotate", TIE_MODES, ids=["pnq-uos", "pnq-ocp", "direct-ocp", "postnorm-ocp",
                                                               "postnorm-uos"])
def test_tied_keys_match_oracle(p_mode, rule, rotate, causal):
    """Keys built from five distinct rows, repeated: every score value recurs
    about N/5 times, so many keys tie exactly at the running maximum (P~ = 1
    on each, S26) and POSTNORM's l* counts them (S32).  Outputs and row
    sums against the oracle on every row."""
    B, H, N, d = 1, 2, 300, 128
    x = W.custom(B, H, N, d, seed=13, scale=1.5)
    k = x["k"].copy()
    k[:, :, 5:] = np.concatenate([x["k"][:, :, :5]] * (N // 5 + 1), axis=2)[:, :, 5:N]
    dev = {t: to_device(a, W.BF16) for t, a in (("q", x["q"]), ("k", k), ("v", x["v"]))}
    label = f"tied keys mode {p_mode}/{rule}/{rotate} causal={causal}"
    say(label)
    sums = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    ref_out = mx.quantize_reference_modes(dev["q"], dev["k"], dev["v"], rule=rule, p_mode=p_mode, rotate=rotate,
                                          causal=causal, row_sums=sums)
    torch.cuda.synchronize()
    ref = oracle.attention(x["q"], k, x["v"], W.BF16, B, H, N, d, causal=causal, rotate=rotate, rule=rule,
                           p_mode=p_mode, kv_tile=KV_TILE, amb_delta=DELTA)
    check_output(ref_out.cpu().numpy(), ref, label, (N + KV_TILE - 1) // KV_TILE)
    check_row_sums(sums.cpu().numpy(), ref, label)
    if (p_mode, rule) == (mx.P_PNQ, mx.SCALE_UOS):  # the method itself: the same result through mxattn_forward
        out, _ = run_forward(dev["q"], dev["k"], dev["v"], causal)
        assert torch.equal(out.view(torch.int32), ref_out.view(torch.int32)), "forward and PNQ reference mode differ"


def test_single_key_and_first_causal_row_copy_v():
    B, H, d = 1, 2, 128
    for N, causal in ((1, False), (260, True)):
        x = W.custom(B, H, N, d, seed=11)
        dv = to_device(x["v"], W.BF16)
        out, _ = run_forward(to_device(x["q"], W.BF16), to_device(x["k"], W.BF16), dv, causal)
        vm = mx.rotate_quantize(dv, mx.AXIS_TOKEN, rotate=False)
        codes, scales = mx.unpack_tokens(vm)
        grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
        v0 = grid[codes[:, :, 0, :, 0] & 7] * np.where(codes[:, :, 0, :, 0] & 8, -1.0, 1.0) * \
            np.exp2(scales[:, :, 0].astype(np.float64) - 127)
        assert (out.cpu().numpy()[:, :, 0] == v0.astype(np.float32)).all()


def test_causal_leakage_on_gpu():
    """The MatX block analysis on the GPU path: perturbing V at token j leaves
    rows below its 32-token block bit-identical and changes rows of the block
    before j; perturbing K at j leaves every row i < j bit-identical."""
    B, H, N, d = 1, 2, 400, 128
    x = W.custom(B, H, N, d, seed=12)
    dq, dk = to_device(x["q"], W.BF16), to_device(x["k"], W.BF16)
    base, _ = run_forward(dq, dk, to_device(x["v"], W.BF16), True)
    for j in (45, 200, 399):
        v = x["v"].copy()
        v[:, :, j] = W.to_bits(W.from_bits(v[:, :, j], W.BF16).astype(np.float64) * 256.0, W.BF16)
        o, _ = run_forward(dq, dk, to_device(v, W.BF16), True)
        blk0 = 32 * (j // 32)
        assert torch.equal(o[:, :, :blk0], base[:, :, :blk0])
        assert (o[:, :, blk0:j] != base[:, :, blk0:j]).any(dim=-1).all()
        k = x["k"].copy()
        k[:, :, j] = W.to_bits(W.from_bits(k[:, :, j], W.BF16).astype(np.float64) * -5.0, W.BF16)
        o2, _ = run_forward(dq, to_device(k, W.BF16), to_device(x["v"], W.BF16), True)
        assert torch.equal(o2[:, :, :j], base[:, :, :j])
        say(f"causal leakage j={j}: rows < {blk0} identical, rows {blk0}..{j - 1} changed")


def _bench_forward(dq, dk, dv, causal):
    """The benchmark's launches: one Q, K, V quantizer launch, then the forward."""
    qm, km, vm = mx.rotate_quantize_qkv(dq, dk, dv, rotate=True)
    out = mx.forward(qm, km, vm, causal=causal)
    torch.cuda.synchronize()
    return out


# (b, h, j): j at 32-token block edges (first and last token of a block), inside
# blocks, at query-tile edges, and in both query tiles of a causal tile pair
# (a workgroup runs query tiles nqt-1-i, then i: tiles 63, 32 come first,
# tiles 0, 7, 10, 31 second)
LEAK_CASES = [(0, 0, 31), (0, 5, 32), (1, 17, 4095), (2, 9, 4141), (3, 31, 8191), (1, 3, 1361), (2, 20, 896),
              (3, 8, 8165)]


@pytest.mark.timeout(600)
def test_causal_leakage_at_the_causal_lm_shape():
    """The MatX block analysis ("Leaky quantization", when quantized V leaks
    the future) on the causal LM workload's own inputs, B4 H32 N8192, with the
    benchmark's launches.  V at token j scaled by 2^8 (a new block scale):
    rows below j's 32-token block are bit-identical, and every row from the
    block's start up to j whose output the oracle predicts to move does move
    on the GPU (the leak; those rows also match the oracle).  K at token j
    negated and scaled: every row before j is bit-identical.  Heads without a
    perturbation are bit-identical throughout."""
    w = W.WORKLOADS[4]
    B, H, N, d = w.shape
    say(f"causal leakage at full size: {w.describe()}")
    bits = {t: W.generate(w, t) for t in "qkv"}
    dq, dk, dv = (to_device(bits[t], w.dtype) for t in "qkv")
    base = _bench_forward(dq, dk, dv, True)
    touched = torch.zeros((B, H), dtype=torch.bool)
    for b, h, _ in LEAK_CASES:
        touched[b, h] = True
    same_heads = ~touched.cuda()

    v = bits["v"].copy()
    for b, h, j in LEAK_CASES:
        v[b, h, j] = W.to_bits(W.from_bits(v[b, h, j], w.dtype).astype(np.float64) * 256.0, w.dtype)
    out_v = _bench_forward(dq, dk, to_device(v, w.dtype), True)
    assert torch.equal(out_v[same_heads], base[same_heads])
    leaks = 0
    for b, h, j in LEAK_CASES:
        blk0 = 32 * (j // 32)
        assert torch.equal(out_v[b, h, :blk0], base[b, h, :blk0]), (b, h, j)
        rows = np.arange(blk0, j + 1, dtype=np.int32)
        head = {t: bits[t][b:b + 1, h:h + 1] for t in "qk"}
        ref0 = oracle.attention(head["q"], head["k"], bits["v"][b:b + 1, h:h + 1], w.dtype, 1, 1, N, d, causal=True,
                                kv_tile=KV_TILE, rows=rows, amb_delta=DELTA)
        ref1 = oracle.attention(head["q"], head["k"], v[b:b + 1, h:h + 1], w.dtype, 1, 1, N, d, causal=True,
                                kv_tile=KV_TILE, rows=rows, amb_delta=DELTA)
        moves = (np.abs(ref1["out"] - ref0["out"]).max(axis=-1) > 1e-5)[0, 0]
        gpu_rows = out_v[b, h, blk0:j + 1].cpu().numpy()
        moved = (gpu_rows != base[b, h, blk0:j + 1].cpu().numpy()).any(axis=-1)
        check_output(gpu_rows[None, None], ref1, f"leak V b{b} h{h} j{j}", (N + KV_TILE - 1) // KV_TILE)
        assert (moved | ~moves).all(), (b, h, j, np.nonzero(moves & ~moved))
        leaks += int((moves[:j - blk0] & moved[:j - blk0]).sum())
        say(f"  V at b{b} h{h} j{j}: rows < {blk0} identical; rows {blk0}..{j}: "
            f"{int(moves[:j - blk0].sum())} of {j - blk0} predicted to leak, {int(moved[:j - blk0].sum())} moved")

    assert leaks > 0, "no row before j leaked in any case"
    k = bits["k"].copy()
    for b, h, j in LEAK_CASES:
        k[b, h, j] = W.to_bits(W.from_bits(k[b, h, j], w.dtype).astype(np.float64) * -5.0, w.dtype)
    out_k = _bench_forward(dq, to_device(k, w.dtype), dv, True)
    assert torch.equal(out_k[same_heads], base[same_heads])
    for b, h, j in LEAK_CASES:
        assert torch.equal(out_k[b, h, :j], base[b, h, :j]), (b, h, j)
    say(f"  K perturbations: rows before j identical in all {len(LEAK_CASES)} cases")


def test_forward_is_deterministic():
    w = W.WORKLOADS[1]
    dev = {t: to_device(W.generate(w, t), w.dtype) for t in "qkv"}
    a, sa = run_forward(dev["q"], dev["k"], dev["v"], False)
    b, sb = run_forward(dev["q"], dev["k"], dev["v"], False)
    assert torch.equal(a, b) and torch.equal(sa, sb)


def test_side_stream_gives_the_same_result():
    """Work enqueued on a caller's non-default stream (default priority) gives
    the result of the current-stream path; the caller orders the streams with
    events."""
    say("forward on a side stream")
    w = W.WORKLOADS[1]
    dev = {t: to_device(W.generate(w, t), w.dtype) for t in "qkv"}
    ref, _ = run_forward(dev["q"], dev["k"], dev["v"], False)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        qm, km, vm = mx.rotate_quantize_qkv(dev["q"], dev["k"], dev["v"], rotate=True, stream=side)
        out = mx.forward(qm, km, vm, causal=False, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


def test_hip_graph_replays_match_eager():
    """The path allocates nothing and issues no memsets, so the quantizer and
    forward launches can be captured in a HIP graph.  Several replays, with
    eager work and synchronizations between them, each equal the eager
    result."""
    say("forward under HIP graph capture")
    w = W.WORKLOADS[1]
    dev = {t: to_device(W.generate(w, t), w.dtype) for t in "qkv"}
    B, H, N, d = w.shape
    outs = (mx.MXTensor.empty(B, H, N, d, mx.AXIS_HEAD_DIM), mx.MXTensor.empty(B, H, N, d, mx.AXIS_HEAD_DIM),
            mx.MXTensor.empty(B, H, N, d, mx.AXIS_TOKEN))
    out = torch.empty((B, H, N, d), dtype=torch.float32, device="cuda")
    stats = torch.empty((B, H, N, 2), dtype=torch.float32, device="cuda")

    def path():
        mx.rotate_quantize_qkv(dev["q"], dev["k"], dev["v"], rotate=True, out=outs)
        mx.forward(*outs, causal=False, out=out, row_stats=stats)

    path()
    torch.cuda.synchronize()
    ref, ref_stats = out.clone(), stats.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm up on a side stream before capture
        path()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        path()
    for rep in range(4):
        out.fill_(float("nan"))
        stats.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref) and torch.equal(stats, ref_stats), rep
        path()  # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("p_mode,rule,rotate", [
    (mx.P_DIRECT, mx.SCALE_OCP, False),
    (mx.P_DIRECT, mx.SCALE_UOS, True),
    (mx.P_POSTNORM, mx.SCALE_UOS, True),
    (mx.P_PNQ, mx.SCALE_OCP, True),
])
@pytest.mark.parametrize("d", [64, 128])
def test_reference_modes_causal_match_oracle(p_mode, rule, rotate, d):
    """Every placement under the causal mask (the path whose second-half PV
    products are deferred into the next tile), ragged N, against the oracle."""
    B, H, N = 2, 2, 300
    say(f"reference modes causal: d={d} p_mode={p_mode} rule={rule} rotate={rotate}")
    x = W.custom(B, H, N, d, seed=3 * N + d + p_mode, scale=2.0)
    dev = {t: to_device(x[t], W.BF16) for t in "qkv"}
    sums = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    out = mx.quantize_reference_modes(dev["q"], dev["k"], dev["v"], rule=rule, p_mode=p_mode, rotate=rotate,
                                      causal=True, row_sums=sums)
    torch.cuda.synchronize()
    ref = oracle.attention(x["q"], x["k"], x["v"], W.BF16, B, H, N, d, causal=True, rotate=rotate, rule=rule,
                           p_mode=p_mode, kv_tile=KV_TILE, amb_delta=DELTA)
    check_output(out.cpu().numpy(), ref, f"causal d={d} mode {p_mode}/{rule}/{rotate}", (N + KV_TILE - 1) // KV_TILE)
    rs = sums.cpu().numpy()
    if p_mode == mx.P_PNQ:
        assert np.abs(rs - 1).max() < 1e-5
    else:
        check_row_sums(rs, ref, f"causal d={d} mode {p_mode}/{rule}/{rotate}")
