"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test states the passage it checks.  None of them re-derives a value from
the oracle's own formula: the references are the pages' printed values and
closed forms, textbook identities, library routines (numpy, scipy) and brute
force over small inputs.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden_lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


def grid_from_golden():
    rows = {r[0]: [Fraction(x) for x in r[1:]] for r in golden_lines("e2m1_grid.txt")}
    return rows["grid"], rows["boundaries"]


# --------------------------------------------------------------------------
# E2M1 element format  [P1 Sec. 2 Eqs. 9-10; App. B Eqs. 67-68]


def test_grid_matches_page():
    grid, _ = grid_from_golden()
    assert [Fraction(oracle.e2m1_magnitude(c)) for c in range(8)] == grid
    for c in range(8):
        assert oracle.e2m1_value(c | 8) == -oracle.e2m1_magnitude(c)


def test_projection_is_nearest_grid_point_brute_force():
    """Every dyadic y on a 1/128 lattice in [0, 9] plus random y: the returned
    grid value is a nearest one (exact rational distances), ties go to the
    even code, and everything beyond the grid saturates at 6 [Eq. 10]."""
    grid, _ = grid_from_golden()
    rng = np.random.default_rng(7)
    ys = [Fraction(k, 128) for k in range(0, 9 * 128 + 1)]
    ys += [Fraction(float(y)) for y in rng.uniform(0, 12, 4000)]
    for y in ys:
        c = oracle.e2m1_project(float(y))
        dists = [abs(y - g) for g in grid]
        best = min(dists)
        assert dists[c] == best, (y, c)
        nearest = [i for i, dd in enumerate(dists) if dd == best]
        if len(nearest) == 2:
            assert c % 2 == 0, (y, c)


def test_decision_boundaries_and_ties_match_page():
    """The code changes exactly at the printed boundaries [Eq. 68] and the
    value at each boundary goes to the even code."""
    _, bounds = grid_from_golden()
    for k, t in enumerate(bounds):
        t = float(t)
        below = oracle.e2m1_project(math.nextafter(t, 0.0))
        above = oracle.e2m1_project(math.nextafter(t, 100.0))
        assert (below, above) == (k, k + 1)
        at = oracle.e2m1_project(t)
        assert at in (k, k + 1) and at % 2 == 0
    for y in (5.000001, 6.0, 7.0, 7.25, 8.0, 1e30):
        assert oracle.e2m1_project(y) == 7


def test_sign_and_zero_blocks():
    # all-zero block: sigma = 1 and every element 0 [P1 Sec. 2 end; Alg. 1]
    sb, codes, e = oracle.quantize_block(np.zeros(32))
    assert sb == 127 and e == 0 and not codes.any()
    # negative zero keeps its sign bit (reading of the pages' silence on signed zero)
    sb, codes, _ = oracle.quantize_block(np.full(32, -0.0))
    assert sb == 127 and (codes == 8).all()
    x = np.zeros(32)
    x[0], x[1], x[2] = 12.0, -0.001, -3.0  # e = ceil(log2(12/7.25)) = 1
    sb, codes, e = oracle.quantize_block(x)
    assert e == 1 and sb == 128 and codes[0] == 7 and codes[1] == 8 and codes[2] == 0x8 | 3


# --------------------------------------------------------------------------
# shared-scale rules  [P1 Sec. 2 Eqs. 11-13; Sec. 4.1 Eq. 19, Alg. 1; P2]


def test_uos_worked_examples():
    for M, e, scale, xnorm in golden_lines("uos_worked_examples.txt"):
        M, e, scale, xnorm = float(M), int(e), float(scale), float(xnorm)
        assert oracle.scale_exponent(M, oracle.RULE_UOS) == e
        assert 2.0 ** e == scale and M / scale == xnorm
        blk = np.zeros(32)
        blk[5] = M
        sb, codes, ee = oracle.quantize_block(blk)
        assert ee == e and sb == e + 127
        # dequantized block maximum: Q*(14.5) = 2 * Pi(7.25) = 12 (saturation at 6),
        # Q*(1) = (1/4) * 4 = 1 exactly [App. J Eq. 117]
        deq = oracle.e2m1_value(codes[5]) * scale
        assert deq == {14.5: 12.0, 1.0: 1.0}[M]


def _positive_bf16():
    bits = np.arange(1, 0x7F80, dtype=np.uint32)  # every positive finite bfloat16
    return (bits << 16).view(np.float32).astype(np.float64)


def test_normalized_max_ranges_exhaustive_bf16_and_random_fp32():
    """UOS maps the block maximum into (3.625, 7.25] [Alg. 1 range statement],
    OCP into [4, 8) [Eq. 11, Sec. 3], e_ceil(q) into (q/2, q] [Eq. 19],
    e_floor(q) into [q/2, q) [Eq. 12]."""
    rng = np.random.default_rng(11)
    rnd32 = (rng.integers(0x00800000, 0x7F800000, 200000, dtype=np.uint32)).view(np.float32)
    for M in (_positive_bf16(), rnd32.astype(np.float64)):
        eu = oracle.scale_exponents(M, oracle.RULE_UOS).astype(np.float64)
        eo = oracle.scale_exponents(M, oracle.RULE_OCP).astype(np.float64)
        xu, xo = M / np.exp2(eu), M / np.exp2(eo)
        assert ((xu > 3.625) & (xu <= 7.25)).all()
        assert ((xo >= 4.0) & (xo < 8.0)).all()
        # UOS differs from OCP by at most one binade, exactly when the OCP-normalized
        # maximum lies above 7.25 (difference of Eqs. 11 and 13 with q = 7.25)
        diff = eu - eo
        assert set(np.unique(diff)) <= {0.0, 1.0}
        assert ((diff == 1.0) == (xo > 7.25)).all()
        for q in (6.0, 7.0, 7.25, 8.0, 6.05):
            ec = oracle.scale_exponents(M, oracle.RULE_CEIL_Q, q).astype(np.float64)
            ef = oracle.scale_exponents(M, oracle.RULE_FLOOR_Q, q).astype(np.float64)
            xc, xf = M / np.exp2(ec), M / np.exp2(ef)
            assert ((xc > q / 2) & (xc <= q)).all()
            assert ((xf >= q / 2) & (xf < q)).all()
            # floor and ceiling forms differ only where M/q is a power of two [Sec. 2]
            ratio = M / q
            pow2 = (np.frexp(ratio)[0] == 0.5)
            assert ((ec != ef) == pow2).all()


def test_oas_equivalent_rule_relation():
    """App. G, Eq. 96: the q = 7 exponent is one below the q = 6 (TFS)
    exponent exactly for blocks whose TFS-normalized max lies in (3, 3.5]."""
    M = _positive_bf16()
    e6 = oracle.scale_exponents(M, oracle.RULE_CEIL_Q, 6.0)
    e7 = oracle.scale_exponents(M, oracle.RULE_CEIL_Q, 7.0)
    x6 = M / np.exp2(e6.astype(np.float64))
    expect = np.where((x6 > 3.0) & (x6 <= 3.5), e6 - 1, e6)
    assert (e7 == expect).all()


def test_e8m0_clamp():
    # M = 2^-126 would need e = -128 under UOS; the E8M0 byte clamps at 2^-127
    M = 2.0 ** -126
    assert oracle.scale_exponent(M, oracle.RULE_UOS) == -128
    blk = np.zeros(32)
    blk[0] = M
    sb, codes, e = oracle.quantize_block(blk)
    assert sb == 0 and e == -127 and codes[0] == 4  # 2^-126 / 2^-127 = 2 -> code 4


# --------------------------------------------------------------------------
# closed forms of the error analysis, from the *implemented* projection
# [P1 Sec. 4.1 Eqs. 21, 35-39; App. B Eqs. 69-73; App. C Eq. 81]


def implemented_pieces():
    """Piecewise-constant map of oracle.e2m1_project on [0, inf): boundaries
    located by bisection between lattice points where the code changes."""
    lattice = [k / 64.0 for k in range(0, 64 * 10 + 1)]
    codes = [oracle.e2m1_project(x) for x in lattice]
    cuts = []
    for a, b, ca, cb in zip(lattice, lattice[1:], codes, codes[1:]):
        if ca == cb:
            continue
        lo, hi = a, b
        while math.nextafter(lo, hi) < hi:
            mid = 0.5 * (lo + hi)
            if oracle.e2m1_project(mid) == ca:
                lo = mid
            else:
                hi = mid
        cuts.append((Fraction(hi).limit_denominator(1 << 20), ca, cb))
    pieces, start = [], Fraction(0)
    for t, ca, _ in cuts:
        pieces.append((start, t, Fraction(oracle.e2m1_magnitude(ca))))
        start = t
    pieces.append((start, Fraction(10 ** 9), Fraction(oracle.e2m1_magnitude(cuts[-1][2]))))
    return pieces


PIECES = None


def pieces():
    global PIECES
    if PIECES is None:
        PIECES = implemented_pieces()
    return PIECES


def E_exact(x):
    """E(x) = int_0^x (v - Pi(v))^2 dv, integrated exactly per piece [Eq. 69]."""
    x = Fraction(x)
    total = Fraction(0)
    for a, b, r in pieces():
        if a >= x:
            break
        bb = min(b, x)
        total += ((bb - r) ** 3 - (a - r) ** 3) / 3
    return total


def Delta(q):
    q = Fraction(q)
    return E_exact(q) - 8 * E_exact(q / 2)


def test_implemented_boundaries_are_the_printed_ones():
    _, bounds = grid_from_golden()
    assert [a for a, _, _ in pieces()[1:]] == bounds


def test_error_integral_closed_forms():
    rows = golden_lines("closed_forms.txt")
    for r in rows:
        if r[0] == "E":
            assert E_exact(Fraction(r[1])) == Fraction(r[2])
    # Eq. 70 for q >= 6 and E(29/4) = 7/8 + (5/4)^3/3 = 293/192
    assert E_exact(Fraction(29, 4)) == Fraction(293, 192)
    for q in (Fraction(6), Fraction(13, 2), Fraction(9), Fraction(25, 2)):
        assert E_exact(q) == Fraction(7, 8) + (q - 6) ** 3 / 3


def test_delta_pieces_root_and_sign():
    rows = {r[0]: r[1:] for r in golden_lines("closed_forms.txt")}
    for q in (Fraction(6), Fraction(25, 4), Fraction(13, 2), Fraction(27, 4), Fraction(7)):
        assert Delta(q) == Fraction(rows["delta_6_7"][0])
    for q in (Fraction(7), Fraction(57, 8), Fraction(29, 4), Fraction(15, 2), Fraction(31, 4), Fraction(8)):
        assert Delta(q) == (4 * q - 29) * (4 * q - 27) / 8
    root = Fraction(rows["root"][0])
    assert Delta(root) == 0
    # sign pattern of Eq. 81
    for q in (Fraction(1, 16), Fraction(1, 8), Fraction(1, 4)):
        assert Delta(q) == 0
    for q in (Fraction(1, 4) + Fraction(1, 1024), Fraction(1), Fraction(3), Fraction(29, 4) - Fraction(1, 1000)):
        assert Delta(q) < 0
    for q in (Fraction(29, 4) + Fraction(1, 1000), Fraction(8), Fraction(11), Fraction(100)):
        assert Delta(q) > 0


def test_delta_last_piece_discriminant():
    """For q >= 12 both E(q) and E(q/2) are on the saturated branch, and 8*Delta
    is a quadratic whose discriminant the page prints as -18240 [App. C]."""
    qs = [Fraction(12), Fraction(13), Fraction(14)]
    ys = [8 * Delta(q) for q in qs]
    # exact interpolation of a*q^2 + b*q + c through three points
    (q0, q1, q2), (y0, y1, y2) = qs, ys
    a = ((y2 - y1) / (q2 - q1) - (y1 - y0) / (q1 - q0)) / (q2 - q0)
    b = (y1 - y0) / (q1 - q0) - a * (q1 + q0)
    c = y0 - a * q0 ** 2 - b * q0
    assert 8 * Delta(Fraction(20)) == a * 400 + b * 20 + c
    disc = b * b - 4 * a * c
    assert a > 0 and disc == Fraction(golden_lines("closed_forms.txt")[-2][1])


def _D_vectorized(x):
    """D(x) = E(x)/x^3 evaluated in binary64 from the implemented pieces."""
    E = np.zeros_like(x)
    for a, b, r in pieces():
        a, b, r = float(a), float(b), float(r)
        lo = np.minimum(np.maximum(x, a), b)
        E += ((lo - r) ** 3 - (a - r) ** 3) / 3.0 * (x > a)
    return E / x ** 3


def _law_nodes(law, n=400000):
    """Midpoint-rule nodes and weights for log2(M) under `law` (deterministic)."""
    if law == "uniform01":
        u = (np.arange(n) + 0.5) / n
        return u, np.full(n, 1.0 / n)
    if law == "mixture":
        u1, w1 = _law_nodes(("normal", 0.3, 0.2), n // 2)
        u2, w2 = _law_nodes(("normal", 2.7, 0.5), n // 2)
        return np.concatenate([u1, u2]), np.concatenate([w1, w2]) * 0.5
    _, mu, sd = law
    u = mu + sd * (-8 + 16 * (np.arange(n) + 0.5) / n)
    w = np.exp(-0.5 * ((u - mu) / sd) ** 2)
    return u, w / w.sum()


@pytest.mark.parametrize("law", ["uniform01", ("normal", 0.0, 0.1), ("normal", 3.0, 2.0), "mixture"])
def test_uos_objective_minimized_at_7_25(law):
    """Theorem 1 / Fig. 2: J(q) = E[D(X_q)] over the implemented ceiling rule and
    projection has its minimum at q = 7.25 on the paper's 6.00..8.00 sweep grid
    (step 0.05, Sec. 5.5.1), whatever the law of log2 M."""
    u, w = _law_nodes(law)
    M = np.exp2(u)
    qs = np.round(np.arange(6.0, 8.0001, 0.05), 2)
    J = []
    for q in qs:
        e = oracle.scale_exponents(M, oracle.RULE_CEIL_Q, q).astype(np.float64)
        J.append(float(np.sum(w * _D_vectorized(M / np.exp2(e)))))
    assert qs[int(np.argmin(J))] == 7.25


def test_ocp_overflow_region_probability():
    """Eq. 15: under a log-uniform block maximum, Pr(x_max >= 7) = log2(8/7)
    for the OCP rule (the page's printed 19.27 % rounds the exact 0.192645)."""
    n = 2_000_000
    u = (np.arange(n) + 0.5) / n * 7.0 - 3.0  # seven whole binades
    M = np.exp2(u)
    e = oracle.scale_exponents(M, oracle.RULE_OCP).astype(np.float64)
    p = float(np.mean(M / np.exp2(e) >= 7.0))
    assert abs(p - math.log2(8 / 7)) < 2e-6
    assert round(math.log2(8 / 7) * 100, 2) == 19.26


# --------------------------------------------------------------------------
# element decode and Hadamard rotation  [P1 Sec. 4.3, Alg. 2; P2]


def test_decode_half_exhaustive():
    bits = np.arange(0, 1 << 16, dtype=np.uint16)
    ref16 = bits.view(np.float16).astype(np.float32)
    ref_bf = (bits.astype(np.uint32) << 16).view(np.float32)
    got16 = np.array([oracle.decode_half(int(b), oracle.FP16) for b in bits], np.float32)
    gotbf = np.array([oracle.decode_half(int(b), oracle.BF16) for b in bits], np.float32)
    for got, ref in ((got16, ref16), (gotbf, ref_bf)):
        nan = np.isnan(ref)
        assert (np.isnan(got) == nan).all()
        assert (got[~nan].view(np.uint32) == ref[~nan].view(np.uint32)).all()


@pytest.mark.parametrize("d", [32, 64, 128, 256])
def test_rotation_is_scaled_sylvester_hadamard(d):
    H = scipy.linalg.hadamard(d).astype(np.float64)  # Sylvester construction
    r = np.float32(1.0 / math.sqrt(d))
    R = np.stack([oracle.hadamard_rotate_f32(np.eye(d, dtype=np.float32)[i]) for i in range(d)])
    # e_i maps exactly to row i of H times fl32(1/sqrt d)
    assert (R == (H * np.float64(r)).astype(np.float32)).all()
    # orthogonality up to the rounding of fl32(1/sqrt d)
    G = R.astype(np.float64) @ R.T.astype(np.float64)
    assert np.allclose(G, np.eye(d) * d * float(r) ** 2, rtol=0, atol=1e-13)
    assert abs(d * float(r) ** 2 - 1) < 2 ** -22
    if d == 128:
        assert int(np.array(r).view(np.uint32)) == 0x3DB504F3
    if d == 64:
        assert int(np.array(r).view(np.uint32)) == 0x3E000000
    # the all-ones row concentrates on channel 0: sqrt(d) e_0
    ones = oracle.hadamard_rotate_f32(np.ones(d, np.float32))
    assert ones[0] == np.float32(d) * r and not ones[1:].any()


def test_rotation_error_bound_norms_and_dot_products():
    """Against x H / sqrt(d) in binary64 (scipy): each of log2(d) add stages and
    the final multiply contributes at most 2^-24 relative, so the error is
    bounded by (log2 d + 1) 2^-24 ||x||_1 / sqrt(d) (plus the same for the
    binary64 reference).  Norms and dot products are preserved [P2 glossary]."""
    rng = np.random.default_rng(3)
    for d in (64, 128):
        H = scipy.linalg.hadamard(d) / math.sqrt(d)
        for _ in range(200):
            x = (rng.standard_normal(d) * np.exp(rng.standard_normal(d))).astype(np.float32)
            y = oracle.hadamard_rotate_f32(x).astype(np.float64)
            ref = x.astype(np.float64) @ H
            bound = (math.log2(d) + 2) * 2 ** -24 * np.abs(x).astype(np.float64).sum() / math.sqrt(d)
            assert np.abs(y - ref).max() <= bound
            assert abs(np.linalg.norm(ref) - np.linalg.norm(x.astype(np.float64))) < 1e-12 * np.linalg.norm(x)
        q = rng.standard_normal(d)
        k = rng.standard_normal(d)
        assert abs((q @ H) @ (k @ H) - q @ k) < 1e-12 * (np.linalg.norm(q) * np.linalg.norm(k))


def test_outlier_is_spread_over_every_channel():
    """P2 'Rotate Q and K': a single outlier of magnitude A becomes magnitude
    A/sqrt(d) on every channel."""
    for d in (64, 128):
        x = np.zeros(d, np.float32)
        x[37] = 1000.0
        y = oracle.hadamard_rotate_f32(x)
        assert np.allclose(np.abs(y), 1000.0 / math.sqrt(d), rtol=2 ** -22)


# --------------------------------------------------------------------------
# tensor quantizers: axes and the block structure  [P3 Quantizing attention]


def test_token_blocks_only_see_their_own_tokens():
    """V is blocked along tokens (32 per block, aligned to token 0): changing
    token j changes the codes/scales of block floor(j/32) only [P3]."""
    N, d = 200, 64
    x = W.custom(1, 1, N, d, seed=5, tensors=("v",))["v"]
    c0, s0 = oracle.quantize_token_blocks(x, oracle.BF16, 1, 1, N, d)
    for j in (0, 31, 32, 100, 199):
        y = x.copy()
        y[0, 0, j, :] = W.to_bits(np.full(d, 300.0), W.BF16)
        c1, s1 = oracle.quantize_token_blocks(y, oracle.BF16, 1, 1, N, d)
        changed = sorted(set(np.nonzero((c0 != c1).any(axis=(1, 2)) | (s0 != s1).any(axis=1))[0]))
        assert changed == [j // 32]


def test_row_quantizer_wiring_and_tail_block():
    """Wiring only: rows assemble decode -> rotate -> 32-blocks along d; a
    partial last token block is padded with +0."""
    B, H, N, d = 2, 3, 45, 64
    x = W.custom(B, H, N, d, dtype=W.FP16, seed=9, tensors=("q",))["q"]
    codes, scales = oracle.quantize_rows(x, oracle.FP16, B, H, N, d, rotate=True)
    g = (1 * H + 2) * N + 17
    row = np.array([oracle.decode_half(int(b), oracle.FP16) for b in x[1, 2, 17]], np.float32)
    row = oracle.hadamard_rotate_f32(row)
    for k in range(d // 32):
        sb, cc, _ = oracle.quantize_block(row[32 * k:32 * k + 32].astype(np.float64))
        assert sb == scales[g, k] and (cc == codes[g, 32 * k:32 * k + 32]).all()
    c, s = oracle.quantize_token_blocks(x, oracle.FP16, B, H, N, d)
    NB = (N + 31) // 32
    last = (0 * H + 0) * NB + NB - 1
    # tokens 45..63 of the last block are padding: codes +0 (no sign bit)
    assert (c[last][:, N - 32 * (NB - 1):] == 0).all()


# --------------------------------------------------------------------------
# attention forward  [P1 Alg. 2; Eqs. 1-8, 42, 44-52; App. H-J; P3]


def dequant_rows(codes, scales):
    grid = np.array([oracle.e2m1_magnitude(c) for c in range(8)])
    v = grid[codes & 7] * np.where(codes & 8, -1.0, 1.0)
    return v * np.exp2(np.repeat(scales.astype(np.float64) - 127, 32, axis=-1))


def quantized_head(x_q, x_k, x_v, dtype, N, d, rotate=True, rule=oracle.RULE_UOS):
    """q^, k^, v^ of a single head [N, d] in binary64 via the oracle's quantizers."""
    cq, sq = oracle.quantize_rows(x_q, dtype, 1, 1, N, d, rotate=rotate, rule=rule)
    ck, sk = oracle.quantize_rows(x_k, dtype, 1, 1, N, d, rotate=rotate, rule=rule)
    cv, sv = oracle.quantize_token_blocks(x_v, dtype, 1, 1, N, d, rule=rule)
    qh, kh = dequant_rows(cq, sq), dequant_rows(ck, sk)
    grid = np.array([oracle.e2m1_magnitude(c) for c in range(8)])
    vv = grid[cv & 7] * np.where(cv & 8, -1.0, 1.0) * np.exp2(sv.astype(np.float64) - 127)[..., None]
    vh = vv.transpose(0, 2, 1).reshape(-1, d)[:N]
    return qh, kh, vh


def exact_attention(q, k, v, causal):
    s = q @ k.T / math.sqrt(q.shape[1])
    if causal:
        s = np.where(np.tril(np.ones_like(s, dtype=bool)), s, -np.inf)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    return (p / p.sum(axis=1, keepdims=True)) @ v


@pytest.mark.parametrize("N", [1, 7, 100, 300])
@pytest.mark.parametrize("causal", [False, True])
def test_online_softmax_recurrence_equals_softmax_attention(N, causal):
    """With quantization off, the tiled recurrence of Eqs. 2-8 equals the plain
    softmax attention of Eq. 1 for every tile width [Sec. 2]."""
    d = 64
    x = W.custom(1, 2, N, d, seed=N, scale=2.0)
    ref = [exact_attention(*(W.from_bits(x[t][0, h], W.BF16).astype(np.float64) for t in "qkv"), causal)
           for h in range(2)]
    for Bc in (32, 64, 128, 256):
        r = oracle.attention(x["q"], x["k"], x["v"], W.BF16, 1, 2, N, d, causal=causal,
                             rotate=False, quant=False, kv_tile=Bc)
        for h in range(2):
            assert np.allclose(r["out"][0, h], ref[h], rtol=1e-12, atol=1e-12)
        assert np.allclose(r["rowsum"], 1.0, atol=1e-12)


def test_pnq_rows_sum_to_one_and_l_at_least_one():
    """Prop. 1 (Eq. 51) via the effective full-row form of Lemma 2 (Eqs. 99-105),
    and App. J (Eq. 118): l >= 1 for every row."""
    for w in (W.WORKLOADS[1],):
        q, k, v = (W.generate(w, t) for t in "qkv")
        r = oracle.attention(q, k, v, w.dtype, w.B, w.H, w.N, w.d)
        assert np.abs(r["rowsum"] - 1.0).max() < 1e-12
        assert (r["l"] >= 1.0).all()
    x = W.custom(2, 2, 333, 64, seed=4, scale=3.0)
    for causal in (False, True):
        r = oracle.attention(x["q"], x["k"], x["v"], W.BF16, 2, 2, 333, 64, causal=causal)
        assert np.abs(r["rowsum"] - 1.0).max() < 1e-12
        assert (r["l"] >= 1.0).all()


def test_direct_placement_normalizer_and_row_sums():
    """Direct placement (Eq. 42): l telescopes to the unquantized softmax
    normalizer sum_j exp(s_j - m) (Eq. 108, computed here from scratch with
    numpy), and the induced row sums (Eq. 110) are not 1 in general (Eq. 18)."""
    N, d = 300, 128
    x = W.custom(1, 1, N, d, seed=21, scale=1.5)
    r = oracle.attention(x["q"], x["k"], x["v"], W.BF16, 1, 1, N, d, p_mode=oracle.P_DIRECT)
    qh, kh, _ = quantized_head(x["q"], x["k"], x["v"], W.BF16, N, d)
    s = qh @ kh.T / math.sqrt(d)
    m = s.max(axis=1)
    assert np.allclose(r["m"][0, 0], m, rtol=1e-14, atol=0)
    assert np.allclose(r["l"][0, 0], np.exp(s - m[:, None]).sum(axis=1), rtol=1e-12)
    rs = r["rowsum"][0, 0]
    assert np.abs(rs - 1).max() > 1e-3
    p = oracle.attention(x["q"], x["k"], x["v"], W.BF16, 1, 1, N, d, p_mode=oracle.P_PNQ)
    assert np.abs(p["rowsum"] - 1).max() < 1e-12


def test_closed_form_outputs():
    """Derived from Alg. 2 and App. J:
    (i) a single visible key gives O = v^_0 exactly;
    (ii) Q = 0 makes every score equal, every P~ = 1 = P^, so O = mean_j v^_j;
    (iii) V constant per channel gives, under PNQ, O = Q*(c) for any Q and K;
          the direct placement gives rowsum * Q*(c) instead."""
    d = 128
    x = W.custom(1, 1, 1, d, seed=2)
    r = oracle.attention(x["q"], x["k"], x["v"], W.BF16, 1, 1, 1, d)
    _, _, vh = quantized_head(x["q"], x["k"], x["v"], W.BF16, 1, d)
    assert (r["out"][0, 0, 0] == vh[0]).all()
    N = 200
    x = W.custom(1, 1, N, d, seed=3)
    rc = oracle.attention(x["q"], x["k"], x["v"], W.BF16, 1, 1, N, d, causal=True, rows=[0])
    _, _, vh = quantized_head(x["q"], x["k"], x["v"], W.BF16, N, d)
    assert (rc["out"][0, 0, 0] == vh[0]).all()
    zq = np.zeros_like(x["q"])
    r0 = oracle.attention(zq, x["k"], x["v"], W.BF16, 1, 1, N, d)
    assert np.allclose(r0["out"][0, 0], vh.mean(axis=0)[None, :], rtol=1e-13, atol=1e-13)
    c = np.linspace(-5, 5, d)
    cv = np.broadcast_to(W.to_bits(c, W.BF16), (1, 1, N, d)).copy()
    xs = W.custom(1, 1, N, d, seed=8, scale=3.0)
    rp = oracle.attention(xs["q"], xs["k"], cv, W.BF16, 1, 1, N, d)
    _, _, vc = quantized_head(xs["q"], xs["k"], cv, W.BF16, N, d)
    assert (vc == vc[0]).all()
    assert np.allclose(rp["out"][0, 0], vc[0][None, :], rtol=1e-13, atol=1e-13)
    rd = oracle.attention(xs["q"], xs["k"], cv, W.BF16, 1, 1, N, d, p_mode=oracle.P_DIRECT)
    assert np.allclose(rd["out"][0, 0], rd["rowsum"][0, 0][:, None] * vc[0][None, :], rtol=1e-12,
                       atol=1e-12)


def test_causal_leakage_block_analysis():
    """P3: with V blocked along tokens, perturbing V at j leaves rows i below
    its block bit-identical, changes rows inside the block with i < j (the
    leak), and perturbing K or Q at j leaves every row i < j bit-identical."""
    N, d = 160, 128
    x = W.custom(1, 1, N, d, seed=13)
    base = oracle.attention(x["q"], x["k"], x["v"], W.BF16, 1, 1, N, d, causal=True)["out"][0, 0]
    for j in (45, 100):
        y = x["v"].copy()
        y[0, 0, j] = W.to_bits(W.from_bits(y[0, 0, j], W.BF16).astype(np.float64) * 256.0, W.BF16)
        o = oracle.attention(x["q"], x["k"], y, W.BF16, 1, 1, N, d, causal=True)["out"][0, 0]
        blk0 = 32 * (j // 32)
        assert (o[:blk0] == base[:blk0]).all()
        assert (o[blk0:j] != base[blk0:j]).any(axis=1).all()
        for t in ("k", "q"):
            z = {kk: vv.copy() for kk, vv in x.items()}
            z[t][0, 0, j] = W.to_bits(W.from_bits(z[t][0, 0, j], W.BF16).astype(np.float64) * -7.0, W.BF16)
            o = oracle.attention(z["q"], z["k"], z["v"], W.BF16, 1, 1, N, d, causal=True)["out"][0, 0]
            assert (o[:j] == base[:j]).all()


def test_result_depends_on_tile_width_but_stays_normalized():
    N, d = 256, 64
    x = W.custom(1, 1, N, d, seed=17, scale=2.5)
    outs = []
    for Bc in (32, 64, 128):
        r = oracle.attention(x["q"], x["k"], x["v"], W.BF16, 1, 1, N, d, kv_tile=Bc)
        assert np.abs(r["rowsum"] - 1).max() < 1e-12
        outs.append(r["out"])
    assert np.abs(outs[0] - outs[1]).max() > 0 and np.abs(outs[1] - outs[2]).max() > 0


def brute_force_pnq(qh, kh, vh, Bc, causal, rule=oracle.RULE_UOS, direct=False):
    """Independent small re-statement of Alg. 2: materialize S, walk the tiles,
    quantize each aligned 32-key block of exp(S - m_new) with the (separately
    pinned) block quantizer.  qh has Nq rows, kh and vh Nk rows."""
    Nq, d = qh.shape
    N = kh.shape[0]
    S = qh @ kh.T / math.sqrt(d)
    out = np.zeros((Nq, d))
    for i in range(Nq):
        m, l, o = -np.inf, 0.0, np.zeros(d)
        for j0 in range(0, N, Bc):
            vis = [j for j in range(j0, min(j0 + Bc, N)) if (not causal or j <= i)]
            if not vis:
                continue
            mn = max(m, max(S[i, j] for j in vis))
            a = 0.0 if m == -np.inf else math.exp(m - mn)
            pt = np.zeros(Bc)
            for j in vis:
                pt[j - j0] = math.exp(S[i, j] - mn)
            ph = np.zeros(Bc)
            for b0 in range(0, Bc, 32):
                sb, codes, _ = oracle.quantize_block(pt[b0:b0 + 32], rule)
                ph[b0:b0 + 32] = [oracle.e2m1_value(c) * 2.0 ** (sb - 127) for c in codes]
            l = a * l + (pt.sum() if direct else ph.sum())
            o = a * o + sum(ph[j - j0] * vh[j] for j in vis)
            m = mn
        out[i] = o / l
    return out


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,Bc", [(1, 32), (37, 32), (70, 64), (64, 128)])
def test_brute_force_tiny(N, Bc, causal):
    d = 32
    x = W.custom(1, 1, N, d, seed=N + Bc, scale=2.0)
    qh, kh, vh = quantized_head(x["q"], x["k"], x["v"], W.BF16, N, d)
    for direct in (False, True):
        ref = brute_force_pnq(qh, kh, vh, Bc, causal, direct=direct)
        r = oracle.attention(x["q"], x["k"], x["v"], W.BF16, 1, 1, N, d, causal=causal, kv_tile=Bc,
                             p_mode=oracle.P_DIRECT if direct else oracle.P_PNQ)
        assert np.allclose(r["out"][0, 0], ref, rtol=1e-12, atol=1e-12)


def test_postnorm_mode_definition():
    """Materialized-P diagnostic (Sec. 5.5.2): O = Q(P) V^ with P the exact
    softmax and no renormalization; with V constant per channel O equals
    (sum_j Q(P)_ij) * Q*(c), and the row sums differ from 1."""
    N, d = 250, 64
    xs = W.custom(1, 1, N, d, seed=31, scale=2.0)
    c = np.linspace(-3, 3, d)
    cv = np.broadcast_to(W.to_bits(c, W.BF16), (1, 1, N, d)).copy()
    r = oracle.attention(xs["q"], xs["k"], cv, W.BF16, 1, 1, N, d, p_mode=oracle.P_POSTNORM)
    _, _, vc = quantized_head(xs["q"], xs["k"], cv, W.BF16, N, d)
    assert np.allclose(r["out"][0, 0], r["rowsum"][0, 0][:, None] * vc[0][None, :], rtol=1e-12, atol=1e-13)
    assert np.abs(r["rowsum"] - 1).max() > 1e-3
    qh, kh, _ = quantized_head(xs["q"], xs["k"], cv, W.BF16, N, d)
    s = qh @ kh.T / math.sqrt(d)
    assert np.allclose(r["l"][0, 0], np.exp(s - s.max(axis=1, keepdims=True)).sum(axis=1), rtol=1e-12)


def test_decision_allowance_is_nonnegative_and_off_by_default():
    w = W.WORKLOADS[1]
    q, k, v = (W.generate(w, t) for t in "qkv")
    r0 = oracle.attention(q, k, v, w.dtype, w.B, w.H, w.N, w.d)
    assert (r0["amb"] == 0).all()
    r1 = oracle.attention(q, k, v, w.dtype, w.B, w.H, w.N, w.d, amb_delta=1e-3)
    assert (r1["amb"] >= 0).all() and r1["amb"].max() > 0
    assert (r1["out"] == r0["out"]).all()


# ---- the decision allowance (binary32 evaluations of P~ against the
# binary64 oracle; the margin delta stands for their rounding)

MIDPOINTS = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)  # E2M1 decision boundaries [P1 Eq. 68]
RANGE = {oracle.RULE_UOS: (3.625, 7.25), oracle.RULE_OCP: (4.0, 8.0)}  # normalized block max (lo, hi]


def _far_from_every_threshold(p, rule, e, delta):
    """True when every normalized element p/2^e lies farther than delta
    (relative) from every rounding midpoint and the normalized block maximum
    farther than delta from both ends of the rule's range -- computed here
    from the printed grid and the range of the rule."""
    y = np.ldexp(p, -e)
    for mid in MIDPOINTS:
        if (np.abs(y - mid) <= delta * mid).any():
            return False
    lo, hi = RANGE[rule]
    r = y.max()
    return r > 0 and abs(r - lo) > delta * lo and abs(r - hi) > delta * hi


@pytest.mark.parametrize("rule", [oracle.RULE_UOS, oracle.RULE_OCP])
def test_allowance_is_zero_far_from_every_threshold(rule):
    """A block whose every decision lies farther than delta from its
    threshold has no allowance; one whose decision lies within delta/2 of its
    threshold has an allowance of at least the step that decision can take."""
    rng = np.random.default_rng(5)
    delta = 2.0 ** -8
    far = near = 0
    for _ in range(3000):
        p = np.exp(rng.normal(0.0, 2.0, 32)) * 2.0 ** rng.integers(-20, 20)
        ph, dp, e = oracle.p_block_allowance(p, rule, delta=delta)
        if _far_from_every_threshold(p, rule, e, delta):
            far += 1
            assert (dp == 0).all()
        # plant one element within delta/2 of a midpoint at this exponent
        t = int(rng.integers(0, 32))
        c = int(rng.integers(0, 7))
        q = p.copy()
        q[t] = np.ldexp(MIDPOINTS[c] * (1 + rng.uniform(-0.5, 0.5) * delta), e)
        if q.max() != p.max() or q[t] >= p.max():
            continue
        _, dq, eq = oracle.p_block_allowance(q, rule, delta=delta)
        if eq == e:
            near += 1
            grid = (0, 0.5, 1, 1.5, 2, 3, 4, 6)
            assert dq[t] >= np.ldexp(grid[c + 1] - grid[c], e)
    assert far > 100 and near > 1000


def test_allowance_closed_form_blocks():
    """Hand-computed blocks.  UOS [P1 Alg. 1]: max 6 gives e = 0; an element at
    the midpoint 2.5 may round to 2 or 3 (allowance 1).  A max at exactly the
    boundary 7.25 (e = 0, saturating to 6) may take e = 1, where it rounds to
    8: allowance 2.  Moving it up by 2 delta gives e = 1 with 3.625 (1 + 2
    delta), clear of the boundary; by delta/2, still within it."""
    delta = 2.0 ** -13
    p = np.zeros(32)
    p[0], p[5] = 6.0, 2.5
    ph, dp, e = oracle.p_block_allowance(p, oracle.RULE_UOS, delta=delta)
    assert e == 0 and ph[0] == 6 and ph[5] == 2 and dp[5] == 1 and (np.delete(dp, 5) == 0).all()
    p = np.zeros(32)
    p[3] = 7.25
    ph, dp, e = oracle.p_block_allowance(p, oracle.RULE_UOS, delta=delta)
    assert e == 0 and ph[3] == 6 and dp[3] == 2 and (np.delete(dp, 3) == 0).all()
    p[3] = 7.25 * (1 + 2 * delta)
    ph, dp, e = oracle.p_block_allowance(p, oracle.RULE_UOS, delta=delta)
    assert e == 1 and (dp == 0).all()
    p[3] = 7.25 * (1 + delta / 2)
    ph, dp, e = oracle.p_block_allowance(p, oracle.RULE_UOS, delta=delta)
    assert e == 1 and dp[3] > 0


def test_allowance_exempts_exact_one_only():
    """OCP puts 1 on a scale boundary (floor(log2 1) - 2 = -2, normalized max
    4 = lo).  P~ = exp(0) = 1 at the row maximum is exact on any hardware, so
    with exact_ref = 1 that boundary offers no alternative; without it the
    alternative e = -3 (1 saturates to 6/8) is allowed.  The same holds for
    P = 1/l* < 1 next to the boundary from below.  Other boundaries are not
    exempt."""
    delta = 2.0 ** -13
    p = np.zeros(32)
    p[7], p[9] = 1.0, 0.01
    ph, dp, e = oracle.p_block_allowance(p, oracle.RULE_OCP, delta=delta)
    assert e == -2 and ph[7] == 1 and dp[7] == 0.25
    ph, dp, e = oracle.p_block_allowance(p, oracle.RULE_OCP, delta=delta, exact_ref=1.0)
    assert e == -2 and (dp == 0).all()
    p[7] = 1.0 / (1.0 + 1e-9)  # post-normalization P at the row maximum
    ph, dp, e = oracle.p_block_allowance(p, oracle.RULE_OCP, delta=delta)
    assert e == -3 and ph[7] == 0.75 and dp[7] == 0.25
    ph, dp, e = oracle.p_block_allowance(p, oracle.RULE_OCP, delta=delta, exact_ref=1.0)
    assert e == -3 and (dp == 0).all()
    p[7] = 0.5 * (1 + delta / 4)  # next to the boundary 1/2: not exempt
    ph, dp, e = oracle.p_block_allowance(p, oracle.RULE_OCP, delta=delta, exact_ref=1.0)
    assert e == -3 and dp[7] > 0


def _one_hot_inputs(N, d, gap, tie=False, seed=0):
    """Q = 1 on channel 0 plus small noise elsewhere; K noise on the other
    channels, 0 on channel 0, except key 5 (in the first tile) with a large
    channel-0 entry: its score exceeds the rest by about `gap`.  `tie` gives
    key 45 the same channel-0 entry, an exact tie of the maximum."""
    rng = np.random.default_rng(seed)
    q = 0.3 * rng.standard_normal((1, 1, N, d))
    q[..., 0] = 1.0
    k = 0.3 * rng.standard_normal((1, 1, N, d))
    k[..., 0] = 0.0
    j0 = 5
    k[0, 0, j0, 0] = gap * math.sqrt(d)
    if tie:
        k[0, 0, j0 + 40] = k[0, 0, j0]
    v = rng.standard_normal((1, 1, N, d))
    return (W.to_bits(q, W.BF16), W.to_bits(k, W.BF16), W.to_bits(v, W.BF16))


@pytest.mark.parametrize("p_mode", [oracle.P_DIRECT, oracle.P_PNQ])
def test_one_hot_row_has_no_allowance_under_ocp(p_mode):
    """A row with one dominant key: P~ = 1 there, every other P~ below
    e^-20, far under the first midpoint at any exponent the block can take.
    Under OCP (unrotated, the vanilla baseline) nothing is a close decision:
    amb = 0.  A second key tying the maximum makes the row's maximum
    uncertain (binary32 scores may break the tie either way), and the
    allowance appears."""
    N, d, delta = 96, 32, 2.0 ** -13
    q, k, v = _one_hot_inputs(N, d, gap=24.0)
    r = oracle.attention(q, k, v, W.BF16, 1, 1, N, d, rotate=False, rule=oracle.RULE_OCP, p_mode=p_mode,
                         kv_tile=32, amb_delta=delta)
    assert (r["amb"] == 0).all()
    q, k, v = _one_hot_inputs(N, d, gap=24.0, tie=True)
    r = oracle.attention(q, k, v, W.BF16, 1, 1, N, d, rotate=False, rule=oracle.RULE_OCP, p_mode=p_mode,
                         kv_tile=32, amb_delta=delta)
    assert r["amb"].max() > 0


def test_postnorm_one_hot_row_allowance_follows_rho():
    """Post-normalization under OCP: at the row maximum P = 1/l* with
    l* = 1 + rho.  For rho > 0 it lies just below 1, so e = -3 and it
    saturates to 6/8 = 0.75 [P1 Sec. 5.5.2, Eq. 10].  While rho is large
    enough for binary32 to see (gap 24: rho ~ e^-22 N after K's OCP
    quantization; gap 60: rho ~ e^-68 N ~ 2^-91, below binary64's 2^-53
    next to 1, so 1/l* must not round up to the boundary 1), that is an
    exact decision: amb = 0.  With rho below 2^-100 (gap 200: rho ~ e^-181 N)
    the decision is left open."""
    N, d, delta = 96, 32, 2.0 ** -13
    for gap, open_ in ((24.0, False), (60.0, False), (200.0, True)):
        q, k, v = _one_hot_inputs(N, d, gap=gap)
        r = oracle.attention(q, k, v, W.BF16, 1, 1, N, d, rotate=False, rule=oracle.RULE_OCP,
                             p_mode=oracle.P_POSTNORM, kv_tile=32, amb_delta=delta)
        assert abs(r["rowsum"][0, 0].max() - 0.75) < 1e-6 or open_
        assert (r["amb"].max() > 0) == open_


def _forced_attention(qh, kh, vh, Bc, causal, rule, p_mode, delta, force, rows, rowsums=None):
    """Alg. 2 (PNQ / DIRECT) or the post-normalization mode re-stated over
    dequantized q^, k^, v^ for the listed rows (and, into `rowsums` if given,
    each row's induced row sum: sum Q(P) for post-normalization, Eq. 110's
    (sum beta P^ 1) / (sum beta P~ 1) for DIRECT, (sum beta P^ 1) / l for
    PNQ), with one hook:
    force(i, j0, p, ph, exact_ref) returns the quantized block used for row i,
    keys j0..j0+31 (ph is the plain block quantization of p).  exact_ref is 1
    for a block holding the row maximum's element when that maximum stands
    alone (runner-up below (1 - delta) of it; for post-normalization also
    2^-100 <= l* - 1 < 1), else 0."""
    Nq, d = qh.shape
    N = kh.shape[0]
    S = qh @ kh.T / math.sqrt(d)
    out = {}
    for i in rows:
        vis = np.arange(N) <= i if causal else np.ones(N, bool)
        if p_mode == oracle.P_POSTNORM:
            s = np.where(vis, S[i], -np.inf)
            jm = int(np.argmax(s))
            srt = np.sort(s[vis])
            e = np.exp(s - s[jm])
            rho = e.sum() - 1.0 if e.sum() - 1.0 > 1e-3 else np.delete(e, jm).sum()
            alone = len(srt) < 2 or math.exp(srt[-2] - srt[-1]) < 1 - delta
            exact = alone and 2.0 ** -100 <= rho < 1
            P = e / e.sum()
            o, rs = np.zeros(d), 0.0
            for b0 in range(0, N, 32):
                pb = np.zeros(32)
                pb[:min(32, N - b0)] = P[b0:b0 + 32]
                ref = 1.0 if exact and b0 <= jm < b0 + 32 else 0.0
                ph = force(i, b0, pb, oracle.p_block_allowance(pb, rule)[0], ref)
                o += ph[:min(32, N - b0)] @ vh[b0:b0 + 32]
                rs += ph[:min(32, N - b0)].sum()
            out[i] = o
            if rowsums is not None:
                rowsums[i] = rs
            continue
        m, l, o = -np.inf, 0.0, np.zeros(d)
        num = den = 0.0
        seen = []
        for j0 in range(0, N, Bc):
            idx = [j for j in range(j0, min(j0 + Bc, N)) if vis[j]]
            if not idx:
                continue
            seen.extend(S[i, idx])
            srt = np.sort(seen)
            mn = max(m, S[i, idx].max())
            alone = len(srt) < 2 or math.exp(srt[-2] - srt[-1]) < 1 - delta
            a = 0.0 if m == -np.inf else math.exp(m - mn)
            pt = np.zeros(Bc)
            pt[np.array(idx) - j0] = np.exp(S[i, idx] - mn)
            ph = np.zeros(Bc)
            for b0 in range(0, Bc, 32):
                pb = pt[b0:b0 + 32]
                ref = 1.0 if alone and (pb == 1.0).any() else 0.0
                ph[b0:b0 + 32] = force(i, j0 + b0, pb, oracle.p_block_allowance(pb, rule)[0], ref)
            l = a * l + (pt.sum() if p_mode == oracle.P_DIRECT else ph.sum())
            num, den = a * num + ph.sum(), a * den + pt.sum()
            o = a * o + ph[np.array(idx) - j0] @ vh[idx]
            m = mn
        out[i] = o / l
        if rowsums is not None:
            rowsums[i] = num / den if p_mode == oracle.P_DIRECT else num / l
    return out


def _alternatives(p, ph, dp, rule):
    """Every single decision of a block flipped: an element with dp > 0 moved
    to its other grid neighbour, or the whole block re-projected at e +- 1
    when that stays within dp (a flagged scale alternative)."""
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    alts = []
    e = oracle.p_block_allowance(p, rule)[2]
    for t in np.nonzero(dp > 0)[0]:
        y = math.ldexp(p[t], -e)
        below = grid[grid <= y].max()
        above = grid[grid >= y].min() if y <= 6 else 6.0
        for g in (below, above):
            val = math.ldexp(g, e)
            if val != ph[t] and abs(val - ph[t]) <= dp[t]:
                a = ph.copy()
                a[t] = val
                alts.append(a)
    for ea in (e - 1, e + 1):
        a = np.array([math.ldexp(grid[oracle.e2m1_project(math.ldexp(x, -ea))], ea) for x in p])
        if (a != ph).any() and (np.abs(a - ph) <= dp).all():
            alts.append(a)
    return alts


@pytest.mark.parametrize("p_mode", [oracle.P_PNQ, oracle.P_DIRECT, oracle.P_POSTNORM])
@pytest.mark.parametrize("rule", [oracle.RULE_UOS, oracle.RULE_OCP])
def test_allowance_bounds_every_flagged_decision_forced(p_mode, rule):
    """amb bounds how far O_i moves when decisions within the margin go the
    other way.  With a wide margin (many flagged decisions), each flagged
    decision is forced the other way, one at a time, in an independent
    re-statement of the forward: the output row moves by at most amb, channel
    by channel.  The re-statement without forcing equals the oracle."""
    N, d, Bc, delta = 80, 32, 32, 0.05
    x = W.custom(1, 1, N, d, seed=50 + rule + 3 * p_mode, scale=2.0)
    qh, kh, vh = quantized_head(x["q"], x["k"], x["v"], W.BF16, N, d, rotate=False, rule=rule)
    r = oracle.attention(x["q"], x["k"], x["v"], W.BF16, 1, 1, N, d, causal=True, rotate=False, rule=rule,
                         p_mode=p_mode, kv_tile=Bc, amb_delta=delta)
    rows = list(range(N))
    base_rs = {}
    base = _forced_attention(qh, kh, vh, Bc, True, rule, p_mode, delta, lambda i, j0, p, ph, ref: ph, rows,
                             rowsums=base_rs)
    for i in rows:
        assert np.allclose(base[i], r["out"][0, 0, i], rtol=1e-12, atol=1e-12)
        assert abs(base_rs[i] - r["rowsum"][0, 0, i]) <= 1e-12
    amb = r["amb"][0, 0]
    amb_rs = r["amb_rowsum"][0, 0]
    if p_mode == oracle.P_PNQ:
        assert (amb_rs == 0).all()  # PNQ's row sum is 1 whatever the decisions
    flips = 0
    for i in rows:
        blocks = []

        def record(ii, j0, p, ph, ref):
            blocks.append((j0, p.copy(), ph.copy(), ref))
            return ph

        _forced_attention(qh, kh, vh, Bc, True, rule, p_mode, delta, record, [i])
        for j0, p, ph, ref in blocks:
            _, dp, _ = oracle.p_block_allowance(p, rule, delta=delta, exact_ref=ref)
            for alt in _alternatives(p, ph, dp, rule):
                def swap(ii, jj, pp, hh, rr, alt=alt, j0=j0):
                    return alt if jj == j0 else hh
                frs = {}
                forced = _forced_attention(qh, kh, vh, Bc, True, rule, p_mode, delta, swap, [i], rowsums=frs)[i]
                moved = np.abs(forced - base[i])
                assert (moved <= amb[i] * (1 + 1e-9) + 1e-15).all(), (i, j0)
                assert abs(frs[i] - base_rs[i]) <= amb_rs[i] * (1 + 1e-9) + 1e-15, (i, j0, "row sum")
                flips += 1
    assert flips > 20


def test_absmass_equals_output_for_nonnegative_values():
    """absmass is the output with |V^| in place of V^: for V >= 0 they coincide."""
    N, d = 150, 64
    x = W.custom(1, 1, N, d, seed=41, scale=2.0)
    vpos = W.to_bits(np.abs(W.from_bits(x["v"], W.BF16).astype(np.float64)), W.BF16)
    for mode in (oracle.P_PNQ, oracle.P_DIRECT, oracle.P_POSTNORM):
        r = oracle.attention(x["q"], x["k"], vpos, W.BF16, 1, 1, N, d, p_mode=mode)
        assert np.allclose(r["absmass"], r["out"], rtol=1e-14, atol=0)
        r2 = oracle.attention(x["q"], x["k"], x["v"], W.BF16, 1, 1, N, d, p_mode=mode)
        assert (r2["absmass"] >= np.abs(r2["out"]) * (1 - 1e-14)).all()


# --------------------------------------------------------------------------
# cross-attention: Nq query rows against Nk key/value tokens [P1 Sec. 5.1,
# Wan2.2's separate cross-attention; Alg. 2 with the key loop over Nk tokens]


def cross_inputs(Nq, Nk, d, seed, scale=2.0):
    xq = W.custom(1, 2, Nq, d, seed=seed, scale=scale)
    xkv = W.custom(1, 2, Nk, d, seed=seed + 1000, scale=scale)
    return xq["q"], xkv["k"], xkv["v"]


@pytest.mark.parametrize("Nq,Nk", [(1, 300), (100, 7), (257, 33), (40, 129)])
def test_cross_attention_unquantized_is_softmax_attention(Nq, Nk):
    """Quantization off: the tiled recurrence over Nk keys equals the plain
    softmax attention of Eq. 1 with a rectangular score matrix."""
    d = 64
    q, k, v = cross_inputs(Nq, Nk, d, seed=Nq * 7 + Nk)
    for Bc in (32, 128):
        r = oracle.attention(q, k, v, W.BF16, 1, 2, Nq, d, rotate=False, quant=False, kv_tile=Bc, Nk=Nk)
        for h in range(2):
            ref = exact_attention(*(W.from_bits(x[0, h], W.BF16).astype(np.float64) for x in (q, k, v)), False)
            assert np.allclose(r["out"][0, h], ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("Nq,Nk,Bc", [(5, 70, 32), (37, 9, 32), (20, 130, 64)])
def test_cross_attention_brute_force_tiny(Nq, Nk, Bc):
    d = 32
    xq = W.custom(1, 1, Nq, d, seed=Nq + Bc, scale=2.0)
    xkv = W.custom(1, 1, Nk, d, seed=Nk + Bc + 500, scale=2.0)
    cq, sq = oracle.quantize_rows(xq["q"], W.BF16, 1, 1, Nq, d, rotate=True)
    qh = dequant_rows(cq, sq)
    _, kh, vh = quantized_head(xkv["q"], xkv["k"], xkv["v"], W.BF16, Nk, d)
    for direct in (False, True):
        ref = brute_force_pnq(qh, kh, vh, Bc, False, direct=direct)
        r = oracle.attention(xq["q"], xkv["k"], xkv["v"], W.BF16, 1, 1, Nq, d, kv_tile=Bc, Nk=Nk,
                             p_mode=oracle.P_DIRECT if direct else oracle.P_PNQ)
        assert np.allclose(r["out"][0, 0], ref, rtol=1e-12, atol=1e-12)
        r1 = oracle.attention(xq["q"], xkv["k"], xkv["v"], W.BF16, 1, 1, Nq, d, kv_tile=Bc, Nk=Nk)
        assert np.abs(r1["rowsum"] - 1).max() < 1e-12


def test_cross_rows_equal_rows_of_a_self_attention_problem():
    """Each query row is independent: embedding the Nq queries among Nk rows
    of a self-attention problem over the same K, V gives the same rows."""
    Nq, Nk, d = 19, 150, 64
    q, k, v = cross_inputs(Nq, Nk, d, seed=3)
    qbig = W.custom(1, 2, Nk, d, seed=9, scale=2.0)["q"].copy()
    pos = np.arange(Nq) * 7 + 3
    qbig[:, :, pos] = q
    cross = oracle.attention(q, k, v, W.BF16, 1, 2, Nq, d, Nk=Nk)
    selfr = oracle.attention(qbig, k, v, W.BF16, 1, 2, Nk, d, rows=pos)
    for key in ("out", "m", "l", "rowsum"):
        assert np.array_equal(cross[key], selfr[key])


def test_cross_attention_argument_checks():
    q, k, v = cross_inputs(8, 16, 32, seed=1)
    with pytest.raises(ValueError):
        oracle.attention(q, k, v, W.BF16, 1, 2, 8, 32, Nk=16, causal=True)


# --------------------------------------------------------------------------
# Q_max sweep  [P1 Sec. 5.5.1, Table 4; Eq. 13; App. G]


def test_sweep_closed_form_block_at_the_uos_boundary():
    """Every value of a block equal to 7.25 * 2^-3 = 0.90625 (exact in bf16):
    for q >= 7.25 the scale is 2^-3 (a tie M = q 2^e keeps the smaller e) and
    7.25 saturates to 6, an error of 1.25 * 2^-3 per element; for q < 7.25 the
    scale doubles and 3.625 rounds up to 4, an error of 0.75 * 2^-3."""
    B, H, N, d = 1, 2, 32, 64
    x = np.full((B, H, N, d), W.to_bits(np.array(0.90625), W.BF16), np.uint16)
    qs = [6.0, 7.0, 7.2, 7.25, 7.3, 8.0]
    per_block_hi = 32 * (1.25 / 8) ** 2
    per_block_lo = 32 * (0.75 / 8) ** 2
    for axis, nblocks in ((oracle.AXIS_TOKEN, d * (N // 32)), (oracle.AXIS_HEAD_DIM, N * d // 32)):
        sse = oracle.scale_sweep(x, W.BF16, B, H, N, d, qs, axis=axis)
        want = [nblocks * (per_block_hi if q >= 7.25 else per_block_lo) for q in qs]
        assert np.array_equal(sse, np.array([want, want]))


def test_sweep_equals_sum_of_squares_of_the_quantizers_errors():
    """Wiring check against the two block quantizers: the sweep's per-head sum
    equals sum (x - x^)^2 computed here from the oracle's own codes and scales
    and the separately pinned rotation, for both axes and a ragged tail."""
    B, H, N, d = 1, 2, 45, 64
    x = W.custom(B, H, N, d, seed=31, scale=3.0)["q"]
    qs = [6.0, 6.55, 7.25, 8.0]
    grid = np.array([oracle.e2m1_magnitude(c) for c in range(8)])
    # head-dim axis with rotation
    sse = oracle.scale_sweep(x, W.BF16, B, H, N, d, qs, rotate=True)
    xs = W.from_bits(x, W.BF16).reshape(-1, d).copy()
    for r in range(xs.shape[0]):
        xs[r] = oracle.hadamard_rotate_f32(xs[r])
    for j, q in enumerate(qs):
        c, s = oracle.quantize_rows(x, W.BF16, B, H, N, d, rotate=True, rule=oracle.RULE_CEIL_Q, q=q)
        xh = grid[c & 7] * np.where(c & 8, -1.0, 1.0) * np.exp2(np.repeat(s.astype(np.float64) - 127, 32, axis=-1))
        err = ((xs.astype(np.float64) - xh) ** 2).reshape(B * H, -1).sum(axis=1)
        assert np.allclose(sse[:, j], err, rtol=1e-13, atol=0)
    # token axis, tail tokens past N count as +0
    sse = oracle.scale_sweep(x, W.BF16, B, H, N, d, qs, axis=oracle.AXIS_TOKEN)
    NB = (N + 31) // 32
    xv = np.zeros((B * H, NB * 32, d))
    xv[:, :N] = W.from_bits(x, W.BF16).reshape(B * H, N, d)
    for j, q in enumerate(qs):
        c, s = oracle.quantize_token_blocks(x, W.BF16, B, H, N, d, rule=oracle.RULE_CEIL_Q, q=q)
        xh = grid[c & 7] * np.where(c & 8, -1.0, 1.0) * np.exp2(s.astype(np.float64) - 127)[..., None]
        xh = xh.reshape(B * H, NB, d, 32).transpose(0, 1, 3, 2).reshape(B * H, NB * 32, d)
        err = ((xv - xh) ** 2).sum(axis=(1, 2))
        assert np.allclose(sse[:, j], err, rtol=1e-13, atol=0)


def test_sweep_head_selection_and_arguments():
    B, H, N, d = 2, 3, 40, 32
    x = W.custom(B, H, N, d, seed=32)["k"]
    full = oracle.scale_sweep(x, W.BF16, B, H, N, d, [6.0, 7.25], rotate=True)
    some = oracle.scale_sweep(x, W.BF16, B, H, N, d, [6.0, 7.25], rotate=True, heads=[5, 0])
    assert np.array_equal(some, full[[5, 0]])
    for bad in (dict(qs=[0.0]), dict(qs=[float("inf")]), dict(qs=[7.0], axis=oracle.AXIS_TOKEN, rotate=True),
                dict(qs=[7.0], heads=[6])):
        qs = bad.pop("qs")
        with pytest.raises(ValueError):
            oracle.scale_sweep(x, W.BF16, B, H, N, d, qs, **bad)


# --------------------------------------------------------------------------
# materialized-P row-sum diagnostics  [P1 Sec. 5.5.2, Fig. 7]


def test_diagnostics_uniform_row_closed_form():
    """Q = 0 makes every score 0, so P = 1/N on every row.  For N = 100 the UOS
    block scale is 2^ceil(log2(0.01/7.25)) = 2^-9, 0.01 * 2^9 = 5.12 rounds up
    to 6, and every element becomes 6/512: row sum 1.171875, all of it upward
    rounding, entropy ln 100.  A pre-quantization scale gamma = 1.25 moves the
    normalized value to 6.4, beyond the grid: every element saturates to 6,
    P^ = 6/512/1.25 and the row sum is 0.9375.  OCP picks the same scale here."""
    B, H, N, d = 1, 1, 100, 64
    x = W.custom(B, H, N, d, seed=40)
    zq = np.zeros_like(x["q"])
    for rule in (oracle.RULE_UOS, oracle.RULE_OCP):
        diag, _ = oracle.p_diagnostics(zq, x["k"], W.BF16, B, H, N, d, rule=rule)
        assert np.allclose(diag[..., 0], 1.171875, rtol=0, atol=1e-12)
        assert np.allclose(diag[..., 4], 0.171875, rtol=0, atol=1e-12)
        assert np.all(diag[..., 1:4] == 0)
        assert np.allclose(diag[..., 5], math.log(100), rtol=0, atol=1e-12)
    diag, _ = oracle.p_diagnostics(zq, x["k"], W.BF16, B, H, N, d, gamma=1.25)
    assert np.allclose(diag[..., 0], 0.9375, rtol=0, atol=1e-12)
    assert np.allclose(diag[..., 2], -0.0625, rtol=0, atol=1e-12)
    assert np.all(diag[..., [1, 3, 4]] == 0)
    # causal: row i sees i + 1 equal keys; row 0 holds P = 1, which UOS maps to
    # the grid value 4 at scale 1/4 exactly
    diag, _ = oracle.p_diagnostics(zq, x["k"], W.BF16, B, H, N, d, causal=True)
    assert diag[0, 0, 0, 0] == 1.0 and diag[0, 0, 0, 5] == 0.0
    assert np.allclose(diag[0, 0, 99], [1.171875, 0, 0, 0, 0.171875, math.log(100)], rtol=0, atol=1e-12)


@pytest.mark.parametrize("cid", [1, 5])
def test_diagnostics_decomposition_and_postnorm_row_sums(cid):
    """The four outcome classes partition the elements, so their contributions
    add up to the row-sum error; the row sum equals the POSTNORM forward's
    induced row sum; a power-of-two gamma changes nothing (the E8M0 scale
    absorbs it)."""
    w = W.WORKLOADS[cid]
    B, H, N, d = w.shape
    heads = [(0, 0), (0, 1)]
    sel = {t: W.generate(w, t, heads=heads)[None] for t in "qkv"}
    rows = np.arange(0, N, max(1, N // 97), dtype=np.int32)
    diag, _ = oracle.p_diagnostics(sel["q"], sel["k"], w.dtype, 1, 2, N, d, rows=rows)
    parts = diag[..., 1:5].sum(axis=-1)
    assert np.abs(diag[..., 0] - 1 - parts).max() < 1e-12
    assert (diag[..., 1] <= 0).all() and (diag[..., 2] <= 0).all() and (diag[..., 3] <= 0).all()
    assert (diag[..., 4] >= 0).all()
    assert (diag[..., 5] >= 0).all() and (diag[..., 5] <= math.log(N) + 1e-9).all()
    ref = oracle.attention(sel["q"], sel["k"], sel["v"], w.dtype, 1, 2, N, d, p_mode=oracle.P_POSTNORM, rows=rows)
    assert np.abs(diag[..., 0] - ref["rowsum"]).max() < 1e-12
    d4, _ = oracle.p_diagnostics(sel["q"], sel["k"], w.dtype, 1, 2, N, d, rows=rows, gamma=4.0)
    assert np.abs(d4[..., :5] - diag[..., :5]).max() < 1e-15
    # the sharp workload zeroes many elements; the outlier one saturates some
    if cid == 5:
        assert diag[..., 1].min() < -1e-3


def test_scale_exponent_outside_its_precondition_returns_zero():
    """M > 0 finite (and q > 0 finite for the boundary rules) is the
    precondition; outside it the exponent search would not terminate, so the
    oracle returns 0 instead.  Inside it nothing changes (the worked examples
    above still hold)."""
    for M in (0.0, -0.0, -1.0, float("inf"), float("nan")):
        for rule in (oracle.RULE_UOS, oracle.RULE_OCP):
            assert oracle.scale_exponent(M, rule) == 0
    assert oracle.scale_exponent(1.0, oracle.RULE_CEIL_Q, 0.0) == 0
    assert oracle.scale_exponent(1.0, oracle.RULE_CEIL_Q, float("inf")) == 0
    assert oracle.scale_exponent(14.5, oracle.RULE_UOS) == 1 and oracle.scale_exponent(1.0, oracle.RULE_UOS) == -2
