#!/usr/bin/env python3
"""Benchmark of MXAttention's MXFP4 attention forward on one MI355X.

One step is the whole hot path on the Wan-like video self-attention shape
(B=1, H=40, N=32760, d=128, bf16 inputs already in HBM):
  rotate + UOS-quantize Q, rotate + UOS-quantize K, UOS-quantize V along
  tokens (one mxattn_rotate_quantize_qkv launch), fused forward (scaled-FP4
  QK^T, online softmax with PNQ, scaled-FP4 PV).

Prints one JSON line.  `value` is whole-step throughput in TFLOPS, counting
4*B*H*N^2*d algorithmic flops (2*d per (query, key) pair for QK^T and as many
for PV).  `roofline` describes the dominant kernel (the fused forward) against
the dense MXFP4 matrix-core peak; its duration comes from HIP events recorded
around each forward launch on the launch stream.  `cpu_baseline` times the
plain CPU oracle on a bounded sample of the same workload.  `accuracy` gives
the error of the output against fp32 softmax attention on the unquantized
inputs (PyTorch on the GPU, sampled rows, outside the timed region).

After the timed steps, in-run probes (libmxprobe.so) measure what this GPU
reaches at its current clock and power state: dense scaled-FP4 matrix
products, the forward's vector work per (query, key) pair (one FMA, one
v_exp_f32, half an FP4 convert, half a max3, at two waves per SIMD) and a
16-byte copy's read+write bandwidth.  `roofline_valu` prices the forward
against the vector-mix probe; `forward` and `quantizer` also give their
fractions against the matrix and copy probes.

With --separate-quantize the three tensors are quantized by three
mxattn_rotate_quantize launches, and the JSON line adds per-launch rates for K
and V.  With --fused-q the step quantizes K and V (two launches) and runs the
forward entry point that rotates and quantizes Q in its own prologue (no Q^
buffer).  With --part sweep or --part diagnostics the line times another part
of the library on the same inputs instead: the Q_max sweep of Q, K and V over
41 boundaries (priced against HBM), or the materialized-P diagnostics call
(priced against the MXFP4 matrix peak).

    python bench.py [--steps K] [--warmup W] [--workload 2] [--separate-quantize] [--fused-q]
                    [--no-cpu-baseline] [--no-probes] [--part step|sweep|diagnostics]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_FP4_PEAK_TFLOPS = 10100.0  # MI355X dense MXFP4 matrix-core peak
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E peak
QUANT_BYTES_PER_ELEMENT = 2.0 + 0.5 + 1.0 / 32.0  # bf16 in, E2M1 codes + E8M0 scales out
QUANT_B2B_LAUNCHES = 10          # back-to-back quantizer launches timed after the steps
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attention_wan_like_traffic.txt")
KERNEL_SOURCE = os.path.join(ROOT, "mxfp4_microscaled_bit_amd", "csrc", "attention.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(launch_bytes_algorithmic: float):
    """HBM bytes per forward launch from the committed rocprofv3 counter
    summary, or None if there is none or the kernel changed since."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    with open(TRAFFIC_FILE) as f:
        for ln in f:
            if ":" in ln and not ln.startswith("#"):
                k, v = ln.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256") != kernel_source_hash():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, target_s: float = 15.0):
    """The CPU oracle on a bounded sample of the workload: query rows of a few
    heads, each row against all N keys, sized to about target_s seconds (the
    per-head quantization inside each call is part of the measured work)."""
    import numpy as np
    import oracle
    import workloads as W

    nth = oracle.default_threads()
    max_heads = min(4, w.B * w.H)
    heads = [(i // w.H, (i * max(1, w.H // max_heads)) % w.H) for i in range(max_heads)]
    sel = {t: W.generate(w, t, heads=heads)[None] for t in "qkv"}

    def run(n_heads, n_rows):
        rows = np.linspace(0, w.N - 1, n_rows).astype(np.int32)
        sub = {t: sel[t][:, :n_heads] for t in "qkv"}
        t0 = time.perf_counter()
        oracle.attention(sub["q"], sub["k"], sub["v"], w.dtype, 1, n_heads, w.N, w.d,
                         causal=w.causal, kv_tile=128, rows=rows, nthreads=nth)
        return time.perf_counter() - t0

    # grow the sample (rows per head up to N, then heads) until one run takes
    # a quarter of target_s; the final run scales that one to target_s, where
    # the per-head quantization is a small part of the time
    n_heads, n_rows = 2, 2 * nth
    t = run(n_heads, n_rows)
    while t < target_s / 4 and (n_rows < w.N or n_heads < max_heads):
        if n_rows < w.N:
            n_rows = min(w.N, 4 * n_rows)
        else:
            n_heads = min(max_heads, 2 * n_heads)
        t = run(n_heads, n_rows)
    want = n_heads * n_rows * target_s / max(t, 1e-3)  # (head, row) pairs for target_s
    n_heads = int(min(max_heads, max(n_heads, -(-want // w.N))))
    n_rows = int(min(w.N, max(1, want // n_heads)))
    t = run(n_heads, n_rows)
    pairs = n_heads * n_rows * w.N  # non-causal: every row sees every key
    flops = 4.0 * w.d * pairs
    return {
        "value": flops / t / 1e12,
        "unit": "TFLOPS",
        "cores": nth,
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "seconds": round(t, 3),
        "sample": (f"{n_heads} heads x {n_rows} query rows x all {w.N} keys of {w.name} "
                   f"({w.describe()}), including the oracle's own quantization of those heads; "
                   f"flops counted as 4*d per (query, key) pair"),
    }


def accuracy_vs_fp32(w, dev, out, n_rows: int = 256):
    """Error of the MXFP4 output against plain fp32 softmax attention computed
    by PyTorch on the GPU from the same unquantized 16-bit inputs, on n_rows
    evenly spaced query rows of two heads (outside the timed region)."""
    import torch

    B, H, N, d = w.shape
    heads = [(0, 0), (B - 1, H // 2)]
    rows = torch.linspace(0, N - 1, n_rows, device="cuda").round().long()
    num = den = 0.0
    max_abs = 0.0
    cos = []
    for b, h in heads:
        q = dev["q"][b, h].index_select(0, rows).float()
        k = dev["k"][b, h].float()
        v = dev["v"][b, h].float()
        s = torch.matmul(q, k.t().contiguous()) / float(d) ** 0.5
        if w.causal:
            keys = torch.arange(k.shape[0], device="cuda")
            s = s.masked_fill(keys[None, :] > rows[:, None], float("-inf"))
        ref = torch.matmul(torch.softmax(s, dim=-1), v)
        got = out[b, h].index_select(0, rows)
        diff = (got - ref).abs()
        cos.append(torch.nn.functional.cosine_similarity(got, ref, dim=-1))
        max_abs = max(max_abs, float(diff.max()))
        num += float(diff.sum())
        den += float(ref.abs().sum())
    return {"reference": "fp32 softmax attention (PyTorch) on the unquantized inputs",
            "sample": f"{n_rows} query rows x {len(heads)} heads",
            "mean_row_cosine": round(float(torch.cat(cos).mean()), 6), "max_abs": round(max_abs, 6),
            "mean_rel": round(num / den, 6)}


SWEEP_Q = [6.0 + 0.05 * i for i in range(41)]  # the Q_max grid 6.00, 6.05, ..., 8.00


ENTROPY_EDGES = (1.0, 2.0, 3.0, 4.0, 5.0)  # nats


def diagnostics_report(diag) -> dict:
    """The materialized-P row-sum statistics of MXAttention Sec. 5.5.2 (Fig. 7)
    from per-row diagnostics [..., 6] (row sum, zeroing, saturation, down, up,
    entropy in nats): the mean row sum (A), its mean decomposition by
    outcome (B), and row sums binned by entropy (D), each bin with its share
    of rows, mean row sum and share of over-normalized rows (sum > 1)."""
    import numpy as np

    d = np.asarray(diag, dtype=np.float64).reshape(-1, 6)
    rs, ent = d[:, 0], d[:, 5]
    rep = {"rows": int(d.shape[0]), "mean_row_sum": float(rs.mean()),
           "mean_zeroing": float(d[:, 1].mean()), "mean_saturation": float(d[:, 2].mean()),
           "mean_down": float(d[:, 3].mean()), "mean_up": float(d[:, 4].mean()),
           "over_normalized_rows": float((rs > 1.0).mean()), "under_normalized_rows": float((rs < 1.0).mean())}
    edges = (-np.inf,) + ENTROPY_EDGES + (np.inf,)
    bins = []
    for lo, hi in zip(edges[:-1], edges[1:]):
        m = (ent >= lo) & (ent < hi)
        label = f"<{hi:g}" if lo == -np.inf else (f">={lo:g}" if hi == np.inf else f"{lo:g}-{hi:g}")
        bins.append({"entropy_nats": label, "share": float(m.mean()),
                     "mean_row_sum": float(rs[m].mean()) if m.any() else None,
                     "over_normalized": float((rs[m] > 1.0).mean()) if m.any() else None})
    rep["entropy_bins"] = bins
    return rep


def sweep_report(sse, qs) -> dict:
    """Q_max optima of one tensor (MXAttention Sec. 5.5.1, Table 4) from its
    per-head squared errors [heads, len(qs)]: the tensor's objective J(q)
    (the sum over heads) with its argmin, and how often each q is a head's
    argmin.  Ties go to the smallest q."""
    import numpy as np

    e = np.asarray(sse, dtype=np.float64)
    J = e.sum(axis=0)
    heads = np.argmin(e, axis=1)
    counts = {f"{qs[j]:.2f}": int(c) for j, c in zip(*np.unique(heads, return_counts=True))}
    j = int(np.argmin(J))
    return {"tensor_optimum_q": round(float(qs[j]), 2), "J_at_optimum_over_J_at_7.25":
            float(J[j] / J[int(np.argmin(np.abs(np.asarray(qs) - 7.25)))]), "head_optimum_counts": counts}


def measure_part(args, w, dev, stream):
    """Time one of the other parts on the workload's inputs, resident in HBM:
    `sweep` -- mxattn_scale_sweep of Q and K (head-dim blocks, rotated) and V
    (token blocks) over SWEEP_Q, three launches per step, priced against HBM
    (2 bytes read per element; the per-head sums are negligible);
    `diagnostics` -- mxattn_p_diagnostics of (Q, K) with the UOS rule, the
    statistics pass and the diagnostics pass (plus its own quantization of Q
    and K), priced against the MXFP4 matrix peak with the score products of
    both passes, 2 x 2d flops per visible pair (the forward's 4d)."""
    import torch
    import mxfp4_microscaled_bit_amd as mx

    B, H, N, d = w.shape
    Nk = w.kv_tokens
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    if args.part == "sweep":
        outs = {t: torch.empty((B * H, len(SWEEP_Q)), dtype=torch.float64, device="cuda") for t in "qkv"}
        ws = {t: torch.empty(max(1, mx.scale_sweep_workspace_bytes(B, H, dev[t].shape[2], d,
                                                                   mx.AXIS_TOKEN if t == "v" else mx.AXIS_HEAD_DIM,
                                                                   len(SWEEP_Q))), dtype=torch.uint8, device="cuda")
              for t in "qkv"}

        def run():
            for t in "qkv":
                axis = mx.AXIS_TOKEN if t == "v" else mx.AXIS_HEAD_DIM
                mx.scale_sweep(dev[t], SWEEP_Q, axis=axis, rotate=(t != "v"), out=outs[t], workspace=ws[t])
        elements = B * H * (N + 2 * Nk) * d
        work, unit, peak, bound = elements * 2.0, "GB/s", HBM_PEAK_GBS, "hbm"
        metric = "Q_max sweep of Q, K, V (per-head squared error, 41 boundaries; MXAttention Sec. 5.5.1)"
    else:
        out = torch.empty((B, H, N, 6), dtype=torch.float32, device="cuda")
        ws = torch.empty(max(1, mx.p_diagnostics_workspace_bytes(B, H, N, d)), dtype=torch.uint8, device="cuda")
        if Nk != N:
            raise SystemExit("--part diagnostics needs self-attention (Nk = N)")

        def run():
            mx.p_diagnostics(dev["q"], dev["k"], rule=mx.SCALE_UOS, rotate=True, causal=w.causal, out=out,
                             workspace=ws)
        work, unit, peak, bound = w.flops(), "TFLOP/s", MFMA_FP4_PEAK_TFLOPS, "mfma"
        metric = "materialized-P diagnostics (statistics + diagnostics passes; MXAttention Sec. 5.5.2)"
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    e0, e1 = ev(), ev()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / args.steps
    rate = work / (ms * 1e-3) / (1e9 if unit == "GB/s" else 1e12)
    report = None
    if args.part == "sweep":
        report = {t: sweep_report(outs[t].cpu().numpy(), SWEEP_Q) for t in "qkv"}
    if args.part == "diagnostics":
        # Fig. 7 of the pages, after the timed calls, under the path's UOS rule and the vanilla OCP rule (the
        # pages do not say which rule their diagnostic uses): statistics at gamma = 1, then the
        # pre-quantization global-scaling baseline (C).  A power of two in gamma cancels, so its fraction
        # gamma_f in [1, 2) is scanned for the mean row sum closest to 1.
        # Two readings of the baseline: the kernel returns Q(gamma P) / gamma (the factor taken out again,
        # so it only moves rounding decisions); with the factor kept, Q(gamma P) = gamma (Q(gamma P) / gamma)
        # and its row sums are gamma times the kernel's, so gamma near 1 / mean sets the mean to 1.
        report = {}

        def sums(rule, gamma):
            mx.p_diagnostics(dev["q"], dev["k"], rule=rule, rotate=True, causal=w.causal, gamma=gamma, out=out,
                             workspace=ws)
            return out.cpu().numpy().reshape(-1, 6).astype("float64")

        for name, rule in (("uos", mx.SCALE_UOS), ("ocp", mx.SCALE_OCP)):
            scan, rep = [], None
            for i in range(16):
                gf = 1.0 + i / 16.0
                g = sums(rule, gf)
                if i == 0:
                    rep = diagnostics_report(g)
                scan.append({"gamma_f": gf, "mean_row_sum": float(g[:, 0].mean()),
                             "over_normalized_rows": float((g[:, 0] > 1.0).mean())})
            best = min(scan, key=lambda r: abs(r["mean_row_sum"] - 1.0))
            kept = []
            g0 = 1.0 / rep["mean_row_sum"]
            for i in range(-8, 9):
                gam = g0 * (1.0 + 0.005 * i)
                rs = gam * sums(rule, gam)[:, 0]
                kept.append({"gamma": gam, "mean_row_sum": float(rs.mean()), "over_normalized_rows": float((rs > 1.0).mean())})
            rep["global_scaling"] = {
                "factor_removed": {"scan": scan, "closest_to_unit_mean": best},
                "factor_kept": {"scan": kept, "closest_to_unit_mean": min(kept, key=lambda r: abs(r["mean_row_sum"] - 1.0)),
                                "over_normalized_rows_at_gamma_1": rep["over_normalized_rows"]}}
            report[name] = rep
    return {
        "metric": metric, "value": round(rate, 2), "unit": unit, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(wall * 1000.0 / args.steps, 4), "ms_per_call": round(ms, 4),
        "higher_is_better": True, "dtype": "fp4", "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.describe()}", "part": args.part, "B": B, "H": H, "N": N, "d": d,
                   "causal": w.causal, **({"Nk": Nk} if Nk != N else {})},
        "roofline": {"bound": bound, "achieved": round(rate, 2), "peak": peak, "unit": unit,
                     "frac": round(rate / peak, 4), "traffic": None,
                     "work_per_call": work, "work_unit": "bytes" if unit == "GB/s" else "flops"},
        **({"report": report} if report is not None else {}),
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=2)
    ap.add_argument("--fused-q", action="store_true",
                    help="rotate and quantize Q inside the forward (mxattn_forward_fused_q)")
    ap.add_argument("--separate-quantize", action="store_true",
                    help="quantize Q, K and V with three mxattn_rotate_quantize launches instead of one "
                         "mxattn_rotate_quantize_qkv launch")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probes", action="store_true", help="skip the in-run throughput probes")
    ap.add_argument("--part", choices=("step", "sweep", "diagnostics"), default="step",
                    help="step: the benchmark (quantize + forward); sweep: the Q_max sweep of Q, K and V "
                         "over 41 boundaries; diagnostics: the materialized-P diagnostics call")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="run three plain device-to-device copies of BYTES bytes and exit "
                         "(reference kernel for scaling the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the path shards by "
              "(batch, head) with no communication, so per-GPU throughput is the one-GPU value.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import mxfp4_microscaled_bit_amd as mx
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    if args.copy_probe:
        # plain device-to-device copies: the reference kernel for scaling the
        # HBM byte counters, and the achievable read+write bandwidth
        n = args.copy_probe // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        times = []
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            dst.copy_(src)
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        best = min(times)
        print(json.dumps({"copy_bytes_per_launch": n * 4, "launches": 3, "best_ms": round(best, 4),
                          "read_plus_write_gb_per_s": round(2 * n * 4 / (best * 1e-3) / 1e9, 1)}), flush=True)
        return

    w = W.WORKLOADS[args.workload]
    B, H, N, d = w.shape
    Nk = w.kv_tokens  # key/value tokens (N unless cross-attention)
    log(f"workload {args.workload}: {w.name} {w.describe()}; generating inputs")
    t0 = time.perf_counter()
    dev = {}
    for t in "qkv":
        bits = W.generate(w, t)
        ten = torch.from_numpy(bits.view("int16")).view(torch.bfloat16 if w.dtype == W.BF16 else torch.float16)
        dev[t] = ten.cuda()
        del bits
    log(f"inputs resident in HBM after {time.perf_counter() - t0:.1f}s")

    stream = torch.cuda.current_stream()
    if args.part != "step":
        print(json.dumps(measure_part(args, w, dev, stream)), flush=True)
        return
    qm = mx.MXTensor.empty(B, H, N, d, mx.AXIS_HEAD_DIM)
    km = mx.MXTensor.empty(B, H, Nk, d, mx.AXIS_HEAD_DIM)
    vm = mx.MXTensor.empty(B, H, Nk, d, mx.AXIS_TOKEN)
    out = torch.empty((B, H, N, d), dtype=torch.float32, device="cuda")

    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    # events (on the launch stream) around the step's parts: e[0] start,
    # e[1] after Q's quantizer, e[2] after K's, e[3] after V's (with the
    # single Q, K, V launch e[1] = e[2] = e[0] and e[3] follows that launch),
    # e[4] after the forward
    separate = args.fused_q or args.separate_quantize

    def step(record=None):
        e = [ev() for _ in range(5)] if record is not None else None
        if e:
            e[0].record(stream)
        if not separate:
            mx.rotate_quantize_qkv(dev["q"], dev["k"], dev["v"], rotate=True, out=(qm, km, vm))
        else:
            if not args.fused_q:
                mx.rotate_quantize(dev["q"], mx.AXIS_HEAD_DIM, rotate=True, out=qm)
            if e:
                e[1].record(stream)
            mx.rotate_quantize(dev["k"], mx.AXIS_HEAD_DIM, rotate=True, out=km)
            if e:
                e[2].record(stream)
            mx.rotate_quantize(dev["v"], mx.AXIS_TOKEN, rotate=False, out=vm)
        if e:
            e[3].record(stream)
        if args.fused_q:
            mx.forward_fused_q(dev["q"], km, vm, causal=w.causal, out=out)
        else:
            mx.forward(qm, km, vm, causal=w.causal, out=out)
        if e:
            e[4].record(stream)
            record.append(e)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(events)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    quant_ms = sum(e[0].elapsed_time(e[3]) for e in events) / len(events)
    # The single quantizer launch on its own: ten back-to-back launches
    # between two events, behind one untimed launch that keeps the GPU busy
    # while they are queued.  The in-step events (quant_ms) also bracket the
    # stream's gap after the previous step's forward.
    quant_b2b_ms = None
    if not separate:
        torch.cuda.synchronize()
        qkv = lambda: mx.rotate_quantize_qkv(dev["q"], dev["k"], dev["v"], rotate=True, out=(qm, km, vm))  # noqa: E731
        qkv()
        e0, e1 = ev(), ev()
        e0.record(stream)
        for _ in range(QUANT_B2B_LAUNCHES):
            qkv()
        e1.record(stream)
        torch.cuda.synchronize()
        quant_b2b_ms = e0.elapsed_time(e1) / QUANT_B2B_LAUNCHES
    if separate:
        k_ms = sum(e[1].elapsed_time(e[2]) for e in events) / len(events)  # K's rotate + quantize
        v_ms = sum(e[2].elapsed_time(e[3]) for e in events) / len(events)  # V's quantize
    fwd_ms = sum(e[3].elapsed_time(e[4]) for e in events) / len(events)
    ms_per_step = wall * 1000.0 / args.steps
    flops = w.flops()
    pairs = flops / (4.0 * d)  # visible (query, key) pairs of one forward
    traffic = measured_traffic(flops) if args.workload == 2 and not args.fused_q else None
    value = flops / (ms_per_step * 1e-3) / 1e12
    fwd_tflops = flops / (fwd_ms * 1e-3) / 1e12
    quant_bytes = B * H * ((0 if args.fused_q else N) + 2 * Nk) * d * QUANT_BYTES_PER_ELEMENT
    quant_gbs_in_step = quant_bytes / (quant_ms * 1e-3) / 1e9
    quant_rate_ms = quant_b2b_ms if quant_b2b_ms is not None else quant_ms
    quant_gbs = quant_bytes / (quant_rate_ms * 1e-3) / 1e9

    def per_launch(ms, elements):
        gbs = elements * QUANT_BYTES_PER_ELEMENT / (ms * 1e-3) / 1e9
        return {"us": round(ms * 1e3, 2), "gb_per_s": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}

    result = {
        "metric": "fused MXFP4 attention fwd TFLOPS (1 GPU) + % of MXFP4 MFMA peak; quantizer GB/s",
        "value": round(value, 3),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp4",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.describe()}, one step = " +
                               ("rotate+quantize K; quantize V; fused PNQ forward with Q rotated and "
                                "quantized in its prologue" if args.fused_q else
                                "rotate+quantize Q, K and quantize V (three launches); fused PNQ forward"
                                if separate else
                                "rotate+quantize Q, K and quantize V (one launch); fused PNQ forward"),
                   "B": B, "H": H, "N": N, "d": d, "fused_q": bool(args.fused_q),
                   "quantizer_launches": (2 if args.fused_q else 3) if separate else 1,
                   "causal": w.causal, "kv_tile": mx.forward_kv_tile(d, w.causal),
                   **({"Nk": Nk} if Nk != N else {})},
        "forward": {"ms": round(fwd_ms, 4), "tflops": round(fwd_tflops, 2),
                    "frac_mfma_peak": round(fwd_tflops / MFMA_FP4_PEAK_TFLOPS, 4)},
        "quantizer": {"ms": round(quant_rate_ms, 4), "gb_per_s": round(quant_gbs, 1),
                      "frac_hbm_peak": round(quant_gbs / HBM_PEAK_GBS, 4),
                      "bytes": quant_bytes,
                      "timing": (f"per launch over {QUANT_B2B_LAUNCHES} back-to-back launches after the timed steps"
                                 if quant_b2b_ms is not None else "events around the launches in each timed step"),
                      "ms_in_step": round(quant_ms, 4),
                      "frac_hbm_peak_in_step": round(quant_gbs_in_step / HBM_PEAK_GBS, 4),
                      # separate launches: K's rotate+quantize (head-dim blocks)
                      # and V's quantize (token blocks), event-timed on the stream
                      **({"rotate_quantize_k": per_launch(k_ms, B * H * Nk * d),
                          "quantize_v": per_launch(v_ms, B * H * Nk * d)} if separate else {})},
        "roofline": {"bound": "mfma", "achieved": round(fwd_tflops, 2), "peak": MFMA_FP4_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(fwd_tflops / MFMA_FP4_PEAK_TFLOPS, 4),
                     "traffic": traffic,
                     "traffic_source": (f"stored: {os.path.relpath(TRAFFIC_FILE, ROOT)} (rocprofv3 FETCH_SIZE and "
                                        f"WRITE_SIZE of this kernel source, sha256 {kernel_source_hash()})"
                                        if traffic is not None else None)},
    }
    result["accuracy"] = accuracy_vs_fp32(w, dev, out)
    if not args.no_probes:
        from mxfp4_microscaled_bit_amd import probes

        log("running the in-run throughput probes")
        del dev
        torch.cuda.empty_cache()
        mfma = max(probes.mfma_fp4_tflops(groups=g) for g in (256, 512))
        mix = probes.pair_mix_gpairs()
        copy = probes.stream_gbs()
        read = probes.read_gbs()
        fwd_gpairs = pairs / (fwd_ms * 1e-3) / 1e9
        result["probes"] = {
            "mfma_fp4_tflops": round(mfma, 1),
            "pair_mix_gpair_per_s": round(mix, 1),
            "copy_read_write_gb_per_s": round(copy, 1),
            "read_gb_per_s": round(read, 1),
            "note": "measured in this run after the timed steps; the matrix probe runs four independent "
                    "32x32x64 FP4 accumulators per wave, the mix probe the forward's per-pair vector work at "
                    "two waves per SIMD, the copy probe 16-byte elements read and written, the read probe "
                    "16-byte elements read",
        }
        result["forward"]["frac_mfma_probe"] = round(fwd_tflops / mfma, 4)
        result["quantizer"]["frac_copy_probe"] = round(quant_gbs / copy, 4)
        result["quantizer"]["frac_read_probe"] = round(quant_gbs / read, 4)
        result["roofline_valu"] = {
            "bound": "alu", "achieved": round(fwd_gpairs, 2), "peak": round(mix, 2), "unit": "Gpair/s",
            "frac": round(fwd_gpairs / mix, 4), "traffic": None,
            "peak_source": "in-run probe of the per-pair vector work (1 v_fma_f32, 1 v_exp_f32, 1/2 "
                           "v_cvt_scalef32_pk_fp4_f32, 1/2 v_max3_f32) on every SIMD at two waves per SIMD",
            "pairs_per_launch": pairs,
        }
    if not args.no_cpu_baseline and Nk == N and not w.causal:
        log("timing the CPU oracle on a bounded sample")
        result["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
