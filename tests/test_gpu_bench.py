"""The benchmark's output contract on the GPU: one JSON line with the agreed
fields, consistent units and a roofline entry, from a short run of the
small workload (the full Wan-like run is the benchmark itself)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                       timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1, r.stdout
    return json.loads(lines[0])


@pytest.mark.gpu
def test_bench_json_line():
    d = _run("--workload", "1", "--steps", "2", "--warmup", "1", "--no-cpu-baseline")
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "forward", "quantizer", "accuracy"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 2 and d["warmup"] == 1
    assert d["unit"] == "TFLOPS" and d["higher_is_better"] is True and d["data"] == "synthetic"
    assert d["value"] > 0 and d["ms_per_step"] > 0
    assert d["config"]["workload"].startswith("tiny_outliers")
    rf = d["roofline"]
    assert rf["bound"] == "mfma" and rf["unit"] == "TFLOP/s" and rf["peak"] == 10100.0
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    assert rf["achieved"] == d["forward"]["tflops"]
    q = d["quantizer"]
    assert q["gb_per_s"] > 0 and 0 < q["frac_hbm_peak"] < 1
    assert d["config"]["quantizer_launches"] == 1 and "rotate_quantize_k" not in q
    # the rate comes from back-to-back launches; the in-step events are reported beside it
    assert q["timing"].startswith("per launch over") and q["ms"] > 0 and q["ms_in_step"] > 0
    a = d["accuracy"]
    assert -1.0 <= a["mean_row_cosine"] <= 1.0 and a["max_abs"] >= 0
    # in-run probes and the vector-unit roofline priced against them
    p = d["probes"]
    assert p["mfma_fp4_tflops"] > 0 and p["pair_mix_gpair_per_s"] > 0 and p["copy_read_write_gb_per_s"] > 0
    rv = d["roofline_valu"]
    assert rv["bound"] == "alu" and rv["unit"] == "Gpair/s" and abs(rv["peak"] - p["pair_mix_gpair_per_s"]) < 0.1
    assert abs(rv["frac"] - rv["achieved"] / rv["peak"]) < 1e-3
    assert rv["pairs_per_launch"] == 1 * 2 * 256 * 256  # B H N Nk of the tiny workload
    assert d["forward"]["frac_mfma_probe"] > 0 and d["quantizer"]["frac_copy_probe"] > 0


@pytest.mark.gpu
def test_bench_probes_measure_plausible_rates():
    """The probes on their own: the dense FP4 matrix rate is within the
    published 10.1 PFLOP/s (and above a third of it), the copy bandwidth
    within the 8 TB/s HBM peak."""
    sys.path.insert(0, ROOT)
    from mxfp4_microscaled_bit_amd import probes
    mfma = probes.mfma_fp4_tflops(groups=256, iters=500)
    copy = probes.stream_gbs(nbytes=256 << 20)
    read = probes.read_gbs(nbytes=256 << 20)
    mix = probes.pair_mix_gpairs(iters=200)
    assert 3000 < mfma < 10100 * 1.02, mfma
    assert 500 < copy < 8000 and 500 < read < 8000, (copy, read)
    assert mix > 0


@pytest.mark.gpu
def test_bench_separate_quantizer_launches():
    d = _run("--workload", "1", "--steps", "2", "--warmup", "1", "--no-cpu-baseline", "--separate-quantize")
    q = d["quantizer"]
    assert d["config"]["quantizer_launches"] == 3
    assert q["rotate_quantize_k"]["us"] > 0 and q["quantize_v"]["us"] > 0


@pytest.mark.gpu
def test_bench_fused_q_step():
    d = _run("--workload", "1", "--steps", "2", "--warmup", "1", "--no-cpu-baseline", "--fused-q")
    assert d["config"]["fused_q"] is True and d["config"]["quantizer_launches"] == 2
    assert d["forward"]["tflops"] > 0 and d["quantizer"]["quantize_v"]["us"] > 0


@pytest.mark.gpu
@pytest.mark.parametrize("part,unit,bound", [("sweep", "GB/s", "hbm"), ("diagnostics", "TFLOP/s", "mfma")])
def test_bench_other_parts(part, unit, bound):
    """The Q_max sweep and the diagnostics call timed on their own, each with
    a roofline against its own peak."""
    d = _run("--workload", "1", "--steps", "2", "--warmup", "1", "--part", part)
    assert d["config"]["part"] == part and d["unit"] == unit and d["value"] > 0
    rf = d["roofline"]
    assert rf["bound"] == bound and abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3 and rf["work_per_call"] > 0
    if part == "sweep":
        for t in "qkv":
            rep = d["report"][t]
            assert 6.0 <= rep["tensor_optimum_q"] <= 8.0 and 0 < rep["J_at_optimum_over_J_at_7.25"] <= 1.0
            assert sum(rep["head_optimum_counts"].values()) == 2
    if part == "diagnostics":
        for rule in ("uos", "ocp"):
            rep = d["report"][rule]
            assert rep["rows"] == 2 * 256 and 0.5 < rep["mean_row_sum"] < 1.5
            assert abs(sum(b["share"] for b in rep["entropy_bins"]) - 1.0) < 1e-9
            parts = rep["mean_zeroing"] + rep["mean_saturation"] + rep["mean_down"] + rep["mean_up"]
            assert abs((rep["mean_row_sum"] - 1.0) - parts) < 1e-4
            gs = rep["global_scaling"]["factor_removed"]
            assert len(gs["scan"]) == 16 and gs["scan"][0]["gamma_f"] == 1.0
            assert abs(gs["scan"][0]["mean_row_sum"] - rep["mean_row_sum"]) < 1e-12
            assert gs["closest_to_unit_mean"] in gs["scan"]
            gk = rep["global_scaling"]["factor_kept"]
            assert len(gk["scan"]) == 17 and gk["closest_to_unit_mean"] in gk["scan"]
            assert abs(gk["closest_to_unit_mean"]["mean_row_sum"] - 1.0) < 0.05  # small tensors: decisions jump with gamma


def test_diagnostics_report_statistics():
    """(CPU) the Fig. 7 statistics of the diagnostics line on a hand-made
    array: means, over/under-normalized shares and the entropy bins."""
    import numpy as np
    sys.path.insert(0, ROOT)
    import bench
    d = np.zeros((1, 2, 5, 6))
    d[..., 0] = [[0.9, 1.1, 1.0, 0.8, 1.2], [0.9, 1.1, 1.0, 0.8, 1.2]]
    d[..., 1] = -0.05
    d[..., 4] = 0.02
    d[..., 5] = [[0.5, 2.5, 6.0, 7.0, 1.0], [0.5, 2.5, 6.0, 7.0, 1.0]]
    r = bench.diagnostics_report(d)
    assert r["rows"] == 10 and abs(r["mean_row_sum"] - 1.0) < 1e-12
    assert abs(r["mean_zeroing"] + 0.05) < 1e-12 and abs(r["mean_up"] - 0.02) < 1e-12
    assert r["over_normalized_rows"] == 0.4 and r["under_normalized_rows"] == 0.4
    bins = {b["entropy_nats"]: b for b in r["entropy_bins"]}
    assert list(bins) == ["<1", "1-2", "2-3", "3-4", "4-5", ">=5"]
    assert bins["<1"]["share"] == 0.2 and abs(bins["<1"]["mean_row_sum"] - 0.9) < 1e-12
    assert bins["1-2"]["share"] == 0.2 and bins["1-2"]["over_normalized"] == 1.0  # entropy 1.0 opens its bin
    assert bins[">=5"]["share"] == 0.4 and abs(bins[">=5"]["mean_row_sum"] - 0.9) < 1e-12
    assert bins[">=5"]["over_normalized"] == 0.0
    assert bins["3-4"]["share"] == 0.0 and bins["3-4"]["mean_row_sum"] is None


def test_sweep_report_optima():
    """(CPU) Table 4's statistics of the sweep line on a hand-made array:
    the tensor optimum minimizes the sum over heads, ties go to the smaller q."""
    import numpy as np
    sys.path.insert(0, ROOT)
    import bench
    qs = [6.0 + 0.05 * i for i in range(41)]
    e = np.full((3, 41), 10.0)
    e[0, 25] = 1.0   # head 0: 7.25
    e[1, 24] = 2.0   # head 1: 7.20
    e[2, 25] = 9.0   # head 2: 7.25 (J(7.25) = 20, J(7.20) = 22)
    e[2, 30] = 9.0   # ... tied with 7.50: the smaller q wins
    r = bench.sweep_report(e, qs)
    assert r["tensor_optimum_q"] == 7.25 and r["J_at_optimum_over_J_at_7.25"] == 1.0
    assert r["head_optimum_counts"] == {"7.20": 1, "7.25": 2}


def test_bench_refuses_more_than_one_gpu():
    """(CPU) the one-GPU scope is enforced before any GPU work."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0 and "one GPU" in r.stderr
