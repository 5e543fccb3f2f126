"""The scaled matrix products of every forward kernel keep their E8M0 scale
registers until the product is known to be done (see tests/scale_liveness.py).

The rule itself is pinned on hand-written snippets (an immediate register
reuse, an LDS load into the scale register, a later product over it, and the
covered cases); then attention.hip is compiled to gfx950 assembly with the
library's own flags and every k_attention* kernel is checked."""
import os
import shutil
import subprocess
import sys

import pytest

from scale_liveness import functions, unsafe_products

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

PRODUCT = "v_mfma_scale_f32_32x32x64_f8f6f4 v[2:17], v[102:105], v[110:113], v[2:17], v129, v124 op_sel_hi:[0,0,0]"


def _fn(*lines):
    return "_Zkernel:\n" + "\n".join("\t" + ln for ln in lines) + "\n.Lfunc_end0:\n"


def _check(*lines):
    (ins,) = functions(_fn(*lines)).values()
    return unsafe_products(ins)


def test_immediate_reuse_of_a_scale_register_is_flagged():
    n, bad = _check(PRODUCT, "v_mov_b32_e32 v129, v90", "v_add_f32_e32 v3, v2, v4")
    assert n == 1 and bad == [(0, ["v124", "v129"], 1)]


def test_lds_load_into_a_scale_register_is_flagged():
    n, bad = _check(PRODUCT, "ds_read_b64 v[128:129], v34 offset:8704", "s_nop 5", "v_mul_f32_e32 v17, v17, v1")
    assert len(bad) == 1 and bad[0][2] == 1


def test_later_product_over_a_scale_register_is_flagged():
    later = "v_mfma_scale_f32_16x16x128_f8f6f4 v[122:125], v[98:101], v[110:113], v[114:117], v133, v140"
    _, bad = _check(PRODUCT, later, "v_add_f32_e32 v3, v122, v4")
    assert len(bad) == 1


def test_read_of_the_result_covers_the_product():
    n, bad = _check(PRODUCT, "s_nop 7", "v_add_f32_e32 v3, v2, v4", "v_mov_b32_e32 v129, v90")
    assert n == 1 and bad == []


def test_read_of_a_later_result_covers_the_product():
    later = "v_mfma_scale_f32_32x32x64_f8f6f4 v[18:33], v[106:109], v[110:113], v[18:33], v140, v141"
    _, bad = _check(PRODUCT, later, "v_max3_f32 v3, v18, v19, v20", "v_mov_b32_e32 v124, 0")
    assert bad == []


def test_store_of_the_result_covers_the_product():
    _, bad = _check(PRODUCT, "global_store_dwordx4 v[64:65], v[2:5], off", "v_mov_b32_e32 v129, v90")
    assert bad == []


def test_conditional_branch_is_scanned_through():
    _, bad = _check(PRODUCT, "s_cbranch_vccz .LBB0_3", "v_mov_b32_e32 v124, v90")
    assert len(bad) == 1


def _hipcc():
    path = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    return path if shutil.which(path) else None


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not available")
def test_every_forward_kernel_keeps_its_scale_registers(tmp_path):
    from mxfp4_microscaled_bit_amd import build as B
    out = tmp_path / "attention.s"
    cmd = [_hipcc()] + B.COMMON + B.SOURCES["attention.hip"] + [
        "--cuda-device-only", "-S", os.path.join(B.CSRC, "attention.hip"), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    fns = {k: v for k, v in functions(out.read_text()).items() if "k_attention" in k}
    assert len(fns) >= 30
    report = []
    for name, ins in fns.items():
        n, bad = unsafe_products(ins)
        assert n > 0, name
        report += [(name, b) for b in bad]
    assert not report, report[:5]
