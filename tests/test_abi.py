"""CPU checks of the C-ABI library: it loads, exports every function the header
declares, computes buffer sizes, and rejects bad arguments before touching
the GPU (nothing here launches a kernel)."""
import ctypes
import os
import re

import pytest

import mxfp4_microscaled_bit_amd as mx

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxattn.h")

FAKE = 0x100000  # 16-byte-aligned address never dereferenced by these calls


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mxattn_\w+)\s*\(", text)))


def test_library_exports_every_declared_function():
    L = mx.lib()
    names = declared_functions()
    assert set(names) == set(mx.EXPORTED)
    for n in names:
        assert hasattr(L, n), n


def test_sizes_and_tile():
    # Np = N rounded up to 128; head-dim codes d/2 and scales d/32 bytes per token
    assert mx.mx_codes_bytes(1, 2, 256, 128, mx.AXIS_HEAD_DIM) == 2 * 256 * 64
    assert mx.mx_scales_bytes(1, 2, 256, 128, mx.AXIS_HEAD_DIM) == 2 * 256 * 4
    assert mx.mx_codes_bytes(1, 40, 32760, 128, mx.AXIS_TOKEN) == 40 * 32768 * 64
    assert mx.mx_scales_bytes(16, 16, 4096, 64, mx.AXIS_TOKEN) == 256 * 4096 * 2
    assert mx.mx_codes_bytes(1, 1, 1, 64) == 128 * 32
    assert mx.mx_codes_bytes(1, 1, 1, 96) == 0
    assert mx.mx_codes_bytes(1, 1, 0, 64) == 0
    assert mx.mx_codes_bytes(1, 1, 5, 64, 7) == 0
    # at most 2^36 elements per tensor (B H Np d), so that every launch fits a dispatch
    assert mx.mx_codes_bytes(1, 1, 2 ** 29, 128) == 2 ** 35
    assert mx.mx_codes_bytes(1, 2, 2 ** 29, 128) == 0
    assert mx.mx_codes_bytes(2 ** 20, 1, 2 ** 9, 128) == 2 ** 35 and mx.mx_codes_bytes(2 ** 20, 1, 2 ** 9 + 1, 128) == 0
    assert mx.forward_kv_tile(128) == 128 and mx.forward_kv_tile(64, True) == 128
    assert mx.forward_kv_tile(80) == 0
    ws = mx.reference_modes_workspace_bytes(1, 2, 256, 128, mx.P_POSTNORM)
    assert ws >= 3 * (2 * 256 * 64 + 2 * 256 * 4) + 2 * 256 * 2 * 4
    assert mx.reference_modes_workspace_bytes(1, 2, 256, 128, 9) == 0


def test_status_strings():
    for s in range(10):
        assert mx.status_string(s)
    assert "unknown" in mx.status_string(42)


def _desc(axis, B=1, H=1, N=64, d=64, codes=FAKE, scales=FAKE, rotated=1):
    return mx.MXTensorDesc(codes, scales, mx.Shape(B, H, N, d), axis, 0, rotated)


def _rq(x=FAKE, dtype=mx.BF16, shape=(1, 1, 64, 64), strides=None, axis=0, rotate=1, rule=0, out=None):
    L = mx.lib()
    if out is None:
        out = mx.MXTensorDesc(FAKE, FAKE + 4096, mx.Shape(0, 0, 0, 0), 5, 5, 5)
    st = None if strides is None else (ctypes.c_int64 * 3)(*strides)
    return L.mxattn_rotate_quantize(x, dtype, mx.Shape(*shape), st, axis, rotate, rule, ctypes.byref(out),
                                    None), out


def test_rotate_quantize_rejects_bad_arguments_without_writing():
    cases = [
        (dict(x=None), 1),
        (dict(out=mx.MXTensorDesc(None, FAKE, mx.Shape(0, 0, 0, 0), 5, 5, 5)), 1),
        (dict(shape=(1, 1, 64, 96)), 2),
        (dict(shape=(0, 1, 64, 64)), 2),
        (dict(shape=(1, 1, 0, 64)), 2),
        (dict(dtype=7), 3),
        (dict(x=FAKE + 8), 4),
        (dict(strides=(4096, 4096, 60)), 5),
        (dict(strides=(4096, -64, 64)), 5),
        (dict(strides=(4096, 4096, 32)), 5),
        (dict(axis=3), 8),
        (dict(rule=2), 8),
        (dict(axis=1, rotate=1), 8),
        (dict(rotate=2), 8),
    ]
    for kwargs, expect in cases:
        status, out = _rq(**kwargs)
        assert status == expect, (kwargs, status)
        # on error the descriptor is not touched
        if "out" not in kwargs:
            assert (out.axis, out.rule, out.rotated, out.shape.N) == (5, 5, 5, 0)


def test_forward_rejects_bad_arguments():
    L = mx.lib()

    def fwd(q=None, k=None, v=None, causal=0, out=FAKE, stats=None):
        q = q or _desc(0)
        k = k or _desc(0)
        v = v or _desc(1)
        return L.mxattn_forward(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), causal, out, stats, None)

    assert fwd(out=None) == 1
    assert fwd(q=_desc(0, codes=None)) == 1
    assert fwd(k=_desc(1)) == 6          # K must be head-dim blocked
    assert fwd(v=_desc(0)) == 6          # V must be token blocked
    assert fwd(k=_desc(0, N=65)) == 6    # K and V shapes disagree
    assert fwd(k=_desc(0, N=65), v=_desc(1, N=65), causal=1) == 6  # causal cross-attention
    assert fwd(k=_desc(0, H=2), v=_desc(1, H=2)) == 6  # heads disagree
    assert fwd(k=_desc(0, d=128), v=_desc(1, d=128)) == 6  # head dims disagree
    assert fwd(k=_desc(0, rotated=0)) == 6  # Q rotated, K not
    assert fwd(v=_desc(1, d=96)) == 2
    assert fwd(causal=2) == 8
    assert fwd(out=FAKE + 4) == 4
    assert fwd(stats=FAKE + 4) == 4
    assert fwd(q=_desc(0, scales=FAKE + 1)) == 4


def test_reference_modes_reject_bad_arguments():
    L = mx.lib()
    need = mx.reference_modes_workspace_bytes(1, 1, 64, 64, mx.P_DIRECT)

    def ref(q=FAKE, rule=0, p_mode=1, rotate=0, causal=0, ws=FAKE, ws_bytes=None, out=FAKE, shape=(1, 1, 64, 64),
            dtype=0, sums=None):
        return L.mxattn_quantize_reference_modes(q, FAKE, FAKE, dtype, mx.Shape(*shape), None, rule, p_mode, rotate,
                                                 causal, out, sums, ws, need if ws_bytes is None else ws_bytes, None)

    assert ref(q=None) == 1
    assert ref(out=None) == 1
    assert ref(dtype=3) == 3
    assert ref(rule=5) == 8
    assert ref(p_mode=3) == 8
    assert ref(rotate=3) == 8
    assert ref(causal=-1) == 8
    assert ref(shape=(1, 1, 64, 32)) == 2
    assert ref(ws=None) == 7
    assert ref(ws_bytes=need - 1) == 7
    assert ref(q=FAKE + 2) == 4
    assert ref(sums=FAKE + 12) == 4


def test_ceiling_rule_and_sweep_reject_bad_arguments():
    L = mx.lib()
    out = mx.MXTensorDesc(FAKE, FAKE + 4096, mx.Shape(0, 0, 0, 0), 5, 5, 5)
    shp = mx.Shape(1, 1, 64, 64)

    def rq(q=7.0, x=FAKE, axis=0, rotate=1, dtype=0):
        return L.mxattn_rotate_quantize_q(x, dtype, shp, None, axis, rotate, q, ctypes.byref(out), None)

    assert rq(x=None) == 1
    assert rq(dtype=4) == 3
    for q in (1.99, 64.5, float("nan"), float("inf"), -7.0):
        assert rq(q=q) == 8
    assert rq(axis=1, rotate=1) == 8
    assert (out.axis, out.rule, out.rotated) == (5, 5, 5)  # untouched on error
    # the plain entry point does not take the ceiling rule (it needs q)
    assert L.mxattn_rotate_quantize(FAKE, 0, shp, None, 0, 1, mx.SCALE_CEIL_Q, ctypes.byref(out), None) == 8

    need = mx.scale_sweep_workspace_bytes(1, 1, 64, 64, mx.AXIS_HEAD_DIM, 3)
    assert need > 0 and mx.scale_sweep_workspace_bytes(1, 1, 64, 64, mx.AXIS_HEAD_DIM, 49) == 0
    assert mx.scale_sweep_workspace_bytes(1, 1, 64, 64, 3, 1) == 0

    def sw(qs=(6.0, 7.0, 8.0), x=FAKE, sse=FAKE, ws=FAKE, ws_bytes=None, axis=0, rotate=1):
        arr = (ctypes.c_double * max(len(qs), 1))(*qs)
        return L.mxattn_scale_sweep(x, 0, shp, None, axis, rotate, arr, len(qs), sse, ws,
                                    need if ws_bytes is None else ws_bytes, None)

    assert sw(x=None) == 1 and sw(sse=None) == 1
    assert sw(qs=()) == 8
    assert sw(qs=tuple([7.0] * 49)) == 8
    assert sw(qs=(6.0, 12.5)) == 8          # max > 2 min
    assert sw(qs=(1.5, 2.5)) == 8           # below the range
    assert sw(axis=1, rotate=1) == 8
    assert sw(ws=None) == 7 and sw(ws_bytes=need - 1) == 7
    assert sw(sse=FAKE + 8) == 4


def test_p_diagnostics_rejects_bad_arguments():
    L = mx.lib()
    need = mx.p_diagnostics_workspace_bytes(1, 1, 64, 64)
    # Q^, K^ (codes + scales, 128 padded rows each) and the fp32 (m, l) pairs
    assert need >= 2 * (128 * 32 + 128 * 2) + 128 * 2 * 4
    assert mx.p_diagnostics_workspace_bytes(1, 1, 64, 96) == 0

    def dg(q=FAKE, k=FAKE, dtype=0, shape=(1, 1, 64, 64), rule=0, rotate=1, causal=0, gamma=1.0, out=FAKE,
           ws=FAKE, ws_bytes=None):
        return L.mxattn_p_diagnostics(q, k, dtype, mx.Shape(*shape), None, rule, rotate, causal, gamma, out, ws,
                                      need if ws_bytes is None else ws_bytes, None)

    assert dg(q=None) == 1 and dg(k=None) == 1 and dg(out=None) == 1
    assert dg(dtype=2) == 3
    assert dg(rule=mx.SCALE_CEIL_Q) == 8 and dg(rule=-1) == 8
    assert dg(rotate=2) == 8 and dg(causal=3) == 8
    for gamma in (0.0, -1.0, float("nan"), float("inf"), 2.0 ** 21, 2.0 ** -21):
        assert dg(gamma=gamma) == 8, gamma
    assert dg(shape=(1, 1, 64, 32)) == 2
    assert dg(ws=None) == 7 and dg(ws_bytes=need - 1) == 7
    assert dg(out=FAKE + 4) == 4 and dg(k=FAKE + 2) == 4


def test_forward_fused_q_rejects_bad_arguments():
    L = mx.lib()

    def fq(q=FAKE, dtype=0, shape=(1, 1, 64, 64), strides=None, k=None, v=None, causal=0, out=FAKE, stats=None):
        k = k or _desc(0)
        v = v or _desc(1)
        st = None if strides is None else (ctypes.c_int64 * 3)(*strides)
        return L.mxattn_forward_fused_q(q, dtype, mx.Shape(*shape), st, ctypes.byref(k), ctypes.byref(v), causal,
                                        out, stats, None)

    assert fq(q=None) == 1 and fq(out=None) == 1
    assert fq(dtype=5) == 3
    assert fq(shape=(1, 1, 64, 96)) == 2 and fq(shape=(1, 0, 64, 64)) == 2
    assert fq(strides=(4096, 4096, 60)) == 5
    assert fq(q=FAKE + 8) == 4 and fq(out=FAKE + 4) == 4
    assert fq(shape=(1, 2, 64, 64)) == 6                 # heads disagree with K^
    assert fq(shape=(1, 1, 64, 128)) == 6                # head dims disagree
    assert fq(shape=(1, 1, 65, 64), causal=1) == 6       # causal cross-attention
    assert fq(causal=2) == 8
    k_ceil = mx.MXTensorDesc(FAKE, FAKE, mx.Shape(1, 1, 64, 64), 0, mx.SCALE_CEIL_Q, 1)
    assert fq(k=k_ceil) == 8
    assert fq(v=_desc(0)) == 6                           # V must be token blocked


def test_binding_refuses_host_tensors_before_any_call():
    """The library receives raw addresses and launches on the current device:
    the binding refuses host tensors (whose addresses a kernel cannot read)
    before anything reaches the library."""
    import torch
    x = torch.zeros(1, 1, 128, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="device tensors"):
        mx.rotate_quantize(x)
    with pytest.raises(ValueError, match="device tensors"):
        mx.scale_sweep(x, [7.25])
    with pytest.raises(ValueError, match="device tensors"):
        mx.quantize_reference_modes(x, x, x)
    with pytest.raises(ValueError, match="device tensors"):
        mx.p_diagnostics(x, x)
    with pytest.raises(ValueError, match="device tensors"):
        mx._device(torch.zeros(1, device="meta"))
    host = mx.MXTensor(torch.zeros(4096, dtype=torch.uint8), torch.zeros(256, dtype=torch.uint8), (1, 1, 128, 64),
                       mx.AXIS_HEAD_DIM)
    with pytest.raises(ValueError, match="device tensors"):
        host.desc()
    with pytest.raises(ValueError, match="device tensors"):
        mx.forward(host, host, host, out=torch.zeros(1, 1, 128, 64))


def test_binding_buffer_lengths():
    """Outputs and workspaces must be contiguous and long enough: the C ABI
    cannot see their lengths."""
    import torch
    mx._buffer(torch.zeros(16, dtype=torch.float32), 64, "out")
    with pytest.raises(ValueError, match="holds 60 bytes; 64 are needed"):
        mx._buffer(torch.zeros(15, dtype=torch.float32), 64, "out")
    with pytest.raises(ValueError, match="contiguous"):
        mx._buffer(torch.zeros(8, 8)[:, ::2], 16, "out")


def test_rotate_quantize_qkv_rejects_bad_arguments_without_writing():
    """Every case fails validation, so nothing is launched and no descriptor
    is written."""
    L = mx.lib()

    def qkv(q=FAKE, k=FAKE, v=FAKE, dtype=mx.BF16, qs=(1, 2, 64, 64), kvs=(1, 2, 64, 64), rotate=1, rule=0,
            outs=None):
        if outs is None:
            outs = [mx.MXTensorDesc(FAKE, FAKE + 4096, mx.Shape(0, 0, 0, 0), 5, 5, 5) for _ in range(3)]
        st = L.mxattn_rotate_quantize_qkv(q, k, v, dtype, mx.Shape(*qs), mx.Shape(*kvs), None, None, None, rotate,
                                          rule, *[ctypes.byref(o) if o is not None else None for o in outs], None)
        return st, outs

    cases = [
        (dict(q=None), 1),
        (dict(v=None), 1),
        (dict(outs=[None, None, None]), 1),
        (dict(dtype=5), 3),
        (dict(qs=(1, 2, 64, 96), kvs=(1, 2, 64, 96)), 2),
        (dict(k=FAKE + 8), 4),
        (dict(rotate=2), 8),
        (dict(rule=2), 8),
        (dict(rule=9), 8),
        (dict(qs=(1, 3, 64, 64)), 6),
        (dict(qs=(1, 2, 64, 128)), 6),
    ]
    for kwargs, expect in cases:
        status, outs = qkv(**kwargs)
        assert status == expect, (kwargs, status)
        if "outs" not in kwargs:
            for o in outs:
                assert (o.axis, o.rule, o.rotated, o.shape.N) == (5, 5, 5, 0)
