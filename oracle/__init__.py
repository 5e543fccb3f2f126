"""CPU oracle for MXAttention's MXFP4 attention forward -- TEST INFRASTRUCTURE.

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The product path (the HIP kernels behind
``libmxattn``) never calls it, and shares no code with it.

This module is a thin ctypes layer over ``oracle.c``: argument marshalling
only, no arithmetic of the method.  See ``oracle.h`` for the definitions and
the passages of the pages each function follows.
"""
import ctypes
import os

import numpy as np

from . import build as _build

BF16, FP16 = 0, 1
AXIS_HEAD_DIM, AXIS_TOKEN = 0, 1
RULE_UOS, RULE_OCP, RULE_CEIL_Q, RULE_FLOOR_Q = 0, 1, 2, 3
P_PNQ, P_DIRECT, P_POSTNORM, P_EXACT = 0, 1, 2, 3

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = _build.LIB
    src = os.path.join(os.path.dirname(path), "oracle.c")
    if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(src):
        _build.build()
    lib = ctypes.CDLL(path)
    u8p = ctypes.POINTER(ctypes.c_uint8)
    lib.oracle_e2m1_magnitude.restype = ctypes.c_double
    lib.oracle_e2m1_magnitude.argtypes = [ctypes.c_int]
    lib.oracle_e2m1_value.restype = ctypes.c_double
    lib.oracle_e2m1_value.argtypes = [ctypes.c_int]
    lib.oracle_e2m1_project.restype = ctypes.c_int
    lib.oracle_e2m1_project.argtypes = [ctypes.c_double]
    lib.oracle_scale_exponent.restype = ctypes.c_int
    lib.oracle_scale_exponent.argtypes = [ctypes.c_double, ctypes.c_int, ctypes.c_double]
    lib.oracle_scale_exponents.restype = None
    lib.oracle_scale_exponents.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                           ctypes.c_double, ctypes.c_void_p]
    lib.oracle_quantize_block.restype = ctypes.c_int
    lib.oracle_quantize_block.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_double, u8p, ctypes.c_void_p]
    lib.oracle_p_block_allowance.restype = ctypes.c_int
    lib.oracle_p_block_allowance.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_double, ctypes.c_double,
                                             ctypes.c_double, ctypes.c_void_p, ctypes.c_void_p]
    lib.oracle_decode_half.restype = ctypes.c_float
    lib.oracle_decode_half.argtypes = [ctypes.c_uint16, ctypes.c_int]
    lib.oracle_hadamard_rotate_f32.restype = None
    lib.oracle_hadamard_rotate_f32.argtypes = [ctypes.c_void_p, ctypes.c_int]
    lib.oracle_quantize_rows.restype = ctypes.c_int
    lib.oracle_quantize_rows.argtypes = [
        ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_double,
        ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
    lib.oracle_p_diagnostics.restype = ctypes.c_int
    lib.oracle_p_diagnostics.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.c_int32, ctypes.c_double, ctypes.c_void_p,
                                         ctypes.c_void_p]
    lib.oracle_scale_sweep.restype = ctypes.c_int
    lib.oracle_scale_sweep.argtypes = [
        ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
        ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int]
    lib.oracle_quantize_token_blocks.restype = ctypes.c_int
    lib.oracle_quantize_token_blocks.argtypes = [
        ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_void_p, ctypes.c_int, ctypes.c_double,
        ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
    lib.oracle_attention.restype = ctypes.c_int
    lib.oracle_attention.argtypes = [ctypes.c_void_p] + [ctypes.c_void_p] * 4 + [
        ctypes.c_void_p, ctypes.c_int32] + [ctypes.c_void_p] * 7
    _lib = lib
    return lib


class AttnCfg(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("N", ctypes.c_int32),
                ("d", ctypes.c_int32), ("dtype", ctypes.c_int32), ("causal", ctypes.c_int32),
                ("rotate", ctypes.c_int32), ("quant", ctypes.c_int32), ("rule", ctypes.c_int32),
                ("p_mode", ctypes.c_int32), ("kv_tile", ctypes.c_int32),
                ("nthreads", ctypes.c_int32), ("q", ctypes.c_double),
                ("amb_delta", ctypes.c_double), ("Nk", ctypes.c_int32)]


def default_threads() -> int:
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        return int(env)
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def e2m1_magnitude(code: int) -> float:
    return _load().oracle_e2m1_magnitude(code)


def e2m1_value(code: int) -> float:
    return _load().oracle_e2m1_value(code)


def e2m1_project(y: float) -> int:
    return _load().oracle_e2m1_project(float(y))


def scale_exponent(M: float, rule: int = RULE_UOS, q: float = 0.0) -> int:
    return _load().oracle_scale_exponent(float(M), rule, float(q))


def scale_exponents(M, rule: int = RULE_UOS, q: float = 0.0):
    """Vectorized scale_exponent over a float64 array of positive maxima."""
    M = np.ascontiguousarray(M, dtype=np.float64)
    out = np.empty(M.shape, np.int32)
    _load().oracle_scale_exponents(_ptr(M), M.size, rule, float(q), _ptr(out))
    return out


def quantize_block(x, rule: int = RULE_UOS, q: float = 0.0):
    """Returns (scale_byte, codes[n], clamped exponent) for one block of <= 32 values."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    assert x.ndim == 1 and x.size <= 32
    codes = np.zeros(x.size, np.uint8)
    sb = ctypes.c_uint8(0)
    e = _load().oracle_quantize_block(_ptr(x), x.size, rule, float(q), ctypes.byref(sb), _ptr(codes))
    return sb.value, codes, e


def p_block_allowance(p, rule: int = RULE_UOS, q: float = 0.0, delta: float = 0.0, exact_ref: float = 0.0):
    """One 32-key block of the softmax-path quantizer with its decision
    allowance.  Returns (dequantized P^ [32], allowance dp [32], exponent)."""
    p = np.ascontiguousarray(p, dtype=np.float64)
    assert p.shape == (32,)
    ph = np.empty(32, np.float64)
    dp = np.empty(32, np.float64)
    e = _load().oracle_p_block_allowance(_ptr(p), rule, float(q), float(delta), float(exact_ref), _ptr(ph), _ptr(dp))
    return ph, dp, e


def decode_half(bits: int, dtype: int) -> float:
    return _load().oracle_decode_half(int(bits), dtype)


def hadamard_rotate_f32(x):
    """Rotates a float32 vector of power-of-two length; returns a new array."""
    x = np.array(x, dtype=np.float32, copy=True)
    assert x.ndim == 1
    _load().oracle_hadamard_rotate_f32(_ptr(x), x.size)
    return x


def _strides(strides):
    if strides is None:
        return None
    return np.ascontiguousarray(np.asarray(strides, dtype=np.int64))


def quantize_rows(x_bits, dtype, B, H, N, d, *, rotate, rule=RULE_UOS, q=0.0, rows=None,
                  strides=None, nthreads=None):
    """Head-dimension quantization of Q/K rows.

    ``x_bits``: uint16 array holding the B*H*N*d input elements (contiguous unless
    ``strides`` is given).  ``rows``: global row indices (b*H+h)*N+n, or None for all.
    Returns (codes uint8 [n_rows, d], scales uint8 [n_rows, d//32]).
    """
    x_bits = np.asarray(x_bits)
    assert x_bits.dtype == np.uint16
    if strides is None:
        x_bits = np.ascontiguousarray(x_bits)
    rows_a = None if rows is None else np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    n_rows = B * H * N if rows_a is None else rows_a.size
    codes = np.empty((n_rows, d), np.uint8)
    scales = np.empty((n_rows, d // 32), np.uint8)
    st = _strides(strides)
    rc = _load().oracle_quantize_rows(
        _ptr(x_bits), dtype, B, H, N, d, _ptr(st), int(bool(rotate)), rule, float(q),
        _ptr(rows_a), n_rows, _ptr(codes), _ptr(scales), nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_quantize_rows rejected its arguments")
    return codes, scales


def quantize_token_blocks(x_bits, dtype, B, H, N, d, *, rule=RULE_UOS, q=0.0, blocks=None,
                          strides=None, nthreads=None):
    """Token-axis quantization of V.  ``blocks``: global block indices (b*H+h)*NB+kb
    with NB = ceil(N/32), or None for all.  Returns (codes uint8 [n_blocks, d, 32],
    scales uint8 [n_blocks, d])."""
    x_bits = np.asarray(x_bits)
    assert x_bits.dtype == np.uint16
    if strides is None:
        x_bits = np.ascontiguousarray(x_bits)
    NB = (N + 31) // 32
    blk_a = None if blocks is None else np.ascontiguousarray(np.asarray(blocks, dtype=np.int64))
    n_blocks = B * H * NB if blk_a is None else blk_a.size
    codes = np.empty((n_blocks, d, 32), np.uint8)
    scales = np.empty((n_blocks, d), np.uint8)
    st = _strides(strides)
    rc = _load().oracle_quantize_token_blocks(
        _ptr(x_bits), dtype, B, H, N, d, _ptr(st), rule, float(q), _ptr(blk_a), n_blocks,
        _ptr(codes), _ptr(scales), nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_quantize_token_blocks rejected its arguments")
    return codes, scales


def scale_sweep(x_bits, dtype, B, H, N, d, qs, *, axis=AXIS_HEAD_DIM, rotate=False, heads=None,
                strides=None, nthreads=None):
    """Per-head sum of squared MXFP4 quantization errors for each boundary in
    ``qs`` (rule e = ceil(log2(M/q))).  ``heads``: indices b*H+h or None for all.
    Returns float64 [n_heads, len(qs)]."""
    x_bits = np.asarray(x_bits)
    assert x_bits.dtype == np.uint16
    if strides is None:
        x_bits = np.ascontiguousarray(x_bits)
    qa = np.ascontiguousarray(np.asarray(qs, dtype=np.float64))
    hd = None if heads is None else np.ascontiguousarray(np.asarray(heads, dtype=np.int64))
    nh = B * H if hd is None else hd.size
    sse = np.empty((nh, qa.size), np.float64)
    rc = _load().oracle_scale_sweep(_ptr(x_bits), dtype, B, H, N, d, _ptr(_strides(strides)), axis,
                                    int(bool(rotate)), _ptr(qa), qa.size, _ptr(hd), nh, _ptr(sse),
                                    nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_scale_sweep rejected its arguments")
    return sse


def p_diagnostics(q_bits, k_bits, dtype, B, H, N, d, *, causal=False, rotate=True, rule=RULE_UOS,
                  gamma=1.0, rows=None, strides=None, amb_delta=0.0, nthreads=None):
    """Row-sum diagnostics of materialized-P quantization (see oracle.h).
    Returns (diag float64 [B,H,R,6], amb float64 [B,H,R])."""
    for a in (q_bits, k_bits):
        assert np.asarray(a).dtype == np.uint16
    rows_a = None if rows is None else np.ascontiguousarray(np.asarray(rows, dtype=np.int32))
    R = N if rows_a is None else rows_a.size
    cfg = AttnCfg(B, H, N, d, dtype, int(bool(causal)), int(bool(rotate)), 1, rule, P_POSTNORM, 128,
                  nthreads or default_threads(), 0.0, float(amb_delta), 0)
    diag = np.empty((B, H, R, 6), np.float64)
    amb = np.empty((B, H, R), np.float64)
    st = _strides(strides)
    qa, ka = np.asarray(q_bits), np.asarray(k_bits)
    if st is None:
        qa, ka = np.ascontiguousarray(qa), np.ascontiguousarray(ka)
    rc = _load().oracle_p_diagnostics(ctypes.byref(cfg), _ptr(qa), _ptr(ka), _ptr(st), _ptr(rows_a), R,
                                      float(gamma), _ptr(diag), _ptr(amb))
    if rc != 0:
        raise ValueError("oracle_p_diagnostics rejected its arguments")
    return diag, amb


def attention(q_bits, k_bits, v_bits, dtype, B, H, N, d, *, causal=False, rotate=True,
              quant=True, rule=RULE_UOS, p_mode=P_PNQ, kv_tile=128, rows=None, strides=None,
              q=0.0, amb_delta=0.0, nthreads=None, Nk=None):
    """Attention forward for the listed query rows of every head.  ``Nk`` is
    the number of key/value tokens (cross-attention; default N).

    Returns a dict with ``out`` [B,H,R,d], ``m``, ``l``, ``rowsum`` [B,H,R], ``amb``
    and ``absmass`` [B,H,R,d], ``amb_rowsum`` [B,H,R] (all float64), R = len(rows) or N.
    """
    for a in (q_bits, k_bits, v_bits):
        assert np.asarray(a).dtype == np.uint16
    rows_a = None if rows is None else np.ascontiguousarray(np.asarray(rows, dtype=np.int32))
    R = N if rows_a is None else rows_a.size
    cfg = AttnCfg(B, H, N, d, dtype, int(bool(causal)), int(bool(rotate)), int(bool(quant)), rule,
                  p_mode, kv_tile, nthreads or default_threads(), float(q), float(amb_delta),
                  0 if Nk is None else int(Nk))
    out = np.empty((B, H, R, d), np.float64)
    m = np.empty((B, H, R), np.float64)
    l = np.empty((B, H, R), np.float64)
    rs = np.empty((B, H, R), np.float64)
    amb = np.empty((B, H, R, d), np.float64)
    absm = np.empty((B, H, R, d), np.float64)
    ars = np.empty((B, H, R), np.float64)
    st = _strides(strides)
    qa, ka, va = (np.asarray(a) for a in (q_bits, k_bits, v_bits))
    if st is None:
        qa, ka, va = (np.ascontiguousarray(a) for a in (qa, ka, va))
    rc = _load().oracle_attention(ctypes.byref(cfg), _ptr(qa), _ptr(ka), _ptr(va), _ptr(st),
                                  _ptr(rows_a), R, _ptr(out), _ptr(m), _ptr(l), _ptr(rs), _ptr(amb),
                                  _ptr(absm), _ptr(ars))
    if rc != 0:
        raise ValueError("oracle_attention rejected its arguments")
    return {"out": out, "m": m, "l": l, "rowsum": rs, "amb": amb, "absmass": absm, "amb_rowsum": ars}
