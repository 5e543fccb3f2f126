"""Python binding of libmxattn (include/mxattn.h): MXAttention's MXFP4
attention forward on AMD Instinct MI355X (gfx950).

Argument marshalling only.  Every step of the path runs in the HIP kernels of
libmxattn.so; PyTorch provides device memory and the stream.  Importing the
package does not need a GPU; calling into the library without the built
shared library raises immediately (there is no fallback path).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmxattn.so")

# enums of include/mxattn.h
OK = 0
BF16, FP16 = 0, 1
AXIS_HEAD_DIM, AXIS_TOKEN = 0, 1
SCALE_UOS, SCALE_OCP, SCALE_CEIL_Q = 0, 1, 2
P_PNQ, P_DIRECT, P_POSTNORM = 0, 1, 2
TOKEN_ALIGN = 128
SWEEP_MAX = 48
SWEEP_SCRATCH_BYTES = 16 << 20  # MXATTN_SWEEP_SCRATCH_BYTES

EXPORTED = (
    "mxattn_mx_codes_bytes",
    "mxattn_mx_scales_bytes",
    "mxattn_forward_kv_tile",
    "mxattn_rotate_quantize",
    "mxattn_rotate_quantize_q",
    "mxattn_rotate_quantize_qkv",
    "mxattn_scale_sweep_workspace_bytes",
    "mxattn_scale_sweep",
    "mxattn_scale_sweep_noalloc",
    "mxattn_forward",
    "mxattn_forward_fused_q",
    "mxattn_reference_modes_workspace_bytes",
    "mxattn_quantize_reference_modes",
    "mxattn_p_diagnostics_workspace_bytes",
    "mxattn_p_diagnostics",
    "mxattn_status_string",
)


class Shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("N", ctypes.c_int32),
                ("d", ctypes.c_int32)]


class MXTensorDesc(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("shape", Shape),
                ("axis", ctypes.c_int32), ("rule", ctypes.c_int32), ("rotated", ctypes.c_int32)]


class MXAttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_string(status)} (status {status})")
        self.status = status


_lib = None


def lib():
    """The loaded libmxattn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m mxfp4_microscaled_bit_amd.build` (or __graft_entry__.build())")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    L.mxattn_mx_codes_bytes.restype = sz
    L.mxattn_mx_codes_bytes.argtypes = [Shape, i32]
    L.mxattn_mx_scales_bytes.restype = sz
    L.mxattn_mx_scales_bytes.argtypes = [Shape, i32]
    L.mxattn_forward_kv_tile.restype = i32
    L.mxattn_forward_kv_tile.argtypes = [i32, i32]
    L.mxattn_rotate_quantize.restype = i32
    L.mxattn_rotate_quantize.argtypes = [vp, i32, Shape, vp, i32, i32, i32,
                                         ctypes.POINTER(MXTensorDesc), vp]
    L.mxattn_rotate_quantize_q.restype = i32
    L.mxattn_rotate_quantize_q.argtypes = [vp, i32, Shape, vp, i32, i32, ctypes.c_double,
                                           ctypes.POINTER(MXTensorDesc), vp]
    L.mxattn_rotate_quantize_qkv.restype = i32
    L.mxattn_rotate_quantize_qkv.argtypes = [vp, vp, vp, i32, Shape, Shape, vp, vp, vp, i32, i32,
                                             ctypes.POINTER(MXTensorDesc), ctypes.POINTER(MXTensorDesc),
                                             ctypes.POINTER(MXTensorDesc), vp]
    L.mxattn_scale_sweep_workspace_bytes.restype = sz
    L.mxattn_scale_sweep_workspace_bytes.argtypes = [Shape, i32, i32]
    L.mxattn_scale_sweep.restype = i32
    L.mxattn_scale_sweep.argtypes = [vp, i32, Shape, vp, i32, i32, vp, i32, vp, vp, sz, vp]
    L.mxattn_scale_sweep_noalloc.restype = i32
    L.mxattn_scale_sweep_noalloc.argtypes = [vp, i32, Shape, vp, i32, i32, vp, i32, vp, vp]
    L.mxattn_forward.restype = i32
    L.mxattn_forward.argtypes = [ctypes.POINTER(MXTensorDesc)] * 3 + [i32, vp, vp, vp]
    L.mxattn_reference_modes_workspace_bytes.restype = sz
    L.mxattn_reference_modes_workspace_bytes.argtypes = [Shape, i32]
    L.mxattn_quantize_reference_modes.restype = i32
    L.mxattn_quantize_reference_modes.argtypes = [vp, vp, vp, i32, Shape, vp, i32, i32, i32, i32,
                                                  vp, vp, vp, sz, vp]
    L.mxattn_p_diagnostics_workspace_bytes.restype = sz
    L.mxattn_p_diagnostics_workspace_bytes.argtypes = [Shape]
    L.mxattn_p_diagnostics.restype = i32
    L.mxattn_p_diagnostics.argtypes = [vp, vp, i32, Shape, vp, i32, i32, i32, ctypes.c_float, vp, vp, sz, vp]
    L.mxattn_forward_fused_q.restype = i32
    L.mxattn_forward_fused_q.argtypes = [vp, i32, Shape, vp, vp, vp, i32, vp, vp, vp]
    L.mxattn_status_string.restype = ctypes.c_char_p
    L.mxattn_status_string.argtypes = [i32]
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().mxattn_status_string(status).decode()


def _check(status: int, where: str):
    if status != OK:
        raise MXAttnError(status, where)


def _shape(B, H, N, d) -> Shape:
    return Shape(int(B), int(H), int(N), int(d))


def mx_codes_bytes(B, H, N, d, axis=AXIS_HEAD_DIM) -> int:
    return lib().mxattn_mx_codes_bytes(_shape(B, H, N, d), axis)


def mx_scales_bytes(B, H, N, d, axis=AXIS_HEAD_DIM) -> int:
    return lib().mxattn_mx_scales_bytes(_shape(B, H, N, d), axis)


def forward_kv_tile(d: int, causal: bool = False) -> int:
    return lib().mxattn_forward_kv_tile(int(d), int(bool(causal)))


def reference_modes_workspace_bytes(B, H, N, d, p_mode) -> int:
    return lib().mxattn_reference_modes_workspace_bytes(_shape(B, H, N, d), p_mode)


def _device(*tensors) -> torch.device:
    """The one device every given tensor lives on.  The library receives raw
    device addresses and launches on the current device, so host tensors and
    tensors of different devices are refused here."""
    dev = None
    for t in tensors:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"libmxattn takes device tensors; got one on {t.device}")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"tensors on {dev} and on {t.device}: all must be on one device")
    return dev


def _stream(stream, dev: torch.device):
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    elif stream.device != dev:
        raise ValueError(f"stream on {stream.device}, tensors on {dev}")
    return ctypes.c_void_p(stream.cuda_stream)


def _buffer(t: torch.Tensor, nbytes: int, what: str):
    """An output or workspace tensor the library writes: contiguous and at
    least nbytes long (the C ABI cannot see buffer lengths)."""
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise ValueError(f"{what} holds {have} bytes; {nbytes} are needed")


def _dtype_enum(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float16:
        return FP16
    raise TypeError(f"inputs must be bfloat16 or float16, got {t.dtype}")


def _strides(x: torch.Tensor):
    if x.dim() != 4:
        raise ValueError("inputs are [B, H, N, d] tensors")
    if x.stride(3) != 1:
        raise ValueError("the d dimension must be contiguous")
    return (ctypes.c_int64 * 3)(*x.stride()[:3])


@dataclass
class MXTensor:
    """A caller-owned MXFP4 tensor: uint8 codes and E8M0 scales on the device."""
    codes: torch.Tensor
    scales: torch.Tensor
    shape: tuple
    axis: int
    rule: int = SCALE_UOS
    rotated: int = 0

    @classmethod
    def empty(cls, B, H, N, d, axis, device="cuda"):
        cb = mx_codes_bytes(B, H, N, d, axis)
        sb = mx_scales_bytes(B, H, N, d, axis)
        if cb == 0 or sb == 0:
            raise ValueError("unsupported MXFP4 tensor shape")
        return cls(torch.empty(cb, dtype=torch.uint8, device=device),
                   torch.empty(sb, dtype=torch.uint8, device=device), (B, H, N, d), axis)

    def desc(self) -> MXTensorDesc:
        """The C descriptor, after checking that codes and scales are
        contiguous device buffers long enough for the shape."""
        _device(self.codes, self.scales)
        _buffer(self.codes, mx_codes_bytes(*self.shape, self.axis), "MXFP4 codes")
        _buffer(self.scales, mx_scales_bytes(*self.shape, self.axis), "MXFP4 scales")
        return MXTensorDesc(self.codes.data_ptr(), self.scales.data_ptr(), _shape(*self.shape),
                            self.axis, self.rule, self.rotated)


def rotate_quantize(x: torch.Tensor, axis: int = AXIS_HEAD_DIM, rotate: bool = True,
                    rule: int = SCALE_UOS, out: MXTensor | None = None, stream=None) -> MXTensor:
    """mxattn_rotate_quantize on a [B, H, N, d] bf16/fp16 device tensor."""
    B, H, N, d = x.shape
    dev = _device(x)
    if out is None:
        out = MXTensor.empty(B, H, N, d, axis, device=dev)
    out.shape, out.axis = (B, H, N, d), axis
    _device(x, out.codes, out.scales)
    desc = out.desc()
    with torch.cuda.device(dev):
        _check(lib().mxattn_rotate_quantize(ctypes.c_void_p(x.data_ptr()), _dtype_enum(x), _shape(B, H, N, d),
                                            _strides(x), axis, int(bool(rotate)), rule, ctypes.byref(desc),
                                            _stream(stream, dev)), "mxattn_rotate_quantize")
    out.shape, out.axis, out.rule, out.rotated = (B, H, N, d), axis, rule, int(bool(rotate))
    return out


def rotate_quantize_q(x: torch.Tensor, q_max: float, axis: int = AXIS_HEAD_DIM, rotate: bool = True,
                      out: MXTensor | None = None, stream=None) -> MXTensor:
    """mxattn_rotate_quantize_q: the ceiling rule e = ceil(log2(M / q_max))."""
    B, H, N, d = x.shape
    dev = _device(x)
    if out is None:
        out = MXTensor.empty(B, H, N, d, axis, device=dev)
    out.shape, out.axis = (B, H, N, d), axis
    _device(x, out.codes, out.scales)
    desc = out.desc()
    with torch.cuda.device(dev):
        _check(lib().mxattn_rotate_quantize_q(ctypes.c_void_p(x.data_ptr()), _dtype_enum(x), _shape(B, H, N, d),
                                              _strides(x), axis, int(bool(rotate)), float(q_max),
                                              ctypes.byref(desc), _stream(stream, dev)), "mxattn_rotate_quantize_q")
    out.shape, out.axis, out.rule, out.rotated = (B, H, N, d), axis, SCALE_CEIL_Q, int(bool(rotate))
    return out


def rotate_quantize_qkv(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, rotate: bool = True,
                        rule: int = SCALE_UOS, out: tuple | None = None, stream=None) -> tuple:
    """mxattn_rotate_quantize_qkv: Q and K along d (rotated if `rotate`), V along
    tokens, in one launch; returns the three MXTensors (Q^, K^, V^)."""
    if q.dtype != k.dtype or q.dtype != v.dtype:
        raise TypeError("q, k and v must share one dtype")
    if k.shape != v.shape:
        raise ValueError("k and v must share a shape")
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    dev = _device(q, k, v)
    if out is None:
        out = (MXTensor.empty(B, H, Nq, d, AXIS_HEAD_DIM, device=dev),
               MXTensor.empty(B, H, Nk, d, AXIS_HEAD_DIM, device=dev),
               MXTensor.empty(B, H, Nk, d, AXIS_TOKEN, device=dev))
    oq, ok, ov = out
    oq.shape, oq.axis = (B, H, Nq, d), AXIS_HEAD_DIM
    ok.shape, ok.axis = (B, H, Nk, d), AXIS_HEAD_DIM
    ov.shape, ov.axis = (B, H, Nk, d), AXIS_TOKEN
    _device(q, k, v, oq.codes, oq.scales, ok.codes, ok.scales, ov.codes, ov.scales)
    dq, dk, dv = oq.desc(), ok.desc(), ov.desc()
    with torch.cuda.device(dev):
        _check(lib().mxattn_rotate_quantize_qkv(
            ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()),
            _dtype_enum(q), _shape(B, H, Nq, d), _shape(B, H, Nk, d), _strides(q), _strides(k), _strides(v),
            int(bool(rotate)), rule, ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv), _stream(stream, dev)),
            "mxattn_rotate_quantize_qkv")
    for o in out:
        o.rule = rule
    oq.rotated = ok.rotated = int(bool(rotate))
    ov.rotated = 0
    return out


def scale_sweep_workspace_bytes(B, H, N, d, axis, n_q) -> int:
    return lib().mxattn_scale_sweep_workspace_bytes(_shape(B, H, N, d), axis, int(n_q))


def scale_sweep(x: torch.Tensor, q_values, axis: int = AXIS_HEAD_DIM, rotate: bool = True,
                out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                stream=None) -> torch.Tensor:
    """mxattn_scale_sweep: per-head sum of squared quantization errors for each
    boundary; returns float64 [B*H, len(q_values)] on the device."""
    B, H, N, d = x.shape
    dev = _device(x)
    qs = (ctypes.c_double * len(q_values))(*[float(q) for q in q_values])
    if out is None:
        out = torch.empty((B * H, len(q_values)), dtype=torch.float64, device=dev)
    need = scale_sweep_workspace_bytes(B, H, N, d, axis, len(q_values))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _device(x, out, workspace)
    _buffer(out, B * H * len(q_values) * 8, "out")
    _buffer(workspace, 0, "workspace")
    with torch.cuda.device(dev):
        _check(lib().mxattn_scale_sweep(ctypes.c_void_p(x.data_ptr()), _dtype_enum(x), _shape(B, H, N, d),
                                        _strides(x), axis, int(bool(rotate)), qs, len(q_values),
                                        ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(workspace.data_ptr()),
                                        workspace.numel() * workspace.element_size(), _stream(stream, dev)),
               "mxattn_scale_sweep")
    return out


def scale_sweep_noalloc(x: torch.Tensor, q_values, axis: int = AXIS_HEAD_DIM, rotate: bool = True,
                        out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """mxattn_scale_sweep_noalloc: scale_sweep with the library's static scratch
    in place of a workspace (the library allocates nothing; pass `out` to
    allocate nothing here either).  Returns float64 [B*H, len(q_values)]."""
    B, H, N, d = x.shape
    dev = _device(x)
    qs = (ctypes.c_double * len(q_values))(*[float(q) for q in q_values])
    if out is None:
        out = torch.empty((B * H, len(q_values)), dtype=torch.float64, device=dev)
    _device(x, out)
    _buffer(out, B * H * len(q_values) * 8, "out")
    with torch.cuda.device(dev):
        _check(lib().mxattn_scale_sweep_noalloc(ctypes.c_void_p(x.data_ptr()), _dtype_enum(x), _shape(B, H, N, d),
                                                _strides(x), axis, int(bool(rotate)), qs, len(q_values),
                                                ctypes.c_void_p(out.data_ptr()), _stream(stream, dev)),
               "mxattn_scale_sweep_noalloc")
    return out


def forward(q: MXTensor, k: MXTensor, v: MXTensor, causal: bool = False, out: torch.Tensor | None = None,
            row_stats: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """mxattn_forward; returns O as float32 [B, H, Nq, d] (Nq = q's tokens; k and v
    may hold another token count: cross-attention)."""
    B, H, N, d = q.shape
    if out is None:
        out = torch.empty((B, H, N, d), dtype=torch.float32, device=q.codes.device)
    if out.dtype != torch.float32 or not out.is_contiguous() or tuple(out.shape) != (B, H, N, d):
        raise ValueError("out must be a contiguous float32 [B, H, N, d] tensor")
    if row_stats is not None and (row_stats.dtype != torch.float32 or not row_stats.is_contiguous()
                                  or row_stats.numel() != B * H * N * 2):
        raise ValueError("row_stats must be a contiguous float32 [B, H, N, 2] tensor")
    dev = _device(q.codes, q.scales, k.codes, k.scales, v.codes, v.scales, out, row_stats)
    dq, dk, dv = q.desc(), k.desc(), v.desc()
    with torch.cuda.device(dev):
        _check(lib().mxattn_forward(ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv), int(bool(causal)),
                                    ctypes.c_void_p(out.data_ptr()),
                                    None if row_stats is None else ctypes.c_void_p(row_stats.data_ptr()),
                                    _stream(stream, dev)), "mxattn_forward")
    return out


def forward_fused_q(q: torch.Tensor, k: MXTensor, v: MXTensor, causal: bool = False,
                    out: torch.Tensor | None = None, row_stats: torch.Tensor | None = None,
                    stream=None) -> torch.Tensor:
    """mxattn_forward_fused_q: Q is a 16-bit [B, H, Nq, d] tensor, rotated (if k
    is) and quantized with k's rule inside the forward; returns O as float32
    [B, H, Nq, d]."""
    B, H, N, d = q.shape
    if out is None:
        out = torch.empty((B, H, N, d), dtype=torch.float32, device=q.device)
    if out.dtype != torch.float32 or not out.is_contiguous() or tuple(out.shape) != (B, H, N, d):
        raise ValueError("out must be a contiguous float32 [B, H, N, d] tensor")
    if row_stats is not None and (row_stats.dtype != torch.float32 or not row_stats.is_contiguous()
                                  or row_stats.numel() != B * H * N * 2):
        raise ValueError("row_stats must be a contiguous float32 [B, H, N, 2] tensor")
    dev = _device(q, k.codes, k.scales, v.codes, v.scales, out, row_stats)
    dk, dv = k.desc(), v.desc()
    with torch.cuda.device(dev):
        _check(lib().mxattn_forward_fused_q(
            ctypes.c_void_p(q.data_ptr()), _dtype_enum(q), _shape(B, H, N, d), _strides(q), ctypes.byref(dk),
            ctypes.byref(dv), int(bool(causal)), ctypes.c_void_p(out.data_ptr()),
            None if row_stats is None else ctypes.c_void_p(row_stats.data_ptr()), _stream(stream, dev)),
            "mxattn_forward_fused_q")
    return out


def quantize_reference_modes(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, rule: int = SCALE_UOS,
                             p_mode: int = P_PNQ, rotate: bool = True, causal: bool = False,
                             out: torch.Tensor | None = None, row_sums: torch.Tensor | None = None,
                             workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """mxattn_quantize_reference_modes; returns O as float32 [B, H, N, d]."""
    if q.shape != k.shape or q.shape != v.shape or q.dtype != k.dtype or q.dtype != v.dtype:
        raise ValueError("q, k, v must share shape and dtype")
    if q.stride() != k.stride() or q.stride() != v.stride():
        raise ValueError("q, k, v must share strides")
    B, H, N, d = q.shape
    dev = _device(q, k, v)
    if out is None:
        out = torch.empty((B, H, N, d), dtype=torch.float32, device=dev)
    need = reference_modes_workspace_bytes(B, H, N, d, p_mode)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _device(q, k, v, out, row_sums, workspace)
    _buffer(out, B * H * N * d * 4, "out")
    if row_sums is not None:
        _buffer(row_sums, B * H * N * 4, "row_sums")
    _buffer(workspace, 0, "workspace")
    with torch.cuda.device(dev):
        _check(lib().mxattn_quantize_reference_modes(
            ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()),
            _dtype_enum(q), _shape(B, H, N, d), _strides(q), rule, p_mode, int(bool(rotate)), int(bool(causal)),
            ctypes.c_void_p(out.data_ptr()), None if row_sums is None else ctypes.c_void_p(row_sums.data_ptr()),
            ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size(),
            _stream(stream, dev)), "mxattn_quantize_reference_modes")
    return out


def p_diagnostics_workspace_bytes(B, H, N, d) -> int:
    return lib().mxattn_p_diagnostics_workspace_bytes(_shape(B, H, N, d))


def p_diagnostics(q: torch.Tensor, k: torch.Tensor, rule: int = SCALE_UOS, rotate: bool = True,
                  causal: bool = False, gamma: float = 1.0, out: torch.Tensor | None = None,
                  workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """mxattn_p_diagnostics; returns float32 [B, H, N, 6]: row sum, zeroing,
    saturation, downward, upward rounding contributions, entropy (nats)."""
    if q.shape != k.shape or q.dtype != k.dtype or q.stride() != k.stride():
        raise ValueError("q and k must share shape, dtype and strides")
    B, H, N, d = q.shape
    dev = _device(q, k)
    if out is None:
        out = torch.empty((B, H, N, 6), dtype=torch.float32, device=dev)
    need = p_diagnostics_workspace_bytes(B, H, N, d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _device(q, k, out, workspace)
    _buffer(out, B * H * N * 6 * 4, "out")
    _buffer(workspace, 0, "workspace")
    with torch.cuda.device(dev):
        _check(lib().mxattn_p_diagnostics(
            ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()), _dtype_enum(q), _shape(B, H, N, d),
            _strides(q), rule, int(bool(rotate)), int(bool(causal)), float(gamma), ctypes.c_void_p(out.data_ptr()),
            ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size(),
            _stream(stream, dev)), "mxattn_p_diagnostics")
    return out


def unpack_headdim(mx: MXTensor):
    """Host-side view of a head-dim MXFP4 tensor: (codes uint8 [B,H,N,d], scales uint8 [B,H,N,d/32]),
    padding rows dropped.  For tests and reporting."""
    B, H, N, d = mx.shape
    Np = (N + TOKEN_ALIGN - 1) // TOKEN_ALIGN * TOKEN_ALIGN
    packed = mx.codes.view(B, H, Np, d // 2).cpu()
    codes = torch.stack([packed & 0xF, packed >> 4], dim=-1).reshape(B, H, Np, d)
    scales = mx.scales.view(B, H, Np, d // 32).cpu()
    return codes[:, :, :N].numpy(), scales[:, :, :N].numpy(), codes[:, :, N:].numpy(), scales[:, :, N:].numpy()


def unpack_tokens(mx: MXTensor):
    """Host-side view of a token-axis MXFP4 tensor: (codes uint8 [B,H,NBp,d,32], scales [B,H,NBp,d])."""
    B, H, N, d = mx.shape
    Np = (N + TOKEN_ALIGN - 1) // TOKEN_ALIGN * TOKEN_ALIGN
    packed = mx.codes.view(B, H, Np // 32, d, 16).cpu()
    codes = torch.stack([packed & 0xF, packed >> 4], dim=-1).reshape(B, H, Np // 32, d, 32)
    return codes.numpy(), mx.scales.view(B, H, Np // 32, d).cpu().numpy()
