"""NVFP4 W4A4 linear layers for MI355X (gfx950).

A thin ctypes binding over ``libnvfp4.so`` (built from ``csrc/`` by
``bit_linear_layer_amd.build``).  Each ``nvfp4_*`` function here has the name
of the C entry point it calls and only marshals arguments: every step of the
computation runs in the library's HIP kernels.  torch supplies device memory
and the current stream.  There is no fallback: if the library is missing or
a call fails, a ``NVFP4Error`` is raised.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

__all__ = [
    "NVFP4Error", "NVFP4Tensor", "load", "lib_path",
    "nvfp4_quantize", "nvfp4_quantize_workspace_bytes", "nvfp4_quantize_noalloc", "nvfp4_gemm",
    "nvfp4_gemm_fused_segments", "nvfp4_silu_mul", "nvfp4_status_string", "nvfp4_version",
    "DecodeWeight", "nvfp4_decode_weight_bytes", "nvfp4_decode_weight_pack", "nvfp4_gemm_decode",
    "nvfp4_linear_decode", "pack_decode", "gemm_decode", "linear_decode",
    "empty_nvfp4", "quantize", "gemm", "gemm_fused_segments", "silu_mul", "workspace_for",
    "DTYPE_BF16", "DTYPE_F32", "SCALE_DYNAMIC", "SCALE_STATIC", "AMAX_PRECOMPUTED", "MAX_SEGMENTS",
]

DTYPE_BF16, DTYPE_F32 = 0, 1
SCALE_DYNAMIC, SCALE_STATIC, AMAX_PRECOMPUTED = 0, 1, 2
MAX_SEGMENTS = 16

lib_path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libnvfp4.so")


class NVFP4Error(RuntimeError):
    pass


class _Tensor(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("global_scale", ctypes.c_void_p), ("rows", ctypes.c_int64),
                ("cols", ctypes.c_int64), ("ld_codes", ctypes.c_int64),
                ("ld_scales", ctypes.c_int64)]


class _Gate(ctypes.Structure):
    _fields_ = [("b_segment", ctypes.c_int), ("a_segment", ctypes.c_int),
                ("A_log", ctypes.c_void_p), ("dt_bias", ctypes.c_void_p)]


class _DecodeWeight(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64)]


class _GdnInputs(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("ld_q", ctypes.c_int64), ("k", ctypes.c_void_p), ("ld_k", ctypes.c_int64),
                ("v", ctypes.c_void_p), ("ld_v", ctypes.c_int64), ("beta", ctypes.c_void_p),
                ("ld_beta", ctypes.c_int64), ("g", ctypes.c_void_p), ("ld_g", ctypes.c_int64)]


_lib = None
_P = ctypes.c_void_p
_I64 = ctypes.c_int64


def load() -> ctypes.CDLL:
    """Load libnvfp4.so (once).  Raises NVFP4Error if it was not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(lib_path):
            raise NVFP4Error(f"{lib_path} is missing: build it with "
                             "`python -m bit_linear_layer_amd.build` (no fallback exists)")
        lib = ctypes.CDLL(lib_path)
        lib.nvfp4_quantize_workspace_bytes.argtypes = [_I64, _I64]
        lib.nvfp4_quantize_workspace_bytes.restype = ctypes.c_size_t
        lib.nvfp4_quantize.argtypes = [_P, ctypes.c_int, _I64, _I64, _I64, _P, _I64, _P, _I64, _P,
                                       ctypes.c_int, _P, ctypes.c_size_t, _P]
        lib.nvfp4_quantize.restype = ctypes.c_int
        lib.nvfp4_quantize_noalloc.argtypes = [_P, ctypes.c_int, _I64, _I64, _I64, _P, _I64, _P, _I64, _P,
                                               ctypes.c_int, _P]
        lib.nvfp4_quantize_noalloc.restype = ctypes.c_int
        lib.nvfp4_gemm.argtypes = [ctypes.POINTER(_Tensor), ctypes.POINTER(_Tensor), _P,
                                   ctypes.c_int, _I64, _P]
        lib.nvfp4_gemm.restype = ctypes.c_int
        lib.nvfp4_gemm_fused_segments.argtypes = [
            ctypes.POINTER(_Tensor), ctypes.POINTER(_Tensor), ctypes.c_int,
            ctypes.POINTER(ctypes.c_int64), _P, ctypes.POINTER(_Gate), _P, ctypes.c_int, _I64, _P]
        lib.nvfp4_gemm_fused_segments.restype = ctypes.c_int
        lib.nvfp4_decode_weight_bytes.argtypes = [_I64, _I64]
        lib.nvfp4_decode_weight_bytes.restype = ctypes.c_size_t
        lib.nvfp4_decode_weight_pack.argtypes = [ctypes.POINTER(_Tensor), _P, ctypes.c_size_t, _P]
        lib.nvfp4_decode_weight_pack.restype = ctypes.c_int
        lib.nvfp4_gemm_decode.argtypes = [
            ctypes.POINTER(_Tensor), ctypes.POINTER(_DecodeWeight), ctypes.c_int,
            ctypes.POINTER(ctypes.c_int64), _P, ctypes.POINTER(_Gate), _P, ctypes.c_int, _I64, _P]
        lib.nvfp4_gemm_decode.restype = ctypes.c_int
        lib.nvfp4_linear_decode.argtypes = [
            _P, ctypes.c_int, _I64, _I64, _P, ctypes.POINTER(_DecodeWeight), ctypes.c_int,
            ctypes.POINTER(ctypes.c_int64), _P, ctypes.POINTER(_Gate), _P, ctypes.c_int, _I64, _P]
        lib.nvfp4_linear_decode.restype = ctypes.c_int
        lib.nvfp4_silu_mul.argtypes = [_P, _I64, _I64, _I64, _P, _I64, _P, ctypes.c_size_t, _P]
        lib.nvfp4_silu_mul.restype = ctypes.c_int
        lib.nvfp4_gemm_swiglu.argtypes = [ctypes.POINTER(_Tensor), ctypes.POINTER(_Tensor), _P, _P, _I64,
                                          _P, ctypes.c_size_t, ctypes.POINTER(_Tensor), _P]
        lib.nvfp4_gemm_swiglu.restype = ctypes.c_int
        lib.nvfp4_kv_fp8_calibrate.argtypes = [_P, ctypes.c_int, _I64, _I64, _I64, _P, _P, ctypes.c_size_t, _P]
        lib.nvfp4_kv_fp8_calibrate.restype = ctypes.c_int
        lib.nvfp4_kv_fp8_quantize.argtypes = [_P, ctypes.c_int, _I64, _I64, _I64, _P, _I64, _P, _I64, _P, _P]
        lib.nvfp4_kv_fp8_quantize.restype = ctypes.c_int
        lib.nvfp4_kv_fp8_dequantize.argtypes = [_P, _I64, _I64, _I64, _P, _P, ctypes.c_int, _I64, _P]
        lib.nvfp4_kv_fp8_dequantize.restype = ctypes.c_int
        lib.nvfp4_harmonize_scales.argtypes = [ctypes.POINTER(_Tensor), ctypes.c_int, ctypes.POINTER(ctypes.c_int64),
                                               _P, _P, _I64, _P, _P]
        lib.nvfp4_harmonize_scales.restype = ctypes.c_int
        lib.nvfp4_gdn_workspace_bytes.argtypes = [_I64, ctypes.c_int]
        lib.nvfp4_gdn_workspace_bytes.restype = ctypes.c_size_t
        lib.nvfp4_gdn_recurrence.argtypes = [ctypes.POINTER(_GdnInputs), ctypes.c_int, _I64, ctypes.c_int, ctypes.c_int,
                                             ctypes.c_int, _P, _P, _P, ctypes.c_int, _I64, _P, ctypes.c_size_t, _P]
        lib.nvfp4_gdn_recurrence.restype = ctypes.c_int
        lib.nvfp4_status_string.argtypes = [ctypes.c_int]
        lib.nvfp4_status_string.restype = ctypes.c_char_p
        lib.nvfp4_version.argtypes = []
        lib.nvfp4_version.restype = ctypes.c_int
        _lib = lib
    return _lib


def nvfp4_status_string(status: int) -> str:
    return load().nvfp4_status_string(status).decode()


def nvfp4_version() -> int:
    return load().nvfp4_version()


def _check(status: int, what: str) -> None:
    if status != 0:
        raise NVFP4Error(f"{what} failed: {nvfp4_status_string(status)} (status {status})")


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(device: torch.device, stream=None) -> int:
    if stream is not None:
        return int(stream.cuda_stream if hasattr(stream, "cuda_stream") else stream)
    return torch.cuda.current_stream(device).cuda_stream


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype == torch.float32:
        return DTYPE_F32
    raise NVFP4Error(f"unsupported dtype {t.dtype}")


def _round_up(v: int, a: int) -> int:
    return (v + a - 1) // a * a


def _check_dense(t: torch.Tensor, rows: int, cols: int, device, what: str) -> None:
    """A caller-supplied dense output or input: [rows, cols], contiguous rows
    (any row stride), on the operands' device."""
    if t.dim() != 2 or tuple(t.shape) != (rows, cols):
        raise NVFP4Error(f"{what} must have shape ({rows}, {cols}), got {tuple(t.shape)}")
    if t.stride(1) != 1 or (rows > 1 and t.stride(0) < cols):
        raise NVFP4Error(f"{what} must have contiguous rows")
    if not t.is_cuda or t.device != torch.device(device):
        raise NVFP4Error(f"{what} must live on {device}, got {t.device}")


def _check_nvfp4(q: "NVFP4Tensor", rows: int, cols: int, device, what: str) -> None:
    """An NVFP4 operand or output of [rows, cols] with room for its codes and scales."""
    if q.rows != rows or q.cols != cols:
        raise NVFP4Error(f"{what} is [{q.rows}, {q.cols}], expected [{rows}, {cols}]")
    for name, t, need in (("codes", q.codes, cols // 2), ("scales", q.scales, cols // 16)):
        if t.dim() != 2 or t.shape[0] < rows or t.shape[1] < need or t.stride(1) != 1 or t.dtype != torch.uint8:
            raise NVFP4Error(f"{what}.{name} must be uint8 [>= {rows}, >= {need}] with contiguous rows")
        if not t.is_cuda or t.device != torch.device(device):
            raise NVFP4Error(f"{what}.{name} must live on {device}, got {t.device}")


@dataclass
class NVFP4Tensor:
    """An NVFP4 matrix [rows, cols] in device memory: codes uint8
    [rows, ld_codes] (two per byte, even element low), scales uint8
    [rows, ld_scales] (E4M3 per 16 elements), global_scale float32 [1]."""
    codes: torch.Tensor
    scales: torch.Tensor
    global_scale: torch.Tensor
    rows: int
    cols: int

    def descriptor(self) -> _Tensor:
        return _Tensor(self.codes.data_ptr(), self.scales.data_ptr(), self.global_scale.data_ptr(),
                       self.rows, self.cols, self.codes.stride(0), self.scales.stride(0))

    def row_slice(self, r0: int, r1: int) -> "NVFP4Tensor":
        return NVFP4Tensor(self.codes[r0:r1], self.scales[r0:r1], self.global_scale, r1 - r0, self.cols)


def empty_nvfp4(rows: int, cols: int, device="cuda") -> NVFP4Tensor:
    """Allocate an NVFP4 matrix with the row strides the kernels want: code
    and scale rows on 16-byte boundaries."""
    ldc = _round_up(max(cols // 2, 1), 16)
    lds = _round_up(max(cols // 16, 1), 16)  # 16-byte rows also suit the decode path's copies
    codes = torch.empty((rows, ldc), dtype=torch.uint8, device=device)
    scales = torch.empty((rows, lds), dtype=torch.uint8, device=device)
    g = torch.empty(1, dtype=torch.float32, device=device)
    return NVFP4Tensor(codes, scales, g, rows, cols)


def nvfp4_quantize_workspace_bytes(rows: int, cols: int) -> int:
    return int(load().nvfp4_quantize_workspace_bytes(rows, cols))


def workspace_for(rows: int, cols: int, device="cuda") -> torch.Tensor:
    return torch.empty(nvfp4_quantize_workspace_bytes(rows, cols) // 4, dtype=torch.float32, device=device)


def nvfp4_quantize(x: torch.Tensor, q: NVFP4Tensor, flags: int = SCALE_DYNAMIC,
                   workspace: torch.Tensor | None = None, stream=None) -> None:
    """C ``nvfp4_quantize`` on a 2-D bf16/float32 tensor x (rows may be
    strided) into the preallocated ``q``."""
    if x.dim() != 2 or x.stride(1) != 1:
        raise NVFP4Error("x must be a 2-D tensor with contiguous rows")
    _check_nvfp4(q, x.shape[0], x.shape[1], x.device, "q")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load().nvfp4_quantize(
        x.data_ptr(), _dtype_code(x), x.shape[0], x.shape[1], x.stride(0),
        q.codes.data_ptr(), q.codes.stride(0), q.scales.data_ptr(), q.scales.stride(0),
        q.global_scale.data_ptr(), flags, _ptr(workspace), ws_bytes, _stream(x.device, stream))
    _check(st, "nvfp4_quantize")


def nvfp4_quantize_noalloc(x: torch.Tensor, q: NVFP4Tensor, flags: int = SCALE_DYNAMIC, stream=None) -> None:
    """C ``nvfp4_quantize_noalloc``: ``nvfp4_quantize`` without a workspace
    (the library's static per-GPU scratch holds the amax partials)."""
    if x.dim() != 2 or x.stride(1) != 1:
        raise NVFP4Error("x must be a 2-D tensor with contiguous rows")
    _check_nvfp4(q, x.shape[0], x.shape[1], x.device, "q")
    st = load().nvfp4_quantize_noalloc(
        x.data_ptr(), _dtype_code(x), x.shape[0], x.shape[1], x.stride(0),
        q.codes.data_ptr(), q.codes.stride(0), q.scales.data_ptr(), q.scales.stride(0),
        q.global_scale.data_ptr(), flags, _stream(x.device, stream))
    _check(st, "nvfp4_quantize_noalloc")


def nvfp4_gemm(a: NVFP4Tensor, w: NVFP4Tensor, out: torch.Tensor, stream=None) -> None:
    """C ``nvfp4_gemm``: out[M, N] = A W^T with both global scales."""
    _check_dense(out, a.rows, w.rows, a.codes.device, "out")
    da, dw = a.descriptor(), w.descriptor()
    st = load().nvfp4_gemm(ctypes.byref(da), ctypes.byref(dw), out.data_ptr(), _dtype_code(out),
                           out.stride(0), _stream(out.device, stream))
    _check(st, "nvfp4_gemm")


def nvfp4_gemm_fused_segments(a: NVFP4Tensor, w: NVFP4Tensor, seg_offsets, seg_global_scales: torch.Tensor,
                              out: torch.Tensor, gate: dict | None = None, stream=None) -> None:
    """C ``nvfp4_gemm_fused_segments``.  seg_offsets: host ints [n+1];
    seg_global_scales: device float32 [n]; gate: None or dict(b_segment,
    a_segment, A_log, dt_bias) with device float32 tensors."""
    _check_dense(out, a.rows, w.rows, a.codes.device, "out")
    offs = (ctypes.c_int64 * len(seg_offsets))(*[int(o) for o in seg_offsets])
    g = _gate(gate)
    da, dw = a.descriptor(), w.descriptor()
    st = load().nvfp4_gemm_fused_segments(
        ctypes.byref(da), ctypes.byref(dw), len(seg_offsets) - 1, offs, seg_global_scales.data_ptr(),
        None if g is None else ctypes.byref(g), out.data_ptr(), _dtype_code(out), out.stride(0),
        _stream(out.device, stream))
    _check(st, "nvfp4_gemm_fused_segments")


def _gate(gate: dict | None):
    if gate is None:
        return None
    return _Gate(int(gate.get("b_segment", -1)), int(gate.get("a_segment", -1)),
                 _ptr(gate.get("A_log")), _ptr(gate.get("dt_bias")))


@dataclass
class DecodeWeight:
    """A weight [rows, cols] in the decode layout (``nvfp4_decode_weight_pack``):
    ``data`` is a uint8 device tensor of ``nvfp4_decode_weight_bytes`` bytes."""
    data: torch.Tensor
    rows: int
    cols: int

    def descriptor(self) -> _DecodeWeight:
        return _DecodeWeight(self.data.data_ptr(), self.rows, self.cols)


def nvfp4_decode_weight_bytes(rows: int, cols: int) -> int:
    return int(load().nvfp4_decode_weight_bytes(rows, cols))


def nvfp4_decode_weight_pack(w: NVFP4Tensor, packed: torch.Tensor, stream=None) -> None:
    """C ``nvfp4_decode_weight_pack``: w (row-major NVFP4) into the decode layout."""
    dw = w.descriptor()
    st = load().nvfp4_decode_weight_pack(ctypes.byref(dw), packed.data_ptr(), packed.numel() * packed.element_size(),
                                         _stream(w.codes.device, stream))
    _check(st, "nvfp4_decode_weight_pack")


def nvfp4_gemm_decode(a: NVFP4Tensor, w: DecodeWeight, seg_offsets, seg_global_scales: torch.Tensor,
                      out: torch.Tensor, gate: dict | None = None, stream=None) -> None:
    """C ``nvfp4_gemm_decode``: ``nvfp4_gemm_fused_segments`` for a packed
    weight and at most 16 activation rows."""
    _check_dense(out, a.rows, w.rows, a.codes.device, "out")
    offs = (ctypes.c_int64 * len(seg_offsets))(*[int(o) for o in seg_offsets])
    g = _gate(gate)
    da, dw = a.descriptor(), w.descriptor()
    st = load().nvfp4_gemm_decode(ctypes.byref(da), ctypes.byref(dw), len(seg_offsets) - 1, offs,
                                  seg_global_scales.data_ptr(), None if g is None else ctypes.byref(g),
                                  out.data_ptr(), _dtype_code(out), out.stride(0), _stream(out.device, stream))
    _check(st, "nvfp4_gemm_decode")


def nvfp4_linear_decode(x: torch.Tensor, w: DecodeWeight, seg_offsets, seg_global_scales: torch.Tensor,
                        out: torch.Tensor, x_global_scale: torch.Tensor | None = None, gate: dict | None = None,
                        stream=None) -> None:
    """C ``nvfp4_linear_decode``: dense x (<= 16 rows) quantized inside the
    launch, then the packed-weight GEMM."""
    if x.dim() != 2 or x.stride(1) != 1 or x.shape[1] != w.cols:
        raise NVFP4Error(f"x must be [rows, {w.cols}] with contiguous rows")
    _check_dense(out, x.shape[0], w.rows, x.device, "out")
    offs = (ctypes.c_int64 * len(seg_offsets))(*[int(o) for o in seg_offsets])
    g = _gate(gate)
    dw = w.descriptor()
    st = load().nvfp4_linear_decode(x.data_ptr(), _dtype_code(x), x.shape[0], x.stride(0), _ptr(x_global_scale),
                                    ctypes.byref(dw), len(seg_offsets) - 1, offs, seg_global_scales.data_ptr(),
                                    None if g is None else ctypes.byref(g), out.data_ptr(), _dtype_code(out),
                                    out.stride(0), _stream(out.device, stream))
    _check(st, "nvfp4_linear_decode")


def nvfp4_silu_mul(gu: torch.Tensor, h: torch.Tensor, inter: int, amax_workspace: torch.Tensor | None = None,
                   stream=None) -> None:
    """C ``nvfp4_silu_mul``: h = bf16(silu(gu[:, :inter]) * gu[:, inter:2*inter])."""
    if gu.dim() != 2 or gu.stride(1) != 1 or gu.shape[1] < 2 * inter:
        raise NVFP4Error(f"gu must be [rows, >= {2 * inter}] with contiguous rows")
    _check_dense(h, gu.shape[0], inter, gu.device, "h")
    ws_bytes = 0 if amax_workspace is None else amax_workspace.numel() * amax_workspace.element_size()
    st = load().nvfp4_silu_mul(gu.data_ptr(), gu.shape[0], inter, gu.stride(0), h.data_ptr(), h.stride(0),
                               _ptr(amax_workspace), ws_bytes, _stream(gu.device, stream))
    _check(st, "nvfp4_silu_mul")


def nvfp4_gemm_swiglu(a: NVFP4Tensor, w_gate_up: NVFP4Tensor, seg_global_scales: torch.Tensor,
                      h: torch.Tensor | None = None, amax_workspace: torch.Tensor | None = None,
                      h_q: NVFP4Tensor | None = None, stream=None) -> None:
    """C ``nvfp4_gemm_swiglu``: h = bf16(silu(gate) * up) from one GEMM over
    w_gate_up = [gate; up] (2 segments), written as bf16 ``h`` and/or as
    NVFP4 ``h_q`` quantized with the static scale already in h_q.global_scale."""
    inter = w_gate_up.rows // 2
    if h is not None:
        _check_dense(h, a.rows, inter, a.codes.device, "h")
    if h_q is not None:
        _check_nvfp4(h_q, a.rows, inter, a.codes.device, "h_q")
    ws_bytes = 0 if amax_workspace is None else amax_workspace.numel() * amax_workspace.element_size()
    da, dw = a.descriptor(), w_gate_up.descriptor()
    dq = None if h_q is None else h_q.descriptor()
    st = load().nvfp4_gemm_swiglu(
        ctypes.byref(da), ctypes.byref(dw), seg_global_scales.data_ptr(), _ptr(h),
        0 if h is None else h.stride(0), _ptr(amax_workspace), ws_bytes,
        None if dq is None else ctypes.byref(dq), _stream(a.codes.device, stream))
    _check(st, "nvfp4_gemm_swiglu")


def nvfp4_kv_fp8_calibrate(x: torch.Tensor, scale: torch.Tensor, workspace: torch.Tensor | None = None,
                           stream=None) -> None:
    """C ``nvfp4_kv_fp8_calibrate``: scale[0] = fl32(max|x| / 448)."""
    ws = workspace if workspace is not None else workspace_for(x.shape[0], x.shape[1], x.device)
    st = load().nvfp4_kv_fp8_calibrate(x.data_ptr(), _dtype_code(x), x.shape[0], x.shape[1], x.stride(0),
                                       scale.data_ptr(), ws.data_ptr(), ws.numel() * ws.element_size(),
                                       _stream(x.device, stream))
    _check(st, "nvfp4_kv_fp8_calibrate")


def nvfp4_kv_fp8_quantize(x: torch.Tensor, cache: torch.Tensor, scale: torch.Tensor,
                          slots: torch.Tensor | None = None, stream=None) -> None:
    """C ``nvfp4_kv_fp8_quantize``: E4M3 bytes of x / scale into cache rows
    ``slots`` (int64 device tensor) or rows 0..len(x)-1."""
    if x.dim() != 2 or x.stride(1) != 1 or cache.dim() != 2 or cache.stride(1) != 1:
        raise NVFP4Error("x and cache must be 2-D with contiguous rows")
    if slots is not None and (slots.dtype != torch.int64 or slots.numel() != x.shape[0]):
        raise NVFP4Error("slots must be int64 with one entry per row of x")
    st = load().nvfp4_kv_fp8_quantize(x.data_ptr(), _dtype_code(x), x.shape[0], x.shape[1], x.stride(0),
                                      _ptr(slots), cache.shape[0], cache.data_ptr(), cache.stride(0),
                                      scale.data_ptr(), _stream(x.device, stream))
    _check(st, "nvfp4_kv_fp8_quantize")


def nvfp4_kv_fp8_dequantize(cache: torch.Tensor, scale: torch.Tensor, out: torch.Tensor, cols: int | None = None,
                            stream=None) -> None:
    """C ``nvfp4_kv_fp8_dequantize``: out = fl32(e4m3(cache) * scale) (bf16 out rounds that)."""
    cols = out.shape[1] if cols is None else cols
    st = load().nvfp4_kv_fp8_dequantize(cache.data_ptr(), out.shape[0], cols, cache.stride(0), scale.data_ptr(),
                                        out.data_ptr(), _dtype_code(out), out.stride(0),
                                        _stream(out.device, stream))
    _check(st, "nvfp4_kv_fp8_dequantize")


def nvfp4_harmonize_scales(w: NVFP4Tensor, seg_offsets, seg_global_scales: torch.Tensor,
                           out_scales: torch.Tensor, out_global_scale: torch.Tensor, stream=None) -> None:
    """C ``nvfp4_harmonize_scales``: block scales of every segment rewritten
    for the common global scale max(seg_global_scales) (written to
    out_global_scale); E2M1 codes unchanged."""
    offs = (ctypes.c_int64 * len(seg_offsets))(*[int(o) for o in seg_offsets])
    dw = w.descriptor()
    st = load().nvfp4_harmonize_scales(ctypes.byref(dw), len(seg_offsets) - 1, offs, seg_global_scales.data_ptr(),
                                       out_scales.data_ptr(), out_scales.stride(0), out_global_scale.data_ptr(),
                                       _stream(w.codes.device, stream))
    _check(st, "nvfp4_harmonize_scales")


def nvfp4_gdn_workspace_bytes(tokens: int, v_heads: int) -> int:
    return int(load().nvfp4_gdn_workspace_bytes(tokens, v_heads))


def nvfp4_gdn_recurrence(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, beta: torch.Tensor, g: torch.Tensor,
                         o: torch.Tensor, k_heads: int, v_heads: int, workspace: torch.Tensor,
                         normalize_qk: bool = True, s0: torch.Tensor | None = None,
                         s_final: torch.Tensor | None = None, stream=None) -> None:
    """C ``nvfp4_gdn_recurrence`` on 2-D row-strided views (one dtype for the
    inputs; they may be column slices of one fused in-projection output)."""
    for t in (q, k, v, beta, g, o):
        if t.dim() != 2 or t.stride(1) != 1:
            raise NVFP4Error("inputs and output must be 2-D with contiguous rows")
    dt = _dtype_code(q)
    if any(_dtype_code(t) != dt for t in (k, v, beta, g)):
        raise NVFP4Error("q, k, v, beta and g must share one dtype")
    ins = _GdnInputs(q.data_ptr(), q.stride(0), k.data_ptr(), k.stride(0), v.data_ptr(), v.stride(0),
                     beta.data_ptr(), beta.stride(0), g.data_ptr(), g.stride(0))
    st = load().nvfp4_gdn_recurrence(ctypes.byref(ins), dt, q.shape[0], k_heads, v_heads, int(normalize_qk),
                                     _ptr(s0), _ptr(s_final), o.data_ptr(), _dtype_code(o), o.stride(0),
                                     workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                     _stream(q.device, stream))
    _check(st, "nvfp4_gdn_recurrence")


# ----------------------------------------------------------- conveniences

def quantize(x: torch.Tensor, static_scale: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
             out: NVFP4Tensor | None = None, amax_precomputed: bool = False) -> NVFP4Tensor:
    """Allocate (unless ``out``) and quantize x; dynamic global scale unless
    ``static_scale`` (device float32 [1]) is given."""
    q = out if out is not None else empty_nvfp4(x.shape[0], x.shape[1], x.device)
    if static_scale is not None:
        q.global_scale.copy_(static_scale)
        nvfp4_quantize(x, q, SCALE_STATIC, None)
    else:
        ws = workspace if workspace is not None else workspace_for(x.shape[0], x.shape[1], x.device)
        nvfp4_quantize(x, q, AMAX_PRECOMPUTED if amax_precomputed else SCALE_DYNAMIC, ws)
    return q


def gemm(a: NVFP4Tensor, w: NVFP4Tensor, out_dtype=torch.bfloat16, out: torch.Tensor | None = None) -> torch.Tensor:
    o = out if out is not None else torch.empty((a.rows, w.rows), dtype=out_dtype, device=a.codes.device)
    nvfp4_gemm(a, w, o)
    return o


def gemm_fused_segments(a: NVFP4Tensor, w: NVFP4Tensor, seg_offsets, seg_global_scales: torch.Tensor,
                        gate: dict | None = None, out_dtype=torch.bfloat16, out: torch.Tensor | None = None) -> torch.Tensor:
    o = out if out is not None else torch.empty((a.rows, w.rows), dtype=out_dtype, device=a.codes.device)
    nvfp4_gemm_fused_segments(a, w, seg_offsets, seg_global_scales, o, gate)
    return o


def pack_decode(w: NVFP4Tensor) -> DecodeWeight:
    """The decode-layout copy of an NVFP4 weight (offline, like quantization)."""
    nbytes = nvfp4_decode_weight_bytes(w.rows, w.cols)
    if nbytes == 0:
        raise NVFP4Error(f"a [{w.rows}, {w.cols}] weight has no decode layout (cols <= 8192, % 16)")
    data = torch.empty(nbytes, dtype=torch.uint8, device=w.codes.device)
    nvfp4_decode_weight_pack(w, data)
    return DecodeWeight(data, w.rows, w.cols)


def gemm_decode(a: NVFP4Tensor, w: DecodeWeight, seg_offsets, seg_global_scales: torch.Tensor,
                gate: dict | None = None, out_dtype=torch.bfloat16, out: torch.Tensor | None = None) -> torch.Tensor:
    o = out if out is not None else torch.empty((a.rows, w.rows), dtype=out_dtype, device=a.codes.device)
    nvfp4_gemm_decode(a, w, seg_offsets, seg_global_scales, o, gate)
    return o


def linear_decode(x: torch.Tensor, w: DecodeWeight, seg_offsets, seg_global_scales: torch.Tensor,
                  gate: dict | None = None, out_dtype=torch.bfloat16, out: torch.Tensor | None = None,
                  x_global_scale: torch.Tensor | None = None) -> torch.Tensor:
    o = out if out is not None else torch.empty((x.shape[0], w.rows), dtype=out_dtype, device=x.device)
    nvfp4_linear_decode(x, w, seg_offsets, seg_global_scales, o, x_global_scale, gate)
    return o


def silu_mul(gu: torch.Tensor, amax_workspace: torch.Tensor | None = None, out: torch.Tensor | None = None) -> torch.Tensor:
    inter = gu.shape[1] // 2
    h = out if out is not None else torch.empty((gu.shape[0], inter), dtype=torch.bfloat16, device=gu.device)
    nvfp4_silu_mul(gu, h, inter, amax_workspace)
    return h


def gemm_swiglu(a: NVFP4Tensor, w_gate_up: NVFP4Tensor, seg_global_scales: torch.Tensor,
                amax_workspace: torch.Tensor | None = None, out: torch.Tensor | None = None) -> torch.Tensor:
    """bf16 h [M, inter] of the fused gate_up GEMM + SiLU*mul."""
    inter = w_gate_up.rows // 2
    h = out if out is not None else torch.empty((a.rows, inter), dtype=torch.bfloat16, device=a.codes.device)
    nvfp4_gemm_swiglu(a, w_gate_up, seg_global_scales, h=h, amax_workspace=amax_workspace)
    return h


def gemm_swiglu_quantized(a: NVFP4Tensor, w_gate_up: NVFP4Tensor, seg_global_scales: torch.Tensor,
                          static_scale: torch.Tensor, out: NVFP4Tensor | None = None) -> NVFP4Tensor:
    """NVFP4 h [M, inter] with the calibrated global scale ``static_scale``
    (device float32 [1]), straight from the fused gate_up epilogue."""
    inter = w_gate_up.rows // 2
    q = out if out is not None else empty_nvfp4(a.rows, inter, a.codes.device)
    q.global_scale.copy_(static_scale)
    nvfp4_gemm_swiglu(a, w_gate_up, seg_global_scales, h_q=q)
    return q


def kv_fp8_quantize(x: torch.Tensor, scale: torch.Tensor, cache: torch.Tensor | None = None,
                    slots: torch.Tensor | None = None) -> torch.Tensor:
    """FP8 E4M3 bytes of x with the per-tensor decode scale ``scale``."""
    c = cache if cache is not None else torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    nvfp4_kv_fp8_quantize(x, c, scale, slots)
    return c


def kv_fp8_dequantize(cache: torch.Tensor, scale: torch.Tensor, out_dtype=torch.bfloat16,
                      cols: int | None = None) -> torch.Tensor:
    cols = cache.shape[1] if cols is None else cols
    out = torch.empty((cache.shape[0], cols), dtype=out_dtype, device=cache.device)
    nvfp4_kv_fp8_dequantize(cache, scale, out, cols)
    return out


def kv_fp8_calibrate(x: torch.Tensor) -> torch.Tensor:
    s = torch.empty(1, dtype=torch.float32, device=x.device)
    nvfp4_kv_fp8_calibrate(x, s)
    return s


def harmonize_scales(w: NVFP4Tensor, seg_offsets, seg_global_scales: torch.Tensor) -> NVFP4Tensor:
    """The harmonized weight: w's codes, new block scales, one global scale."""
    scales = torch.empty_like(w.scales)
    g = torch.empty(1, dtype=torch.float32, device=w.codes.device)
    nvfp4_harmonize_scales(w, seg_offsets, seg_global_scales, scales, g)
    return NVFP4Tensor(w.codes, scales, g, w.rows, w.cols)


def gdn_recurrence(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, beta: torch.Tensor, g: torch.Tensor,
                   k_heads: int, v_heads: int, normalize_qk: bool = True, s0: torch.Tensor | None = None,
                   out_dtype=torch.float32, return_state: bool = False):
    """Outputs [tokens, v_heads*128] (and the final states [v_heads, 128, 128])."""
    tokens = q.shape[0]
    ws = torch.empty(nvfp4_gdn_workspace_bytes(tokens, v_heads) // 4, dtype=torch.float32, device=q.device)
    o = torch.empty((tokens, v_heads * 128), dtype=out_dtype, device=q.device)
    sf = torch.empty((v_heads, 128, 128), dtype=torch.float32, device=q.device) if return_state else None
    nvfp4_gdn_recurrence(q, k, v, beta, g, o, k_heads, v_heads, ws, normalize_qk, s0, sf)
    return (o, sf) if return_state else o
