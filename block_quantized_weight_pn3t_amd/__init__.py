"""Python binding of libpn.so (C ABI in include/pn.h): PN (pn3t / pn4t) and NVFP4 W4A16
decode-step GEMV, validation, decode and quantizers on MI355X (gfx950).

Argument marshalling only: every step runs in the HIP kernels of libpn.so. PyTorch supplies device
memory and the current stream. There is no CPU fallback: if the library is missing, importing
this package raises ImportError; if a call fails, it raises PNError.
"""
from __future__ import annotations

import ctypes as C
import os

__all__ = ["PN3T", "PN4T", "PNError", "row_bytes", "validate_rows", "validate_row",
           "dequantize_rows", "dequantize_row", "gemv", "gemv_group", "quantize_rows", "hadamard_rows",
           "gemv_hadamard", "gemv_hadamard_noalloc", "gemv_group_hadamard", "nvfp4_validate_rows",
           "nvfp4_dequantize_rows", "gemv_nvfp4", "fp8row_validate_rows", "fp8row_dequantize_rows", "gemv_fp8row",
           "library_path", "status_string", "lib"]

PN3T = 124
PN4T = 125
GROUP = {PN3T: 80, PN4T: 64}
MAX_TOKENS = 4         # NVFP4 and row-scaled E4M3 GEMV
GEMV_MAX_TOKENS = 16   # PN GEMV
GEMV_HADAMARD_MAX_TOKENS = 4  # PN GEMV with the rotation fused
GEMV_GROUP_MAX_PARTS = 4  # matrices per pn_gemv_group call
NOALLOC_MAX_FLOATS = 262144  # M * K limit of pn_gemv_hadamard_noalloc

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libpn.so")

if not os.path.exists(library_path):
    raise ImportError(f"{library_path} is not built; run __graft_entry__.build() (hipcc, gfx950)")

_lib = C.CDLL(library_path)
_P, _I64, _I32, _F = C.c_void_p, C.c_int64, C.c_int, C.c_float


class GemvPart(C.Structure):
    """pn_gemv_part of include/pn.h: one matrix of a pn_gemv_group call."""
    _fields_ = [("type", C.c_int), ("W", C.c_void_p), ("N", C.c_int64), ("y", C.c_void_p)]


_SIGS = {
    "pn_row_bytes": (_I64, [_I32, _I64]),
    "pn_status_string": (C.c_char_p, [_I32]),
    "pn_validate_rows": (_I32, [_I32, _P, _I64, _I64, _P, _P]),
    "pn_validate_row": (_I32, [_I32, _P, _I64, _P, _P]),
    "pn_dequantize_rows": (_I32, [_I32, _P, _I64, _I64, _P, _P]),
    "pn_dequantize_row": (_I32, [_I32, _P, _I64, _P, _P]),
    "pn_gemv": (_I32, [_I32, _P, _I64, _I64, _P, _I64, _P, _P]),
    "pn_gemv_group": (_I32, [C.POINTER(GemvPart), _I32, _I64, _P, _I64, _P]),
    "pn_gemv_group_hadamard": (_I32, [C.POINTER(GemvPart), _I32, _I64, _P, _I64, _I64, _P]),
    "pn_quantize_rows": (_I32, [_I32, _P, _I64, _I64, _P, _P, _P]),
    "pn_hadamard_rows": (_I32, [_P, _I64, _I64, _I64, _P, _P]),
    "pn_gemv_hadamard": (_I32, [_I32, _P, _I64, _I64, _P, _I64, _I64, _P, _P]),
    "pn_gemv_hadamard_noalloc": (_I32, [_I32, _P, _I64, _I64, _P, _I64, _I64, _P, _P]),
    "pn_nvfp4_validate_rows": (_I32, [_P, _F, _I64, _I64, _P, _P]),
    "pn_nvfp4_dequantize_rows": (_I32, [_P, _P, _F, _I64, _I64, _P, _P]),
    "pn_gemv_nvfp4": (_I32, [_P, _P, _F, _I64, _I64, _P, _I64, _P, _P]),
    "pn_fp8row_validate_rows": (_I32, [_P, _P, _I64, _I64, _P, _P]),
    "pn_fp8row_dequantize_rows": (_I32, [_P, _P, _I64, _I64, _P, _P]),
    "pn_gemv_fp8row": (_I32, [_P, _P, _I64, _I64, _P, _I64, _P, _P]),
}
for _name, (_res, _args) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args


def lib() -> C.CDLL:
    return _lib


class PNError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


def status_string(status: int) -> str:
    return _lib.pn_status_string(status).decode()


def _check(status: int, what: str):
    if status != 0:
        raise PNError(status, what)


def _stream(stream):
    import torch
    if stream is None:
        return C.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return C.c_void_p(stream)
    return C.c_void_p(stream.cuda_stream)


def _ptr(t) -> int:
    return t.data_ptr() if t is not None else 0


def _dev(t, name, dtype=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def row_bytes(type_: int, K: int) -> int:
    return int(_lib.pn_row_bytes(type_, K))


# ---- PN ---------------------------------------------------------------------------------------

def validate_rows(type_, W, nrows, K, verdict, stream=None):
    """verdict (int32[nrows], device) <- 1 valid / 0 invalid per row."""
    import torch
    _dev(verdict, "verdict", torch.int32)
    _check(_lib.pn_validate_rows(type_, _ptr(W), nrows, K, _ptr(verdict), _stream(stream)),
           "pn_validate_rows")


def validate_row(type_, row, K, verdict, stream=None):
    _check(_lib.pn_validate_row(type_, _ptr(row), K, _ptr(verdict), _stream(stream)),
           "pn_validate_row")


def dequantize_rows(type_, W, nrows, K, out, stream=None):
    import torch
    _dev(out, "out", torch.float32)
    _check(_lib.pn_dequantize_rows(type_, _ptr(W), nrows, K, _ptr(out), _stream(stream)),
           "pn_dequantize_rows")


def dequantize_row(type_, row, K, out, stream=None):
    _check(_lib.pn_dequantize_row(type_, _ptr(row), K, _ptr(out), _stream(stream)),
           "pn_dequantize_row")


def gemv(type_, W, N, K, x, y, M=None, stream=None):
    """y[M, N] <- W[N, K] . x[M, K]^T for PN weights W (raw bytes on the device)."""
    import torch
    _dev(x, "x", torch.float32)
    _dev(y, "y", torch.float32)
    if M is None:
        M = 1 if x.dim() == 1 else x.shape[0]
    _check(_lib.pn_gemv(type_, _ptr(W), N, K, _ptr(x), M, _ptr(y), _stream(stream)), "pn_gemv")


def gemv_group(parts, K, x, M=None, stream=None):
    """Several PN GEMVs that share x: parts is a sequence of (type, W, N, y) with W raw PN bytes
    and y fp32[M, N] on the device; every y[M, N] <- W[N, K] . x[M, K]^T, in one launch where the
    shapes allow (pn_gemv_group)."""
    import torch
    _dev(x, "x", torch.float32)
    if M is None:
        M = 1 if x.dim() == 1 else x.shape[0]
    arr = (GemvPart * len(parts))()
    for i, (type_, W, N, y) in enumerate(parts):
        _dev(y, "y", torch.float32)
        arr[i] = GemvPart(type_, _ptr(W), N, _ptr(y))
    _check(_lib.pn_gemv_group(arr, len(parts), K, _ptr(x), M, _stream(stream)), "pn_gemv_group")


def gemv_group_hadamard(parts, K, x, B, M=None, stream=None):
    """gemv_group over x rotated in slices of B (pn_gemv_group_hadamard); x is not modified."""
    import torch
    _dev(x, "x", torch.float32)
    if M is None:
        M = 1 if x.dim() == 1 else x.shape[0]
    arr = (GemvPart * len(parts))()
    for i, (type_, W, N, y) in enumerate(parts):
        _dev(y, "y", torch.float32)
        arr[i] = GemvPart(type_, _ptr(W), N, _ptr(y))
    _check(_lib.pn_gemv_group_hadamard(arr, len(parts), K, _ptr(x), M, B, _stream(stream)),
           "pn_gemv_group_hadamard")


def gemv_group_hadamard_ptr(parts, K, x_ptr, M, B, stream_handle):
    """Raw-pointer form: parts a prepared GemvPart array; returns the status."""
    return _lib.pn_gemv_group_hadamard(parts, len(parts), K, x_ptr, M, B, stream_handle)


def gemv_group_ptr(parts, K, x_ptr, M, stream_handle):
    """Raw-pointer form for timing loops: parts is a sequence of (type, W_ptr, N, y_ptr) or a
    prepared GemvPart array; returns the status instead of raising."""
    if not isinstance(parts, C.Array):
        arr = (GemvPart * len(parts))()
        for i, (type_, W, N, y) in enumerate(parts):
            arr[i] = GemvPart(type_, W, N, y)
        parts = arr
    return _lib.pn_gemv_group(parts, len(parts), K, x_ptr, M, stream_handle)


def gemv_ptr(type_, W_ptr, N, K, x_ptr, M, y_ptr, stream_handle):
    """Raw-pointer form for timing loops: returns the status instead of raising."""
    return _lib.pn_gemv(type_, W_ptr, N, K, x_ptr, M, y_ptr, stream_handle)


def hadamard_rows(x, B, out, M=None, K=None, stream=None):
    """out[M, K] <- x rotated by the orthonormal Walsh-Hadamard matrix on slices of B elements."""
    import torch
    _dev(x, "x", torch.float32)
    _dev(out, "out", torch.float32)
    if M is None:
        M = 1 if x.dim() == 1 else x.shape[0]
    if K is None:
        K = x.shape[-1]
    _check(_lib.pn_hadamard_rows(_ptr(x), M, K, B, _ptr(out), _stream(stream)), "pn_hadamard_rows")


def gemv_hadamard(type_, W, N, K, x, B, y, M=None, stream=None):
    """y[M, N] <- W[N, K] . (H x)[M, K]^T: x rotated into the library's per-device workspace, then
    the GEMV (M <= 4)."""
    import torch
    _dev(x, "x", torch.float32)
    _dev(y, "y", torch.float32)
    if M is None:
        M = 1 if x.dim() == 1 else x.shape[0]
    _check(_lib.pn_gemv_hadamard(type_, _ptr(W), N, K, _ptr(x), M, B, _ptr(y), _stream(stream)),
           "pn_gemv_hadamard")


def gemv_hadamard_noalloc(type_, W, N, K, x, B, y, M=None, stream=None):
    """As gemv_hadamard, with the rotated x in the library's own device array (no allocation;
    M * K <= PN_NOALLOC_MAX_FLOATS; calls that overlap on one GPU race on that array)."""
    import torch
    _dev(x, "x", torch.float32)
    _dev(y, "y", torch.float32)
    if M is None:
        M = 1 if x.dim() == 1 else x.shape[0]
    _check(_lib.pn_gemv_hadamard_noalloc(type_, _ptr(W), N, K, _ptr(x), M, B, _ptr(y),
                                         _stream(stream)), "pn_gemv_hadamard_noalloc")


def gemv_hadamard_ptr(type_, W_ptr, N, K, x_ptr, M, B, y_ptr, stream_handle):
    """Raw-pointer form for timing loops: returns the status instead of raising."""
    return _lib.pn_gemv_hadamard(type_, W_ptr, N, K, x_ptr, M, B, y_ptr, stream_handle)


def quantize_rows(type_, w, W, status=None, stream=None):
    """PN reference quantizer: W (uint8[nrows, row_bytes], device) <- fp32 w[nrows, K]."""
    import torch
    _dev(w, "w", torch.float32)
    nrows, K = w.shape
    _check(_lib.pn_quantize_rows(type_, _ptr(w), nrows, K, _ptr(W), _ptr(status),
                                 _stream(stream)), "pn_quantize_rows")


# ---- NVFP4 ------------------------------------------------------------------------------------

def nvfp4_validate_rows(scales, g, N, K, verdict, stream=None):
    _check(_lib.pn_nvfp4_validate_rows(_ptr(scales), g, N, K, _ptr(verdict), _stream(stream)),
           "pn_nvfp4_validate_rows")


def nvfp4_dequantize_rows(codes, scales, g, N, K, out, stream=None):
    _check(_lib.pn_nvfp4_dequantize_rows(_ptr(codes), _ptr(scales), g, N, K, _ptr(out),
                                         _stream(stream)), "pn_nvfp4_dequantize_rows")


def gemv_nvfp4(codes, scales, g, N, K, x_bf16, y, M=None, stream=None):
    """y[M, N] <- NVFP4 W . x; x_bf16 holds raw bf16 words (int16/uint16/bfloat16 tensor)."""
    if M is None:
        M = 1 if x_bf16.dim() == 1 else x_bf16.shape[0]
    _check(_lib.pn_gemv_nvfp4(_ptr(codes), _ptr(scales), g, N, K, _ptr(x_bf16), M, _ptr(y),
                              _stream(stream)), "pn_gemv_nvfp4")


def gemv_nvfp4_ptr(codes_ptr, scales_ptr, g, N, K, x_ptr, M, y_ptr, stream_handle):
    return _lib.pn_gemv_nvfp4(codes_ptr, scales_ptr, g, N, K, x_ptr, M, y_ptr, stream_handle)


# ---- row-scaled E4M3FN (FP8_E4M3FN_ROW_BF16S) ----------------------------------------------------

def fp8row_validate_rows(codes, scales, N, K, verdict, stream=None):
    _check(_lib.pn_fp8row_validate_rows(_ptr(codes), _ptr(scales), N, K, _ptr(verdict),
                                        _stream(stream)), "pn_fp8row_validate_rows")


def fp8row_dequantize_rows(codes, scales, N, K, out, stream=None):
    _check(_lib.pn_fp8row_dequantize_rows(_ptr(codes), _ptr(scales), N, K, _ptr(out),
                                          _stream(stream)), "pn_fp8row_dequantize_rows")


def gemv_fp8row(codes, scales, N, K, x, y, M=None, stream=None):
    """y[M, N] <- (row-scaled E4M3) W . x, x fp32[M, K]."""
    if M is None:
        M = 1 if x.dim() == 1 else x.shape[0]
    _check(_lib.pn_gemv_fp8row(_ptr(codes), _ptr(scales), N, K, _ptr(x), M, _ptr(y),
                               _stream(stream)), "pn_gemv_fp8row")


def gemv_fp8row_ptr(codes_ptr, scales_ptr, N, K, x_ptr, M, y_ptr, stream_handle):
    return _lib.pn_gemv_fp8row(codes_ptr, scales_ptr, N, K, x_ptr, M, y_ptr, stream_handle)


