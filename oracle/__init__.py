"""CPU oracle for the PN / NVFP4 / row-scaled E4M3 decode-step GEMV -- TEST INFRASTRUCTURE, NOT
THE PRODUCT.

Only the tests, the smoke entry and the bench's CPU-baseline leg may import this package. It wraps
``oracle/liboracle.so`` (plain C, built with gcc from ``pn_oracle.c``) through ctypes and numpy. It
shares no code with the GPU library and never calls it.

Every function here marshals arrays and, for the slow whole-matrix entry points, splits rows across
host threads (each C call is independent and pure); the arithmetic is all in ``pn_oracle.c``.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

PN3T = 124
PN4T = 125
#: (bits, weights per block, codes per word, zero point) from "PN weight format", "Types".
PARAMS = {PN3T: (3, 80, 10, 4), PN4T: (4, 64, 8, 8)}

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(out: str = _LIB_PATH, src: str = _SRC, defines=()) -> str:
    """Compile the oracle with gcc (no fused multiply-add, no fast-math)."""
    cmd = ["gcc", "-O2", "-std=gnu11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-Wall", *[f"-D{d}" for d in defines], "-o", out, src, "-lm"]
    subprocess.run(cmd, check=True)
    return out


_SIGS = None


def _sigs():
    P, I64, I32 = C.c_void_p, C.c_int64, C.c_int
    return {
        "or_f16_to_double": (C.c_double, [C.c_uint16]),
        "or_double_to_f16": (C.c_uint16, [C.c_double]),
        "or_e4m3_to_double": (C.c_double, [C.c_uint8]),
        "or_e2m1_to_double": (C.c_double, [C.c_uint8]),
        "or_bf16_to_float": (C.c_float, [C.c_uint16]),
        "or_double_to_e4m3_sat": (C.c_uint8, [C.c_double]),
        "or_double_to_e2m1_sat": (C.c_uint8, [C.c_double]),
        "or_pn_row_bytes": (I64, [I32, I64]),
        "or_pn_code": (I32, [C.c_double, C.c_double, I32]),
        "or_pn_unpack_block": (None, [I32, P, P, P]),
        "or_pn_pack_block": (None, [I32, C.c_uint16, P, P]),
        "or_pn_dequantize_rows": (None, [I32, P, I64, I64, P]),
        "or_pn_validate_rows": (None, [I32, P, I64, I64, P]),
        "or_pn_quantize_rows": (I32, [I32, P, I64, I64, P, P]),
        "or_pn_gemv": (None, [I32, P, I64, I64, P, I64, P, P]),
        "or_hadamard_rows": (None, [P, I64, I64, I64, P, P]),
        "or_pn_gemv_dx": (None, [I32, P, I64, I64, P, P, I64, P, P, P]),
        "or_nvfp4_dequantize_rows": (None, [P, P, C.c_float, I64, I64, P]),
        "or_nvfp4_validate_rows": (None, [P, C.c_float, I64, I64, P]),
        "or_nvfp4_global_scale": (C.c_float, [P, I64]),
        "or_nvfp4_quantize_rows": (None, [P, I64, I64, C.c_float, P, P]),
        "or_nvfp4_gemv": (None, [P, P, C.c_float, I64, I64, P, I64, P, P]),
        "or_f16_to_double_n": (None, [P, I64, P]),
        "or_double_to_f16_n": (None, [P, I64, P]),
        "or_double_to_e4m3_sat_n": (None, [P, I64, P]),
        "or_double_to_e2m1_sat_n": (None, [P, I64, P]),
        "or_double_to_bf16": (C.c_uint16, [C.c_double]),
        "or_double_to_bf16_n": (None, [P, I64, P]),
        "or_fp8row_dequantize_rows": (None, [P, P, I64, I64, P]),
        "or_fp8row_validate_rows": (None, [P, P, I64, I64, P]),
        "or_fp8row_quantize_rows": (None, [P, I64, I64, P, P, P]),
        "or_fp8row_gemv": (None, [P, P, I64, I64, P, I64, P, P]),
    }


def load(path: str) -> C.CDLL:
    """Load an oracle build (the default one, or a copy with a planted mistake in a test)."""
    L = C.CDLL(path)
    for name, (res, args) in _sigs().items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    return L


def lib() -> C.CDLL:
    global _lib
    if _lib is None:
        path = os.environ.get("PN_ORACLE_LIB", _LIB_PATH)  # a planted-mistake build in a test
        if path == _LIB_PATH and not os.path.exists(_LIB_PATH):
            build()
        _lib = load(path)
    return _lib


def use(L: C.CDLL | None):
    """Point the module-level functions at another loaded build (None restores the default)."""
    global _lib
    _lib = L


def _p(a: np.ndarray) -> int:
    return a.ctypes.data


def _threads(n: int) -> int:
    env = os.environ.get("PN_ORACLE_THREADS")
    if env:
        return max(1, int(env))
    return max(1, min(16, os.cpu_count() or 1, n))


def _row_split(nrows: int, parts: int):
    step = max(1, -(-nrows // parts))
    return [(s, min(nrows, s + step)) for s in range(0, nrows, step)]


# ---- scalar codecs (vectorised) ----------------------------------------------------------------

def f16_to_double(h) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16).ravel()
    out = np.empty(h.size, dtype=np.float64)
    lib().or_f16_to_double_n(_p(h), h.size, _p(out))
    return out


def double_to_f16(v) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float64).ravel()
    out = np.empty(v.size, dtype=np.uint16)
    lib().or_double_to_f16_n(_p(v), v.size, _p(out))
    return out


def double_to_e4m3_sat(v) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float64).ravel()
    out = np.empty(v.size, dtype=np.uint8)
    lib().or_double_to_e4m3_sat_n(_p(v), v.size, _p(out))
    return out


def double_to_e2m1_sat(v) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float64).ravel()
    out = np.empty(v.size, dtype=np.uint8)
    lib().or_double_to_e2m1_sat_n(_p(v), v.size, _p(out))
    return out


def e4m3_to_double(c: int) -> float:
    return lib().or_e4m3_to_double(c)


def e2m1_to_double(c: int) -> float:
    return lib().or_e2m1_to_double(c)


def bf16_to_float(b: int) -> float:
    return lib().or_bf16_to_float(b)


# ---- PN ----------------------------------------------------------------------------------------

def row_bytes(type_: int, K: int) -> int:
    return int(lib().or_pn_row_bytes(type_, K))


def pn_code(w: float, s: float, z: int) -> int:
    return int(lib().or_pn_code(w, s, z))


def pack_block(type_: int, d16: int, codes) -> np.ndarray:
    G = PARAMS[type_][1]
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    assert codes.size == G
    out = np.zeros(34, dtype=np.uint8)
    lib().or_pn_pack_block(type_, d16, _p(codes), _p(out))
    return out


def unpack_block(type_: int, blk) -> tuple[int, np.ndarray]:
    G = PARAMS[type_][1]
    blk = np.ascontiguousarray(blk, dtype=np.uint8)
    assert blk.size == 34
    d = np.zeros(1, dtype=np.uint16)
    codes = np.zeros(G, dtype=np.uint8)
    lib().or_pn_unpack_block(type_, _p(blk), _p(d), _p(codes))
    return int(d[0]), codes


def dequantize_rows(type_: int, W: np.ndarray, K: int) -> np.ndarray:
    W = np.ascontiguousarray(W, dtype=np.uint8)
    rb = row_bytes(type_, K)
    n = W.size // rb
    out = np.empty((n, K), dtype=np.float32)
    lib().or_pn_dequantize_rows(type_, _p(W), n, K, _p(out))
    return out


def validate_rows(type_: int, W: np.ndarray, K: int) -> np.ndarray:
    W = np.ascontiguousarray(W, dtype=np.uint8)
    rb = row_bytes(type_, K)
    n = W.size // rb
    out = np.empty(n, dtype=np.int32)
    lib().or_pn_validate_rows(type_, _p(W), n, K, _p(out))
    return out


def quantize_rows(type_: int, w: np.ndarray, threads: int | None = None):
    """Reference quantizer over every row of fp32 w[N, K]; returns (blocks [N, row_bytes], status[N])."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    rb = row_bytes(type_, K)
    if rb == 0:
        raise ValueError("K is not a whole number of blocks")
    W = np.empty((N, rb), dtype=np.uint8)
    st = np.empty(N, dtype=np.int32)
    L = lib()

    def run(r):
        s, e = r
        L.or_pn_quantize_rows(type_, _p(w) + s * K * 4, e - s, K, _p(W) + s * rb, _p(st) + s * 4)

    parts = _row_split(N, threads or _threads(N))
    with ThreadPoolExecutor(len(parts)) as ex:
        list(ex.map(run, parts))
    return W, st


def gemv(type_: int, W: np.ndarray, N: int, K: int, x: np.ndarray, threads: int | None = None):
    """y[M, N] and bound[M, N] (float64) for x[M, K] fp32."""
    W = np.ascontiguousarray(W, dtype=np.uint8)
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.ndim == 1:
        x = x[None, :]
    M = x.shape[0]
    rb = row_bytes(type_, K)
    L = lib()
    parts = _row_split(N, threads or _threads(N))
    ys, bs = [None] * len(parts), [None] * len(parts)

    def run(i):
        s, e = parts[i]
        y = np.empty((M, e - s), dtype=np.float64)
        b = np.empty((M, e - s), dtype=np.float64)
        L.or_pn_gemv(type_, _p(W) + s * rb, e - s, K, _p(x), M, _p(y), _p(b))
        ys[i], bs[i] = y, b

    with ThreadPoolExecutor(len(parts)) as ex:
        list(ex.map(run, range(len(parts))))
    return np.concatenate(ys, axis=1), np.concatenate(bs, axis=1)


# ---- Hadamard-rotated activations ----------------------------------------------------------------

def hadamard(x: np.ndarray, B: int):
    """(out, mass) float64 [M, K]: each slice of B elements of each row of x multiplied by the
    orthonormal Sylvester Walsh-Hadamard matrix; mass = (1/sqrt B) * sum of |x| over the slice."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    if x.ndim == 1:
        x = x[None, :]
    M, K = x.shape
    if B < 1 or B & (B - 1) or K % B:
        raise ValueError("B must be a power of two that divides K")
    out = np.empty((M, K), dtype=np.float64)
    mass = np.empty((M, K), dtype=np.float64)
    L = lib()
    parts = _row_split(M, _threads(M))

    def run(i):
        s, e = parts[i]
        L.or_hadamard_rows(_p(x) + s * K * 8, e - s, K, B, _p(out) + s * K * 8,
                           _p(mass) + s * K * 8)

    with ThreadPoolExecutor(len(parts)) as ex:
        list(ex.map(run, range(len(parts))))
    return out, mass


def gemv_hadamard(type_: int, W: np.ndarray, N: int, K: int, x: np.ndarray, B: int,
                  threads: int | None = None):
    """The PN GEMV over Hadamard-rotated activations: (y, bound, rot_bound) float64 [M, N] with
    y = W (H x), bound = sum_k |w_k x'_k| and rot_bound = sum_k |w_k| mass_k (mass from hadamard)."""
    W = np.ascontiguousarray(W, dtype=np.uint8)
    xr, mass = hadamard(np.asarray(x, dtype=np.float32).astype(np.float64), B)
    M = xr.shape[0]
    rb = row_bytes(type_, K)
    L = lib()
    parts = _row_split(N, threads or _threads(N))
    ys, bs, ms = [None] * len(parts), [None] * len(parts), [None] * len(parts)

    def run(i):
        s, e = parts[i]
        y = np.empty((M, e - s), dtype=np.float64)
        b = np.empty((M, e - s), dtype=np.float64)
        mb = np.empty((M, e - s), dtype=np.float64)
        L.or_pn_gemv_dx(type_, _p(W) + s * rb, e - s, K, _p(xr), _p(mass), M, _p(y), _p(b), _p(mb))
        ys[i], bs[i], ms[i] = y, b, mb

    with ThreadPoolExecutor(len(parts)) as ex:
        list(ex.map(run, range(len(parts))))
    return (np.concatenate(ys, axis=1), np.concatenate(bs, axis=1), np.concatenate(ms, axis=1))


# ---- NVFP4 -------------------------------------------------------------------------------------

def nvfp4_global_scale(w: np.ndarray) -> float:
    w = np.ascontiguousarray(w, dtype=np.float32)
    return float(np.float32(lib().or_nvfp4_global_scale(_p(w), w.size)))


def nvfp4_quantize_rows(w: np.ndarray, g: float, threads: int | None = None):
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    codes = np.empty((N, K // 2), dtype=np.uint8)
    scales = np.empty((N, K // 16), dtype=np.uint8)
    L = lib()

    def run(r):
        s, e = r
        L.or_nvfp4_quantize_rows(_p(w) + s * K * 4, e - s, K, g, _p(codes) + s * (K // 2),
                                 _p(scales) + s * (K // 16))

    parts = _row_split(N, threads or _threads(N))
    with ThreadPoolExecutor(len(parts)) as ex:
        list(ex.map(run, parts))
    return codes, scales


def nvfp4_dequantize_rows(codes: np.ndarray, scales: np.ndarray, g: float, N: int, K: int):
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    out = np.empty((N, K), dtype=np.float32)
    lib().or_nvfp4_dequantize_rows(_p(codes), _p(scales), g, N, K, _p(out))
    return out


def nvfp4_validate_rows(scales: np.ndarray, g: float, N: int, K: int):
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    out = np.empty(N, dtype=np.int32)
    lib().or_nvfp4_validate_rows(_p(scales), g, N, K, _p(out))
    return out


def nvfp4_gemv(codes, scales, g: float, N: int, K: int, x_bf16: np.ndarray,
               threads: int | None = None):
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    if x.ndim == 1:
        x = x[None, :]
    M = x.shape[0]
    L = lib()
    parts = _row_split(N, threads or _threads(N))
    ys, bs = [None] * len(parts), [None] * len(parts)

    def run(i):
        s, e = parts[i]
        y = np.empty((M, e - s), dtype=np.float64)
        b = np.empty((M, e - s), dtype=np.float64)
        L.or_nvfp4_gemv(_p(codes) + s * (K // 2), _p(scales) + s * (K // 16), g, e - s, K, _p(x), M,
                        _p(y), _p(b))
        ys[i], bs[i] = y, b

    with ThreadPoolExecutor(len(parts)) as ex:
        list(ex.map(run, range(len(parts))))
    return np.concatenate(ys, axis=1), np.concatenate(bs, axis=1)


# ---- row-scaled E4M3FN (FP8_E4M3FN_ROW_BF16S) ----------------------------------------------------

def double_to_bf16(v) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float64).ravel()
    out = np.empty(v.size, dtype=np.uint16)
    lib().or_double_to_bf16_n(_p(v), v.size, _p(out))
    return out


def fp8row_dequantize_rows(codes: np.ndarray, scales: np.ndarray, N: int, K: int):
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    out = np.empty((N, K), dtype=np.float32)
    lib().or_fp8row_dequantize_rows(_p(codes), _p(scales), N, K, _p(out))
    return out


def fp8row_validate_rows(codes: np.ndarray, scales: np.ndarray, N: int, K: int):
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    out = np.empty(N, dtype=np.int32)
    lib().or_fp8row_validate_rows(_p(codes), _p(scales), N, K, _p(out))
    return out


def fp8row_quantize_rows(w: np.ndarray, threads: int | None = None):
    """Returns (codes uint8[N, K], scales uint16[N], status int32[N])."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    codes = np.empty((N, K), dtype=np.uint8)
    scales = np.empty(N, dtype=np.uint16)
    status = np.empty(N, dtype=np.int32)
    L = lib()

    def run(r):
        s, e = r
        L.or_fp8row_quantize_rows(_p(w) + s * K * 4, e - s, K, _p(codes) + s * K,
                                  _p(scales) + s * 2, _p(status) + s * 4)

    parts = _row_split(N, threads or _threads(N))
    with ThreadPoolExecutor(len(parts)) as ex:
        list(ex.map(run, parts))
    return codes, scales, status


def fp8row_gemv(codes, scales, N: int, K: int, x: np.ndarray, threads: int | None = None):
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.ndim == 1:
        x = x[None, :]
    M = x.shape[0]
    L = lib()
    parts = _row_split(N, threads or _threads(N))
    ys, bs = [None] * len(parts), [None] * len(parts)

    def run(i):
        s, e = parts[i]
        y = np.empty((M, e - s), dtype=np.float64)
        b = np.empty((M, e - s), dtype=np.float64)
        L.or_fp8row_gemv(_p(codes) + s * K, _p(scales) + s * 2, e - s, K, _p(x), M, _p(y), _p(b))
        ys[i], bs[i] = y, b

    with ThreadPoolExecutor(len(parts)) as ex:
        list(ex.map(run, range(len(parts))))
    return np.concatenate(ys, axis=1), np.concatenate(bs, axis=1)
