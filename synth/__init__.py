"""Seeded synthetic inputs for the PN / NVFP4 decode-step GEMV.

This module is shared by the CPU oracle side (tests, baseline timing) and the GPU side (tests,
bench). It holds no part of the method's arithmetic: no decoding, no quantization, no products.
It only draws numbers.

Generator: a counter-based splitmix64. Value i of stream `seed` is the splitmix64 finaliser applied
to ``seed + (i + 1) * 0x9E3779B97F4A7C15`` (mod 2**64), so any element can be recomputed alone and
results do not depend on chunking. Uniforms take the top 53 bits. Normals use Box-Muller in double
and are rounded once to fp32. Laplace draws use the inverse CDF.
"""
from __future__ import annotations

import numpy as np

_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_CHUNK = 1 << 22


def _mix(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def splitmix64(seed: int, start: int, count: int) -> np.ndarray:
    """Raw 64-bit words ``start .. start+count-1`` of stream ``seed``."""
    with np.errstate(over="ignore"):
        idx = np.arange(start + 1, start + count + 1, dtype=np.uint64)
        return _mix(np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + idx * _GOLDEN)


def uniform(seed: int, count: int, start: int = 0) -> np.ndarray:
    """Doubles in the open interval (0, 1): ((h >> 11) + 0.5) * 2**-53."""
    h = splitmix64(seed, start, count)
    return ((h >> np.uint64(11)).astype(np.float64) + 0.5) * (2.0 ** -53)


def normal_f32(seed: int, count: int, sigma: float = 1.0) -> np.ndarray:
    """fp32 draws of N(0, sigma^2): Box-Muller on words 2i and 2i+1, scaled in double, then one
    round-to-nearest-even to fp32."""
    out = np.empty(count, dtype=np.float32)
    for s in range(0, count, _CHUNK):
        n = min(_CHUNK, count - s)
        u = uniform(seed, 2 * n, start=2 * s)
        u1, u2 = u[0::2], u[1::2]
        z = np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2)
        out[s:s + n] = (sigma * z).astype(np.float32)
    return out


def laplace_f32(seed: int, count: int, b: float) -> np.ndarray:
    """fp32 draws of Laplace(0, b) by the inverse CDF: u in (-1/2, 1/2), x = -b sgn(u) ln(1-2|u|)."""
    out = np.empty(count, dtype=np.float32)
    for s in range(0, count, _CHUNK):
        n = min(_CHUNK, count - s)
        u = uniform(seed, n, start=s) - 0.5
        x = -b * np.sign(u) * np.log1p(-2.0 * np.abs(u))
        out[s:s + n] = x.astype(np.float32)
    return out


def outlier_mask(seed: int, count: int, p: float) -> np.ndarray:
    """Boolean mask, each element independently true with probability p."""
    out = np.empty(count, dtype=bool)
    for s in range(0, count, _CHUNK):
        n = min(_CHUNK, count - s)
        out[s:s + n] = uniform(seed, n, start=s) < p
    return out


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bfloat16 (nearest, ties to even) and return the 16-bit words.
    Input values are finite draws; NaN handling is not needed here."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    with np.errstate(over="ignore"):
        return ((u + bias) >> np.uint32(16)).astype(np.uint16)


# ---------------------------------------------------------------------------------------------
# Workload recipes. Each returns plain fp32 (or bf16-word) arrays; quantization happens elsewhere.
# ---------------------------------------------------------------------------------------------

def gaussian_weights(seed: int, n: int, k: int, sigma: float = 0.02) -> np.ndarray:
    return normal_f32(seed, n * k, sigma).reshape(n, k)


def laplace_outlier_weights(seed: int, outlier_seed: int, n: int, k: int, b: float = 0.015,
                            p: float = 0.001, factor: float = 8.0) -> np.ndarray:
    w = laplace_f32(seed, n * k, b)
    m = outlier_mask(outlier_seed, n * k, p)
    w[m] = (w[m].astype(np.float64) * factor).astype(np.float32)
    return w.reshape(n, k)


def activations(seed: int, m: int, k: int) -> np.ndarray:
    return normal_f32(seed, m * k, 1.0).reshape(m, k)


def activations_bf16(seed: int, m: int, k: int) -> np.ndarray:
    return to_bf16_bits(normal_f32(seed, m * k, 1.0)).reshape(m, k)


def random_bytes(seed: int, count: int) -> np.ndarray:
    """Uniform random bytes (for fuzzing block payloads)."""
    words = splitmix64(seed, 0, (count + 7) // 8)
    return words.view(np.uint8)[:count].copy()


def e4m3_row_words(seed: int, n: int, k: int) -> tuple[np.ndarray, np.ndarray]:
    """Seeded row-scaled E4M3FN words: codes uint8[n, k] drawn uniformly, with the two NaN words
    (0x7F, 0xFF) moved to their neighbours 0x7E / 0xFE; one bfloat16 multiplier word per row,
    positive and normal, exponent field 120..135 (about 2^-7 .. 2^8), random fraction."""
    codes = random_bytes(seed, n * k).reshape(n, k)
    nan = (codes & 0x7F) == 0x7F
    codes[nan] ^= 1
    h = splitmix64(seed + 1, 0, n)
    e = (h % np.uint64(16)).astype(np.uint16) + np.uint16(120)
    f = ((h >> np.uint64(8)) & np.uint64(0x7F)).astype(np.uint16)
    scales = (e << np.uint16(7)) | f
    return codes, scales
