"""Pins for the oracle's GEMVs (PN and NVFP4): exact rational brute force on small rows, and the
special inputs whose answer is exact (one-hot x, a block indicator, x = 0)."""
from fractions import Fraction

import numpy as np
import pytest

import synth

PN3T, PN4T = 124, 125


def _exact(wrow, xrow):
    return sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(wrow, xrow))


@pytest.mark.parametrize("typ,K", [(PN3T, 160), (PN4T, 128)])
def test_pn_gemv_matches_exact_sum(orc, typ, K):
    N, M = 5, 3
    w = synth.gaussian_weights(31 + typ, N, K)
    W, _ = orc.quantize_rows(typ, w)
    x = synth.activations(32 + typ, M, K)
    y, bound = orc.gemv(typ, W, N, K, x)
    deq = orc.dequantize_rows(typ, W, K)
    for m in range(M):
        for n in range(N):
            ex = _exact(deq[n], x[m])
            assert abs(Fraction(y[m, n]) - ex) <= Fraction(bound[m, n]) * Fraction(1, 2 ** 48)
            ab = sum(abs(Fraction(float(a)) * Fraction(float(b))) for a, b in zip(deq[n], x[m]))
            assert abs(Fraction(bound[m, n]) - ab) <= ab * Fraction(1, 2 ** 48)


@pytest.mark.parametrize("typ,K", [(PN3T, 240), (PN4T, 192)])
def test_pn_gemv_one_hot_and_block_indicator(orc, typ, K):
    bits, G, cpw, z = orc.PARAMS[typ]
    N = 4
    W, _ = orc.quantize_rows(typ, synth.gaussian_weights(41 + typ, N, K))
    deq = orc.dequantize_rows(typ, W, K).astype(np.float64)
    for k in (0, 1, G - 1, G, K - 1):
        x = np.zeros((1, K), np.float32)
        x[0, k] = 1.0
        y, _ = orc.gemv(typ, W, N, K, x)
        assert np.array_equal(y[0], deq[:, k])
    for b in range(K // G):
        x = np.zeros((1, K), np.float32)
        x[0, b * G:(b + 1) * G] = 1.0
        y, _ = orc.gemv(typ, W, N, K, x)
        for n in range(N):
            d16, codes = orc.unpack_block(typ, W[n, 34 * b:34 * b + 34])
            d = float(np.uint16(d16).view(np.float16))
            assert y[0, n] == d * float(np.sum(codes.astype(np.int64) - z))
    y, bnd = orc.gemv(typ, W, N, K, np.zeros((2, K), np.float32))
    assert np.all(y == 0) and np.all(bnd == 0)


def test_pn_gemv_threads_do_not_change_results(orc):
    typ, N, K = PN4T, 37, 192
    W, _ = orc.quantize_rows(typ, synth.gaussian_weights(51, N, K))
    x = synth.activations(52, 2, K)
    y1, b1 = orc.gemv(typ, W, N, K, x, threads=1)
    y7, b7 = orc.gemv(typ, W, N, K, x, threads=7)
    assert np.array_equal(y1, y7) and np.array_equal(b1, b7)


def test_nvfp4_gemv_matches_exact_sum(orc):
    N, K, M = 4, 64, 2
    w = synth.gaussian_weights(61, N, K)
    g = orc.nvfp4_global_scale(w)
    codes, scales = orc.nvfp4_quantize_rows(w, g)
    x = synth.activations_bf16(62, M, K)
    y, bound = orc.nvfp4_gemv(codes, scales, g, N, K, x)
    deq = orc.nvfp4_dequantize_rows(codes, scales, g, N, K)
    xf = (x.astype(np.uint32) << 16).view(np.float32)
    for m in range(M):
        for n in range(N):
            ex = _exact(deq[n], xf[m])
            assert abs(Fraction(y[m, n]) - ex) <= Fraction(bound[m, n]) * Fraction(1, 2 ** 48)


def test_nvfp4_gemv_one_hot(orc):
    N, K = 3, 48
    w = synth.gaussian_weights(71, N, K)
    g = orc.nvfp4_global_scale(w)
    codes, scales = orc.nvfp4_quantize_rows(w, g)
    deq = orc.nvfp4_dequantize_rows(codes, scales, g, N, K).astype(np.float64)
    for k in (0, 1, 15, 16, 47):
        x = np.zeros((1, K), np.uint16)
        x[0, k] = 0x3F80  # bf16 1.0
        y, _ = orc.nvfp4_gemv(codes, scales, g, N, K, x)
        assert np.array_equal(y[0], deq[:, k])
