"""Pins for the oracle's NVFP4 decode, validation and clip-search quantizer.

Sources: "Quantisation and profiles", sections "NVFP4" (w = e2m1 * weight_scale[n, k/16] *
weight_scale_2, 0.5625 B/weight, the MLP byte counts) and "The clip search" (five multipliers);
NInfer "tensor formats" section 3.3 (E2M1/E4M3FN words, scale validity). The quantizer's base
scale formulas are this library's reading (the pages give only the multipliers): parity with the
engine's own quantizer is unpinned; what is pinned is validity, the grid, and that the kept
multiplier is the brute-force minimum of the five.
"""
import math

import numpy as np

import synth
from conftest import golden_lines


def clip_multipliers():
    (row,) = [r for r in golden_lines("quantizer_grids.txt") if r[0] == "clip_multipliers"]
    return [float(v) for v in row[1:]]


def test_sizes_fixture():
    vals = {r[0]: float(r[1]) for r in golden_lines("sizes.txt")}
    N, K = 17408, 5120
    per_matrix = N * (K // 2) + N * (K // 16)  # codes + one E4M3FN scale per 16
    assert per_matrix / (N * K) == vals["nvfp4_bytes_per_weight"]
    assert round(3 * per_matrix / 1e6, 1) == vals["mlp_nvfp4_MB"]
    assert round(3 * N * K / 1e6, 1) == vals["mlp_fp8_MB"]


def test_decode_is_product_of_words_with_unit_global(orc):
    grid = {int(w): float(v) for w, v in golden_lines("e2m1_grid.txt")}
    N, K = 1, 256
    codes = np.zeros((N, K // 2), np.uint8)
    scales = np.zeros((N, K // 16), np.uint8)
    # every (code, scale) pair across the row: 16 codes x 16 scale words
    scale_words = [0x00, 0x01, 0x07, 0x08, 0x38, 0x3C, 0x40, 0x77, 0x78, 0x7E, 0x10, 0x20, 0x30,
                   0x50, 0x60, 0x70]
    for j, sw in enumerate(scale_words):
        scales[0, j] = sw
        for i in range(16):
            k = 16 * j + i
            c = i
            codes[0, k // 2] |= c << (4 * (k & 1))
    out = orc.nvfp4_dequantize_rows(codes, scales, 1.0, N, K).astype(np.float64)
    for j, sw in enumerate(scale_words):
        S = orc.e4m3_to_double(sw)
        for i in range(16):
            assert out[0, 16 * j + i] == grid[i] * S
            assert math.copysign(1, out[0, 16 * j + i]) == math.copysign(1, grid[i] * S) or S == 0


def test_nibble_order_low_is_even_k(orc):
    codes = np.array([[0x72, 0x00, 0x00, 0x00, 0x00, 0x00, 0x00, 0x00]], np.uint8)
    scales = np.array([[0x38]], np.uint8)  # 1.0
    out = orc.nvfp4_dequantize_rows(codes, scales, 1.0, 1, 16)
    assert out[0, 0] == 1.0 and out[0, 1] == 6.0


def test_global_multiplies_with_one_rounding(orc):
    codes = np.full((1, 8), 0x77, np.uint8)  # 6.0 everywhere
    scales = np.array([[0x3C]], np.uint8)    # 1.5 -> product 9.0 exactly
    g = float(np.float32(0.1))
    out = orc.nvfp4_dequantize_rows(codes, scales, g, 1, 16)
    assert np.all(out == np.float32(9.0) * np.float32(g))


def test_validation_rules(orc):
    N, K = 6, 32
    scales = np.full((N, 2), 0x38, np.uint8)
    scales[1, 1] = 0x80  # -0: invalid
    scales[2, 0] = 0xB8  # negative: invalid
    scales[3, 0] = 0x7F  # NaN: invalid
    scales[4, 1] = 0xFF  # NaN: invalid
    scales[5, 0] = 0x00  # +0: valid
    assert list(orc.nvfp4_validate_rows(scales, 1.0, N, K)) == [1, 0, 0, 0, 0, 1]
    ok = np.full((1, 2), 0x38, np.uint8)
    for g, v in ((1.0, 1), (0.0, 0), (-1.0, 0), (math.inf, 0), (math.nan, 0), (1e-40, 1)):
        assert orc.nvfp4_validate_rows(ok, g, 1, K)[0] == v


def test_global_scale(orc):
    w = np.array([0.5, -2688.0, 3.0], np.float32)
    assert orc.nvfp4_global_scale(w) == 1.0
    assert orc.nvfp4_global_scale(np.zeros(5, np.float32)) == 1.0
    assert math.isnan(orc.nvfp4_global_scale(np.array([1.0, np.nan], np.float32)))


def test_quantizer_invariants_and_bruteforce(orc):
    N, K = 40, 256
    w = synth.gaussian_weights(81, N, K)
    w[3, 5] = 0.3  # a group with an outlier
    g = orc.nvfp4_global_scale(w)
    codes, scales = orc.nvfp4_quantize_rows(w, g)
    assert np.all(orc.nvfp4_validate_rows(scales, g, N, K) == 1)
    deq = orc.nvfp4_dequantize_rows(codes, scales, g, N, K).astype(np.float64)
    mults = clip_multipliers()
    assert mults == [1.00, 0.95, 0.90, 0.85, 0.80]
    for n in range(N):
        for j in range(K // 16):
            wg = w[n, 16 * j:16 * j + 16].astype(np.float64)
            kept = np.sum((wg - deq[n, 16 * j:16 * j + 16]) ** 2)
            amax = np.abs(wg).max()
            errs = []
            for c in mults:
                sw = int(orc.double_to_e4m3_sat([c * amax / (6.0 * g)])[0])
                S = orc.e4m3_to_double(sw)
                if S == 0:
                    q = np.zeros(16)
                else:
                    cw = orc.double_to_e2m1_sat(wg / (S * g))
                    q = np.array([orc.e2m1_to_double(int(v)) for v in cw])
                dq = (np.float32(q) * np.float32(S)).astype(np.float32) * np.float32(g)
                errs.append(np.sum((wg - dq.astype(np.float64)) ** 2))
            assert kept == min(errs)
            # a tie keeps the earlier (larger) multiplier: the kept scale word is the first argmin
            first = int(np.argmin(errs))
            sw = int(orc.double_to_e4m3_sat([mults[first] * amax / (6.0 * g)])[0])
            assert scales[n, j] == sw


def test_clip_search_tie_keeps_the_earlier_multiplier(orc):
    """"The clip search": of two multipliers with exactly equal error the earlier (larger) one is
    kept (tests/golden/nvfp4_clip_tie.txt, built by hand)."""
    from fractions import Fraction
    from conftest import golden_lines
    rows = golden_lines("nvfp4_clip_tie.txt")
    g = float(next(r for r in rows if r[0] == "g")[1])
    w = np.zeros((1, 16), np.float32)
    for r in rows:
        if r[0] == "weight":
            w[0, int(r[1])] = float(r[2])
    scale = int(next(r for r in rows if r[0] == "scale")[1], 16)
    other = int(next(r for r in rows if r[0] == "tie_with")[1], 16)
    c = [int(v) for v in next(r for r in rows if r[0] == "codes")[1:]]
    codes, scales = orc.nvfp4_quantize_rows(w, g)
    assert int(scales[0, 0] if scales.ndim == 2 else scales[0]) == scale
    packed = np.asarray(codes).reshape(-1)
    assert int(packed[0]) == c[0] | (c[1] << 4) and int(packed[1]) == c[2] | (c[3] << 4)
    assert not packed[2:].any()

    # the tie is exact: decode both candidates' codes through the oracle and sum in rationals
    def err(sw):
        S = orc.e4m3_to_double(sw)
        tot = Fraction(0)
        for v in w[0].astype(np.float64):
            code = int(orc.double_to_e2m1_sat([float(v) / (S * g)])[0])
            dq = np.float32(np.float32(orc.e2m1_to_double(code)) * np.float32(S)) * np.float32(g)
            tot += (Fraction(float(v)) - Fraction(float(dq))) ** 2
        return tot

    assert err(scale) == err(other) == Fraction(13, 64)
