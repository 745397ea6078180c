"""Pins of the oracle's row-scaled E4M3FN format (FP8_E4M3FN_ROW_BF16S, NInfer "tensor formats"
section 3.4) and its head quantizer ("Quantisation and profiles", "The FP8 head"), against what
the pages fix and against independent arithmetic -- not against the oracle's own formulas."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth


def bf16_rne_of_binary32(f32: np.ndarray) -> np.ndarray:
    """Round-half-even of binary32 words to their high 16 bits, by integer arithmetic on the bits
    (an independent route to the same rounding for values that are exactly binary32)."""
    u = np.ascontiguousarray(f32, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def test_bf16_rounding_matches_integer_round_half_even():
    h = synth.splitmix64(11, 0, 200000)
    words = (h & np.uint64(0xFFFFFFFF)).astype(np.uint32)
    f = words.view(np.float32)
    f = f[np.isfinite(f)]
    got = oracle.double_to_bf16(f.astype(np.float64))
    assert np.array_equal(got, bf16_rne_of_binary32(f))


def test_bf16_rounding_special_values():
    cases = [(1.0, 0x3F80), (1 + 2**-8, 0x3F80), (1 + 3 * 2**-8, 0x3F82),
             (1 + 2**-8 + 2**-40, 0x3F81), (-2.5, 0xC020), (0.0, 0x0000), (-0.0, 0x8000),
             (float("inf"), 0x7F80), (float("-inf"), 0xFF80), (2.0**-133, 0x0001),
             (2.0**-134, 0x0000), (3 * 2.0**-134, 0x0002), (3.4e38, 0x7F80)]
    got = oracle.double_to_bf16([v for v, _ in cases])
    assert [int(v) for v in got] == [w for _, w in cases]
    assert (int(oracle.double_to_bf16([float("nan")])[0]) & 0x7FFF) > 0x7F80


@pytest.mark.parametrize("scale_word,scale", [(0x3F80, 1.0), (0x4100, 8.0), (0x3E80, 0.25),
                                              (0x3F40, 0.75), (0x40A0, 5.0), (0x0001, 2.0**-133)])
def test_fp8row_decode_is_code_times_multiplier(scale_word, scale):
    """Section 3.4: w = binary32(e4m3(c) * s), the scale a multiplier (not a divisor), over all 256
    code words; the code values are the section 3.3 words pinned by the codec fixtures."""
    codes = np.arange(256, dtype=np.uint8)[None, :]
    out = oracle.fp8row_dequantize_rows(codes, np.array([scale_word], np.uint16), 1, 256)[0]
    for c in range(256):
        v = oracle.e4m3_to_double(c)
        expect = np.float32(np.float32(v) * np.float32(scale)) if np.isfinite(v) else np.nan
        if np.isnan(expect):
            assert np.isnan(out[c]), c
        else:
            assert out[c] == expect and np.signbit(out[c]) == np.signbit(expect), (c, out[c], expect)
    if scale == 0.75:  # a value that only the product gives: 448 * 0.75 = 336
        assert out[0x7E] == 336.0


def _row(codes, scale):
    return np.asarray([codes], np.uint8), np.asarray([scale], np.uint16)


@pytest.mark.parametrize("desc,codes,scale,valid", [
    ("finite codes, positive scale", [0x00, 0x38, 0xB8, 0x7E, 0xFE, 0x80], 0x3F80, 1),
    ("negative scale", [0x38] * 6, 0xBF80, 0),
    ("negative zero scale", [0x00] * 6, 0x8000, 0),
    ("+inf scale", [0x38] * 6, 0x7F80, 0),
    ("NaN scale", [0x38] * 6, 0x7FC0, 0),
    ("positive subnormal scale", [0x38] * 6, 0x0001, 1),
    ("+0 scale, signed zero codes", [0x00, 0x80, 0x00, 0x80, 0x00, 0x00], 0x0000, 1),
    ("+0 scale, one nonzero code", [0x00, 0x80, 0x01, 0x00, 0x00, 0x00], 0x0000, 0),
    ("NaN code 0x7F", [0x38, 0x7F, 0x38, 0x38, 0x38, 0x38], 0x3F80, 0),
    ("NaN code 0xFF", [0x38, 0x38, 0x38, 0x38, 0x38, 0xFF], 0x3F80, 0),
    ("largest codes +-448", [0x7E, 0xFE, 0x7E, 0xFE, 0x7E, 0xFE], 0x3F80, 1),
])
def test_fp8row_validity_clauses(desc, codes, scale, valid):
    c, s = _row(codes, scale)
    assert int(oracle.fp8row_validate_rows(c, s, 1, len(codes))[0]) == valid, desc


def plain_sum(e2: np.ndarray) -> float:
    """The quantizer's error sum: double, over k in increasing order (plain Python floats)."""
    total = 0.0
    for v in e2:
        total += float(v)
    return total


def _decode(codes, scales, N, K):
    return oracle.fp8row_dequantize_rows(codes, scales, N, K).astype(np.float64)


@pytest.mark.parametrize("dist", ["normal", "laplace"])
def test_fp8row_quantizer_invariants_and_rescan(dist):
    N, K = 48, 640
    if dist == "normal":
        w = synth.gaussian_weights(61, N, K, 0.02)
    else:
        w = synth.laplace_outlier_weights(62, 63, N, K, 0.015, 0.01, 8.0)
    codes, scales, status = oracle.fp8row_quantize_rows(w)
    assert not status.any()
    assert oracle.fp8row_validate_rows(codes, scales, N, K).all()
    deq = _decode(codes, scales, N, K)
    wd = w.astype(np.float64)
    for n in range(N):
        amax = float(np.max(np.abs(wd[n])))
        cands = [int(oracle.double_to_bf16([c * amax / 448.0])[0]) for c in (1.0, 0.95, 0.90)]
        assert int(scales[n]) in cands
        # brute-force re-scan: decode every candidate's codes and compare the errors
        errs = []
        for sw in cands:
            sd = float(oracle.bf16_to_float(sw))
            q = wd[n] / sd
            mag = oracle.double_to_e4m3_sat(np.abs(q))
            c = (mag | np.where(np.signbit(q), 0x80, 0)).astype(np.uint8)
            d = _decode(c[None, :], np.array([sw], np.uint16), 1, K)[0]
            errs.append(plain_sum((wd[n] - d) ** 2))
        chosen = cands.index(int(scales[n]))
        assert errs[chosen] == min(errs)
        assert all(errs[i] > errs[chosen] for i in range(chosen))  # ties keep the earlier one
        assert plain_sum((wd[n] - deq[n]) ** 2) == errs[chosen]
        # every weight lands within half a code step, or is clipped at 448 * s
        sd = float(oracle.bf16_to_float(int(scales[n])))
        assert np.all(np.abs(deq[n]) <= 448 * sd)


def test_fp8row_quantizer_special_rows():
    K = 64
    w = np.zeros((4, K), np.float32)
    w[1, 5] = np.nan
    w[2, :] = np.linspace(-1, 1, K)
    w[3, 7] = -3.0
    codes, scales, status = oracle.fp8row_quantize_rows(w)
    assert list(status) == [0, 1, 0, 0]
    assert scales[0] == 0 and not codes[0].any()
    assert scales[1] == 0 and not codes[1].any()
    assert oracle.fp8row_validate_rows(codes, scales, 4, K).all()
    # a row holding one nonzero weight: its decode is within the multiplier's bf16 rounding of it
    deq = _decode(codes, scales, 4, K)
    assert deq[3, 7] < 0 and abs(deq[3, 7] + 3.0) <= 3.0 * 2**-3
    assert np.count_nonzero(deq[3]) == 1


def test_fp8row_gemv_exact_brute_force_and_one_hot():
    N, K = 6, 48
    w = synth.gaussian_weights(71, N, K, 0.02)
    codes, scales, _ = oracle.fp8row_quantize_rows(w)
    x = synth.activations(72, 2, K)
    y, bound = oracle.fp8row_gemv(codes, scales, N, K, x)
    deq = oracle.fp8row_dequantize_rows(codes, scales, N, K)
    for m in range(2):
        for n in range(N):
            exact = sum(Fraction(float(deq[n, k])) * Fraction(float(x[m, k])) for k in range(K))
            assert abs(Fraction(y[m, n]) - exact) <= Fraction(K, 2**52) * Fraction(bound[m, n])
    xo = np.zeros((1, K), np.float32)
    xo[0, 17] = 1.0
    y1, _ = oracle.fp8row_gemv(codes, scales, N, K, xo)
    assert np.array_equal(y1[0], deq[:, 17].astype(np.float64))
