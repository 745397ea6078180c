"""Pins for the oracle's scalar codecs: binary16, bfloat16, E4M3FN, E2M1.

Sources: "PN weight format" ("Block layout": d is fp16; "Value": subnormal d is exact);
NInfer "tensor formats" section 3.1 (BF16 word), section 3.3 (E2M1, E4M3FN closed forms);
"Quantisation and profiles", "NVFP4" (the E2M1 grid). numpy's binary16 conversions are the
library pin for the oracle's fp16 codec.
"""
import math
import struct

import numpy as np

from conftest import golden_lines


def test_f16_decode_all_words_match_numpy(orc):
    h = np.arange(65536, dtype=np.uint16)
    ours = orc.f16_to_double(h)
    ref = h.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # signs of zero and of every finite value agree
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_f16_decode_subnormals_exact(orc):
    # smallest and largest subnormals, positive and negative: m * 2^-24, no flush to zero
    assert orc.f16_to_double([0x0001])[0] == 2.0 ** -24
    assert orc.f16_to_double([0x03FF])[0] == 1023 * 2.0 ** -24
    assert orc.f16_to_double([0x8001])[0] == -(2.0 ** -24)
    assert orc.f16_to_double([0x0400])[0] == 2.0 ** -14
    assert orc.f16_to_double([0x7BFF])[0] == 65504.0


def _f16_neighbours_and_midpoints():
    h = np.arange(0, 0x7C00, dtype=np.uint16)  # all finite non-negative words
    v = h.view(np.float16).astype(np.float64)
    mids = (v[:-1] + v[1:]) / 2.0  # exact in double: ties between neighbours
    return v, mids


def test_f16_round_matches_numpy_on_ties_and_random(orc):
    v, mids = _f16_neighbours_and_midpoints()
    rng = np.random.default_rng(7)
    rand = np.concatenate([
        rng.standard_normal(200000) * 10.0 ** rng.integers(-9, 6, 200000),
        rng.uniform(0, 2.0 ** -14, 20000),         # subnormal range
        rng.uniform(65000, 70000, 2000),          # around overflow
    ])
    vals = np.concatenate([v, mids, -mids, rand, -rand, [65519.99, 65520.0, 65536.0, 1e300,
                                                         2.0 ** -25, 2.0 ** -25 * 1.0000001,
                                                         0.0, -0.0, math.inf, -math.inf]])
    ours = orc.double_to_f16(vals)
    with np.errstate(over="ignore"):
        ref = vals.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref)


def test_f16_round_ties_go_to_even(orc):
    v, mids = _f16_neighbours_and_midpoints()
    out = orc.double_to_f16(mids)
    assert np.all(out % 2 == 0)


def test_bf16_is_high_half_of_binary32(orc):
    # NInfer section 3.1: the exact expansion appends 16 zero low bits
    for w in (0x0000, 0x8000, 0x3F80, 0xBF80, 0x0001, 0x7F80, 0xFF80, 0x4049):
        f = orc.bf16_to_float(w)
        assert struct.unpack("<I", struct.pack("<f", f))[0] == w << 16 or math.isnan(f)


def test_e2m1_grid_fixture(orc):
    for word, val in golden_lines("e2m1_grid.txt"):
        got = orc.e2m1_to_double(int(word))
        assert got == float(val)
        assert math.copysign(1.0, got) == math.copysign(1.0, float(val))


def test_e4m3_examples_fixture(orc):
    for word, val in golden_lines("e4m3fn_examples.txt"):
        got = orc.e4m3_to_double(int(word, 16))
        if val == "nan":
            assert math.isnan(got)
        else:
            assert got == float(val)
            assert math.copysign(1.0, got) == math.copysign(1.0, float(val))


def test_e4m3_structure_all_words(orc):
    vals = [orc.e4m3_to_double(c) for c in range(256)]
    nans = [c for c in range(256) if math.isnan(vals[c])]
    assert nans == [0x7F, 0xFF]
    pos = vals[:0x7F]
    assert all(a < b for a, b in zip(pos, pos[1:]))  # strictly increasing over 0x00..0x7E
    for c in range(0x7F):
        assert vals[c | 0x80] == -vals[c]
    assert max(pos) == 448.0 and pos[1] == 2.0 ** -9
    # each normal binade holds 8 equally spaced values
    for e in range(1, 16):
        b = [vals[(e << 3) | m] for m in range(8 if e < 15 else 7)]
        steps = {b[i + 1] - b[i] for i in range(len(b) - 1)}
        assert len(steps) == 1


def test_e4m3_encoder_roundtrip_ties_and_saturation(orc):
    finite = np.array([orc.e4m3_to_double(c) for c in range(0x7F)])
    assert np.array_equal(orc.double_to_e4m3_sat(finite), np.arange(0x7F, dtype=np.uint8))
    mids = (finite[:-1] + finite[1:]) / 2
    enc = orc.double_to_e4m3_sat(mids).astype(int)
    assert np.all(enc % 2 == 0)  # ties go to the even fraction
    assert np.all((enc == np.arange(0x7E)) | (enc == np.arange(1, 0x7F)))
    # just off the midpoint goes to the nearer neighbour
    assert np.array_equal(orc.double_to_e4m3_sat(np.nextafter(mids, 0)), np.arange(0x7E))
    assert np.array_equal(orc.double_to_e4m3_sat(np.nextafter(mids, 1e9)), np.arange(1, 0x7F))
    assert list(orc.double_to_e4m3_sat([448.0, 460.0, 1e9, math.inf])) == [0x7E] * 4
    assert list(orc.double_to_e4m3_sat([0.0, 2.0 ** -11])) == [0, 0]  # 2^-11 < half of 2^-9


def test_e2m1_encoder_grid_ties_and_saturation(orc):
    grid = [float(v) for _, v in golden_lines("e2m1_grid.txt")][:8]
    assert list(orc.double_to_e2m1_sat(grid)) == list(range(8))
    assert list(orc.double_to_e2m1_sat([-g for g in grid])) == [8 + c for c in range(8)]
    mids = [(a + b) / 2 for a, b in zip(grid, grid[1:])]  # .25 .75 1.25 1.75 2.5 3.5 5
    assert list(orc.double_to_e2m1_sat(mids)) == [0, 2, 2, 4, 4, 6, 6]
    assert list(orc.double_to_e2m1_sat([6.0, 7.0, 100.0, -9.0])) == [7, 7, 7, 15]
    assert list(orc.double_to_e2m1_sat([-0.1, -0.25])) == [8, 8]  # sign kept on negative zero
