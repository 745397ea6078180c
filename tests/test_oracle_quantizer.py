"""Pins for the oracle's PN reference quantizer ("PN weight format", "Reference quantizer").

No printed vectors exist on the pages, so parity with the engine's own quantizer is unpinned.
What is pinned: the tie rule (a group built by hand whose two best candidates tie exactly), the
canonical zero group, the sign rule, the candidate grid of the fixture, the
code step (with the tie examples of NInfer "tensor formats" section 7), the [0, 2z-1] clamp,
and that the kept scale is a brute-force minimum of the error over all 36 candidates (checked
in exact rational arithmetic, so no rounding order is assumed).
"""
from fractions import Fraction

import numpy as np
import pytest

import synth
from conftest import golden_lines

PN3T, PN4T = 124, 125


def multipliers():
    (row,) = [r for r in golden_lines("quantizer_grids.txt") if r[0] == "pn_multipliers"]
    return [float(v) for v in row[1:]]


def test_multiplier_fixture_shape():
    m = multipliers()
    assert len(m) == 36 and m[0] == 0.50 and m[-1] == 1.20
    assert all(abs((b - a) - 0.02) < 1e-12 for a, b in zip(m, m[1:]))


def test_code_step_ties_fixture(orc):
    for v, r in golden_lines("rint_ties.txt"):
        for z in (4, 8):
            assert orc.pn_code(float(v), 1.0, z) - z == int(r)


def test_code_step_clamps(orc):
    assert orc.pn_code(100.0, 1.0, 4) == 7 and orc.pn_code(-100.0, 1.0, 4) == 0
    assert orc.pn_code(100.0, 1.0, 8) == 15 and orc.pn_code(-100.0, 1.0, 8) == 0
    assert orc.pn_code(3.0, -1.0, 4) == 1  # negative scale flips the orientation


def _groups(typ, seed, count):
    G = orc_G(typ)
    a = synth.gaussian_weights(seed, count, G, 0.02)
    b = synth.laplace_outlier_weights(seed + 1, seed + 2, count, G, 0.015, 0.01, 8.0)
    return np.concatenate([a, b])


def orc_G(typ):
    return 80 if typ == PN3T else 64


@pytest.mark.parametrize("typ", [PN3T, PN4T])
def test_canonical_zero_group(orc, typ):
    bits, G, cpw, z = orc.PARAMS[typ]
    W, st = orc.quantize_rows(typ, np.zeros((1, G), np.float32))
    d, codes = orc.unpack_block(typ, W[0])
    assert d == 0x0000 and np.all(codes == z) and st[0] == 0
    W, st = orc.quantize_rows(typ, np.full((1, G), -0.0, np.float32))
    d, codes = orc.unpack_block(typ, W[0])
    assert d == 0x0000 and np.all(codes == z)


@pytest.mark.parametrize("typ", [PN3T, PN4T])
def test_tiny_group_is_canonical_zero(orc, typ):
    # every candidate scale rounds to fp16 zero: nothing is left to score
    bits, G, cpw, z = orc.PARAMS[typ]
    w = np.zeros((1, G), np.float32)
    w[0, 3] = 1e-9
    W, st = orc.quantize_rows(typ, w)
    d, codes = orc.unpack_block(typ, W[0])
    assert d == 0 and np.all(codes == z) and st[0] == 0


@pytest.mark.parametrize("typ", [PN3T, PN4T])
def test_nonfinite_and_overflow_status(orc, typ):
    bits, G, cpw, z = orc.PARAMS[typ]
    w = np.zeros((3, G), np.float32)
    w[0, 5] = np.nan
    w[1, 0] = np.inf
    w[2, 0] = 3.0e38  # every candidate s overflows fp16
    W, st = orc.quantize_rows(typ, w)
    assert list(st) == [1, 1, 2]
    for r in range(3):
        d, codes = orc.unpack_block(typ, W[r])
        assert d == 0 and np.all(codes == z)


def _exact_err(w, s, codes, z):
    S = Fraction(s)
    return sum((Fraction(float(wk)) - S * (int(n) - z)) ** 2 for wk, n in zip(w, codes))


@pytest.mark.parametrize("typ", [PN3T, PN4T])
def test_invariants_and_bruteforce_minimum(orc, typ):
    bits, G, cpw, z = orc.PARAMS[typ]
    w = _groups(typ, 9000 + typ, 150)
    W, st = orc.quantize_rows(typ, w)
    assert np.all(st == 0)
    ms = multipliers()
    for r in range(w.shape[0]):
        row = w[r].astype(np.float64)
        d16, codes = orc.unpack_block(typ, W[r])
        d = float(np.uint16(d16).view(np.float16))
        amax, mx, mn = np.abs(row).max(), row.max(), row.min()
        sigma = 1.0 if abs(mn) > mx else -1.0
        assert np.sign(d) == sigma                         # the sign rule
        cands = np.array([sigma * m * amax / z for m in ms]).astype(np.float16)  # numpy fp16 RNE
        assert np.float16(d) in cands                      # d is one of the 36 candidates
        assert codes.max() <= 2 * z - 1
        # the codes are the code step under the kept scale (np.rint: ties to even)
        expect = np.clip(np.rint(row / d) + z, 0, 2 * z - 1).astype(np.uint8)
        assert np.array_equal(codes, expect)
        # brute force: no candidate has a smaller exact error than the kept one
        kept = _exact_err(row, d, codes, z)
        for c in np.unique(cands):
            c = float(c)
            if c == 0 or not np.isfinite(c):
                continue
            cc = np.clip(np.rint(row / c) + z, 0, 2 * z - 1)
            assert kept <= _exact_err(row, c, cc, z) * (1 + Fraction(1, 10 ** 9))


@pytest.mark.parametrize("typ", [PN3T, PN4T])
def test_chosen_multipliers_cover_the_grid_ends(orc, typ):
    """Over many groups the kept d maps back to multipliers across the printed grid, and only to
    multipliers on it."""
    bits, G, cpw, z = orc.PARAMS[typ]
    w = _groups(typ, 4242 + typ, 3000)
    W, _ = orc.quantize_rows(typ, w)
    ms = np.array(multipliers())
    seen = set()
    for r in range(w.shape[0]):
        row = w[r].astype(np.float64)
        d16, _ = orc.unpack_block(typ, W[r])
        amax, mx, mn = np.abs(row).max(), row.max(), row.min()
        sigma = 1.0 if abs(mn) > mx else -1.0
        cands = (sigma * ms * amax / z).astype(np.float16).view(np.uint16)
        hit = np.where(cands == d16)[0]
        assert hit.size >= 1
        seen.add(int(hit.max()))   # ties between equal candidates resolve to the larger m
    assert max(seen) == 35 and min(seen) <= 16  # m = 1.20 is reached; low m on outlier groups


def test_quantizer_handles_both_signs_of_amax(orc):
    # |min| > max -> sigma = +1 (d > 0); max >= |min| -> sigma = -1 (d < 0); |min| == max -> -1
    G = 80
    a = np.linspace(-1.0, 0.5, G, dtype=np.float32)[None]
    b = np.linspace(-0.5, 1.0, G, dtype=np.float32)[None]
    c = np.linspace(-1.0, 1.0, G, dtype=np.float32)[None]
    for w, sgn in ((a, 1), (b, -1), (c, -1)):
        W, _ = orc.quantize_rows(PN3T, w)
        d16, codes = orc.unpack_block(PN3T, W[0])
        assert (d16 >> 15 == 0) == (sgn > 0)
        # orientation: the largest-magnitude weight (on the side sigma picks) gets the smallest
        # code; it is code 0 only when the kept m is at most 8/7, so that is not asserted
        k = int(np.argmin(w[0])) if sgn > 0 else int(np.argmax(w[0]))
        assert codes[k] == codes.min()


def tie_fixture():
    """The hand-built tie of tests/golden/pn_quantizer_tie.txt: (w[1, 80], d, codes, tied d)."""
    rows = golden_lines("pn_quantizer_tie.txt")
    w = np.zeros((1, 80), np.float32)
    for r in rows:
        if r[0] == "weight":
            w[0, int(r[1])] = float(r[2])
    d = int(next(r for r in rows if r[0] == "d")[1], 16)
    other = int(next(r for r in rows if r[0] == "tie_with")[1], 16)
    c0, c1, rest = (int(v) for v in next(r for r in rows if r[0] == "codes")[1:])
    codes = np.full(80, rest, np.uint8)
    codes[0], codes[1] = c0, c1
    return w, d, codes, other


def test_tie_goes_to_the_larger_m(orc):
    """"Reference quantizer": a tie between candidate scales keeps the larger m."""
    w, d_exp, codes_exp, other = tie_fixture()
    W, st = orc.quantize_rows(PN3T, w)
    d16, codes = orc.unpack_block(PN3T, W[0])
    assert st[0] == 0
    assert d16 == d_exp and np.array_equal(codes, codes_exp)

    # the fixture really is a tie, and the minimum: exact rational errors of every candidate
    def err(s16):
        s = Fraction(float(orc.f16_to_double([s16])[0]))
        tot = Fraction(0)
        for v in w[0].astype(np.float64):
            n = orc.pn_code(float(v), float(s), 4)
            tot += (Fraction(float(v)) - s * (n - 4)) ** 2
        return tot

    assert err(d_exp) == err(other) and other != d_exp
    ms = multipliers()
    cands = [int(c) for c in (-np.array(ms) * 1.25 / 4).astype(np.float16).view(np.uint16)]
    assert cands.index(other) + 1 == cands.index(d_exp)  # 0xB4B3 is m = 0.94, 0xB4CD is m = 0.96
    assert min(err(c) for c in cands) == err(d_exp)
