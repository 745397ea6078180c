"""Pins for the oracle's PN layout, decode and validation.

Source: "PN weight format" (PNX-FORMAT-v0), sections "Types", "Block layout", "Value",
"Validation". The packer in the oracle is written from the bit table, the unpacker from the shift
formula; the fixtures restate the table and the worked values by hand.
"""
import struct

import numpy as np
import pytest

import synth
from conftest import golden_lines

PN3T, PN4T = 124, 125
TYPES = {"pn3t": PN3T, "pn4t": PN4T}


def f32_bits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def test_types_fixture(orc):
    for name, tid, G, nbytes, bpw, cpw, z in golden_lines("pn_types.txt"):
        t = TYPES[name]
        assert int(tid) == t
        assert orc.PARAMS[t][1:] == (int(G), int(cpw), int(z))
        assert orc.row_bytes(t, int(G)) == int(nbytes)
        assert round(int(nbytes) * 8 / int(G), 2) == float(bpw)
        assert 8 * int(cpw) == int(G)  # eight u32 words per block
        assert int(z) == 2 ** (orc.PARAMS[t][0] - 1)


def test_row_bytes_rejects_partial_blocks(orc):
    # "Files that use PN": K = 6144 and 17408 use pn4t; they are not whole pn3t blocks
    assert orc.row_bytes(PN3T, 6144) == 0 and orc.row_bytes(PN3T, 17408) == 0
    assert orc.row_bytes(PN4T, 6144) == 96 * 34 and orc.row_bytes(PN4T, 17408) == 272 * 34
    assert orc.row_bytes(PN3T, 5120) == 64 * 34 and orc.row_bytes(PN4T, 5120) == 80 * 34


def _word(blk, i):
    return struct.unpack("<I", bytes(blk[2 + 4 * i:6 + 4 * i]))[0]


def test_bit_table_fixture_single_codes(orc):
    rows = [r for r in golden_lines("pn_bit_table.txt") if r[0] != "reserved"]
    for name, t, lo, hi in rows:
        typ = TYPES[name]
        bits, G, cpw, z = orc.PARAMS[typ]
        t, lo, hi = int(t), int(lo), int(hi)
        assert hi - lo + 1 == bits
        for i in range(8):
            for v in range(1, 2 ** bits):
                codes = np.zeros(G, dtype=np.uint8)
                codes[i * cpw + t] = v
                blk = orc.pack_block(typ, 0x3C00, codes)
                assert blk[0] == 0x00 and blk[1] == 0x3C  # little-endian d first
                for j in range(8):
                    assert _word(blk, j) == ((v << lo) if j == i else 0)
                d, back = orc.unpack_block(typ, blk)
                assert d == 0x3C00 and np.array_equal(back, codes)


def test_reserved_bits_stay_zero_and_roundtrip(orc):
    (_, name, b0, b1), = [r for r in golden_lines("pn_bit_table.txt") if r[0] == "reserved"]
    assert name == "pn3t" and (int(b0), int(b1)) == (15, 31)
    for typ in (PN3T, PN4T):
        bits, G, cpw, z = orc.PARAMS[typ]
        raw = synth.random_bytes(11 + typ, 300 * G)
        for r in range(300):
            codes = raw[r * G:(r + 1) * G] & ((1 << bits) - 1)
            blk = orc.pack_block(typ, int(r * 977) & 0xFFFF, codes)
            if typ == PN3T:
                assert all(_word(blk, i) & 0x80008000 == 0 for i in range(8))
            d, back = orc.unpack_block(typ, blk)
            assert np.array_equal(back, codes)


def _block_all(orc, typ, d16, code):
    G = orc.PARAMS[typ][1]
    return orc.pack_block(typ, d16, np.full(G, code, dtype=np.uint8))


def test_value_fixture(orc):
    for name, d16, code, bits in golden_lines("pn_value_examples.txt"):
        typ = TYPES[name]
        G = orc.PARAMS[typ][1]
        blk = _block_all(orc, typ, int(d16, 16), int(code))
        out = orc.dequantize_rows(typ, blk, G)
        assert np.all(f32_bits(out) == int(bits, 16)), (name, d16, code)


def test_value_fixture_single_positions(orc):
    # every element position decodes on its own (no neighbour leaks into a code)
    for name, d16, code, bits in golden_lines("pn_value_examples.txt"):
        typ = TYPES[name]
        bits_, G, cpw, z = orc.PARAMS[typ]
        for e in range(G):
            codes = np.full(G, z, dtype=np.uint8)
            codes[e] = int(code)
            out = orc.dequantize_rows(typ, orc.pack_block(typ, int(d16, 16), codes), G)
            assert f32_bits(out)[0, e] == int(bits, 16)


@pytest.mark.parametrize("typ", [PN3T, PN4T])
def test_decode_ranges_exact_and_zero_sign_all_d(orc, typ):
    """All 65,536 d words x all codes: the printed range -z*d .. (z-1)*d, exact in fp32, and the
    sign of zero (code z) follows d."""
    bits, G, cpw, z = orc.PARAMS[typ]
    ncode = 2 ** bits
    d16 = np.arange(65536, dtype=np.uint16)
    # one block per (d, code-pattern): codes 0..2^bits-1 repeated along the block
    pattern = np.arange(G, dtype=np.uint8) % ncode
    W = np.concatenate([orc.pack_block(typ, int(d), pattern) for d in d16])
    out = orc.dequantize_rows(typ, W, G).astype(np.float64)  # [65536, G]
    dv = orc.f16_to_double(d16)
    fin = np.isfinite(dv)
    exact = dv[:, None] * (pattern[None, :].astype(np.float64) - z)  # exact in double
    assert np.array_equal(out[fin], exact[fin])
    lo, hi = out[fin].min(axis=1), out[fin].max(axis=1)
    assert np.array_equal(np.minimum(lo, hi), np.minimum(-z * dv[fin], (z - 1) * dv[fin]))
    assert np.array_equal(np.maximum(lo, hi), np.maximum(-z * dv[fin], (z - 1) * dv[fin]))
    zcol = out[:, np.where(pattern == z)[0][0]]
    assert np.array_equal(np.signbit(zcol[fin]), np.signbit(dv[fin]))
    assert np.all(zcol[fin] == 0)


def test_validation_all_d_words(orc):
    for typ in (PN3T, PN4T):
        G = orc.PARAMS[typ][1]
        d16 = np.arange(65536, dtype=np.uint16)
        W = np.concatenate([orc.pack_block(typ, int(d), np.zeros(G, np.uint8)) for d in d16])
        ver = orc.validate_rows(typ, W, G)
        expect = ((d16 >> 10) & 0x1F) != 0x1F
        assert np.array_equal(ver.astype(bool), expect)


def test_validation_single_bit_flips(orc):
    for typ in (PN3T, PN4T):
        bits, G, cpw, z = orc.PARAMS[typ]
        base = orc.pack_block(typ, 0x2E66, np.arange(G, dtype=np.uint8) % (2 ** bits))
        assert orc.validate_rows(typ, base, G)[0] == 1
        invalid = []
        for byte in range(2, 34):
            for bit in range(8):
                blk = base.copy()
                blk[byte] ^= 1 << bit
                if orc.validate_rows(typ, blk, G)[0] == 0:
                    invalid.append(((byte - 2) // 4, ((byte - 2) % 4) * 8 + bit))
        if typ == PN3T:
            assert sorted(invalid) == sorted([(i, b) for i in range(8) for b in (15, 31)])
        else:
            assert invalid == []
        # flips in d: invalid exactly when d becomes NaN or infinity
        for bit in range(16):
            blk = base.copy()
            d = 0x2E66 ^ (1 << bit)
            blk[0], blk[1] = d & 0xFF, d >> 8
            expect = ((d >> 10) & 0x1F) != 0x1F
            assert orc.validate_rows(typ, blk, G)[0] == int(expect)


def test_row_validation_any_block(orc):
    # a row is invalid when ANY block is; blocks at both alignments
    typ, G = PN3T, 80
    good = orc.pack_block(typ, 0x3C00, np.zeros(G, np.uint8))
    for bad_at in range(8):
        row = [good.copy() for _ in range(8)]
        row[bad_at][33] |= 0x80  # bit 31 of word 7
        assert orc.validate_rows(typ, np.concatenate(row), 8 * G)[0] == 0
    assert orc.validate_rows(typ, np.concatenate([good] * 8), 8 * G)[0] == 1


def test_dequantize_masks_reserved_bits(orc):
    # a reserved bit makes the row invalid, but does not change any code
    typ, G = PN3T, 80
    codes = np.arange(G, dtype=np.uint8) % 8
    blk = orc.pack_block(typ, 0x3C00, codes)
    ref = orc.dequantize_rows(typ, blk, G)
    blk2 = blk.copy()
    for i in range(8):
        blk2[2 + 4 * i + 1] |= 0x80
        blk2[2 + 4 * i + 3] |= 0x80
    assert np.array_equal(f32_bits(orc.dequantize_rows(typ, blk2, G)), f32_bits(ref))
