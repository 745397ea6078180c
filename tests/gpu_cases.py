"""Input builders for the GPU parity tests (host side, numpy). The weights are quantized by the
CPU oracle; nothing here comes from the GPU path."""
from __future__ import annotations

import functools

import numpy as np

import oracle
import synth

PN3T, PN4T = 124, 125


def hand_blocks_pn3t():
    """The 16 hand-built pn3t blocks: (description, block bytes, expected valid)."""
    G, z = 80, 4
    rng_codes = synth.random_bytes(1601, 16 * G) & 7
    blocks = []

    def add(desc, d16, codes, valid=True, post=None):
        blk = oracle.pack_block(PN3T, d16, np.asarray(codes, dtype=np.uint8))
        if post:
            post(blk)
        blocks.append((desc, blk, valid))

    def setbit(word, bit):
        def f(blk):
            blk[2 + 4 * word + bit // 8] |= 1 << (bit % 8)
        return f

    def setbits(*pairs):
        def f(blk):
            for w, b in pairs:
                setbit(w, b)(blk)
        return f

    full = lambda v: np.full(G, v, np.uint8)  # noqa: E731
    add("negative d", 0xA24E, rng_codes[0:G])
    add("canonical zero group", 0x0000, full(z))
    add("code z with negative d", 0xBC00, full(z))
    add("bit 15 set", 0x3C00, rng_codes[G:2 * G], False, setbit(0, 15))
    add("bit 31 set", 0x3C00, rng_codes[2 * G:3 * G], False, setbit(3, 31))
    add("NaN d", 0x7E00, rng_codes[3 * G:4 * G], False)
    add("+inf d", 0x7C00, rng_codes[4 * G:5 * G], False)
    add("-inf d", 0xFC00, rng_codes[5 * G:6 * G], False)
    add("subnormal d 0x0001", 0x0001, rng_codes[6 * G:7 * G])
    add("subnormal d 0x83ff", 0x83FF, rng_codes[7 * G:8 * G])
    add("d = -0.0", 0x8000, rng_codes[8 * G:9 * G])
    add("d = +0, codes != z", 0x0000, rng_codes[9 * G:10 * G])
    add("all codes 0", 0x2A00, full(0))
    add("all codes 7", 0x2A00, full(7))
    add("max d, extreme codes", 0x7BFF, np.arange(G) % 2 * 7)
    add("bits 15 and 31 in word 7", 0x3C00, rng_codes[10 * G:11 * G], False,
        setbits((7, 15), (7, 31)))
    return blocks


def config1():
    """pn3t N=256, K=640: oracle-quantized N(0, 0.02) rows, rows 0..15 carry one hand-built block
    each at block r mod 8 (both alignment parities). Returns (W bytes [256, 272], valid[256])."""
    N, K = 256, 640
    W, st = oracle.quantize_rows(PN3T, synth.gaussian_weights(101, N, K, 0.02))
    assert not st.any()
    valid = np.ones(N, bool)
    for r, (_, blk, ok) in enumerate(hand_blocks_pn3t()):
        b = r % 8
        W[r, 34 * b:34 * b + 34] = blk
        valid[r] = ok
    return W, valid


@functools.lru_cache(maxsize=None)
def quantized(typ: int, N: int, K: int, seed: int, dist: str = "normal"):
    """Oracle-quantized weights for a shape (cached per session). Returns (w fp32, W bytes)."""
    if dist == "normal":
        w = synth.gaussian_weights(seed, N, K, 0.02)
    else:  # Laplace(0, 0.015) with 0.1% outliers at 8x
        w = synth.laplace_outlier_weights(seed, seed + 1, N, K, 0.015, 0.001, 8.0)
    W, st = oracle.quantize_rows(typ, w)
    assert not st.any()
    return w, W


@functools.lru_cache(maxsize=None)
def nvfp4_quantized(N: int, K: int, seed: int):
    w = synth.gaussian_weights(seed, N, K, 0.02)
    g = oracle.nvfp4_global_scale(w)
    codes, scales = oracle.nvfp4_quantize_rows(w, g)
    return w, g, codes, scales


# Full decoder-layer PN GEMV set (N, K, type, seed) for the multi-token case.
LAYER_SET = [
    (17408, 5120, PN3T, 401), (17408, 5120, PN3T, 402), (6144, 5120, PN3T, 403),
    (5120, 5120, PN3T, 404), (1024, 5120, PN4T, 405), (1024, 5120, PN4T, 406),
    (5120, 6144, PN4T, 407), (5120, 17408, PN4T, 408),
]
