"""GPU parity of the row-scaled E4M3FN path (FP8_E4M3FN_ROW_BF16S, NInfer "tensor formats" section
3.4; the FP8 head of "Quantisation and profiles") through the C ABI against the CPU oracle:
bit-exact decode, validation and quantizer; GEMV within 1e-5 * sum |w x|."""
import functools

import numpy as np
import pytest

import oracle
import synth
from test_gpu_pn import assert_bits_equal, assert_within

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_quantized_weight_pn3t_amd as pn
    return pn, torch, torch.device("cuda:0")


def up(torch, dev, a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


@functools.lru_cache(maxsize=None)
def head_like(N, K, seed):
    """Oracle-quantized rows: N(0, 0.02) with every 7th row scaled by 20 (rows of different size,
    as vocabulary rows are)."""
    w = synth.gaussian_weights(seed, N, K, 0.02)
    w[::7] *= 20.0
    codes, scales, status = oracle.fp8row_quantize_rows(w)
    assert not status.any()
    return w, codes, scales


@pytest.mark.parametrize("K,aligned16", [(256, True), (100, False), (5120, True)])
def test_validate_and_dequantize_bit_exact(env, K, aligned16):
    pn, torch, dev = env
    N = 40
    _, codes, scales = head_like(N, K, 310 + K % 11)
    codes, scales = codes.copy(), scales.copy()
    # rows breaking each validity clause
    scales[1] = 0xBF80            # negative multiplier
    scales[2] = 0x8000            # negative zero
    scales[3] = 0x7F80            # infinity
    scales[4] = 0x7FC1            # NaN
    codes[5, K - 1] = 0x7F        # NaN code
    codes[6, 0] = 0xFF
    scales[7] = 0x0000            # +0 multiplier with nonzero codes
    scales[8] = 0x0000
    codes[8] = np.where(np.arange(K) % 2 == 0, 0x00, 0x80)  # +0 multiplier, signed zeros: valid
    scales[9] = 0x0001            # positive subnormal multiplier: valid
    off = 0 if aligned16 else 4
    buf = torch.zeros(N * K + 32, dtype=torch.uint8, device=dev)
    buf[off:off + N * K] = up(torch, dev, codes.reshape(-1))
    cd = buf[off:off + N * K]
    sd = up(torch, dev, scales.view(np.int16))
    ver = torch.full((N,), -1, dtype=torch.int32, device=dev)
    pn.fp8row_validate_rows(cd, sd, N, K, ver)
    out = torch.empty((N, K), dtype=torch.float32, device=dev)
    pn.fp8row_dequantize_rows(cd, sd, N, K, out)
    torch.cuda.synchronize()
    ref_v = oracle.fp8row_validate_rows(codes, scales, N, K)
    assert list(ref_v[:10]) == [1, 0, 0, 0, 0, 0, 0, 0, 1, 1]
    assert np.array_equal(ver.cpu().numpy(), ref_v)
    assert_bits_equal(out.cpu().numpy(), oracle.fp8row_dequantize_rows(codes, scales, N, K))


def test_decode_all_code_words(env):
    pn, torch, dev = env
    scales = np.array([0x3F80, 0x3F40, 0x0001, 0x7F7F, 0x0000, 0x4100], np.uint16)
    N, K = len(scales), 256
    codes = np.tile(np.arange(256, dtype=np.uint8), (N, 1))
    out = torch.empty((N, K), dtype=torch.float32, device=dev)
    pn.fp8row_dequantize_rows(up(torch, dev, codes), up(torch, dev, scales.view(np.int16)), N, K, out)
    torch.cuda.synchronize()
    assert_bits_equal(out.cpu().numpy(), oracle.fp8row_dequantize_rows(codes, scales, N, K))


def gemv(pn, torch, dev, codes, scales, N, K, x, off=0):
    M = x.shape[0]
    xb = torch.zeros(M * K + 8, dtype=torch.float32, device=dev)
    xb[off:off + M * K] = up(torch, dev, x.reshape(-1))
    xd = xb[off:off + M * K].view(M, K)
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev)
    pn.gemv_fp8row(up(torch, dev, codes), up(torch, dev, scales.view(np.int16)), N, K, xd, y)
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.parametrize("M", [1, 2, 3, 4])
@pytest.mark.parametrize("N,K", [(1, 16), (37, 1040), (300, 5120), (65, 8240), (9, 16 * 1030)])
def test_gemv(env, M, N, K):
    """Shapes across the item (1024 codes) and phase (8192 codes) boundaries, x at +4 bytes too."""
    pn, torch, dev = env
    _, codes, scales = head_like(N, K, 320 + K % 13)
    x = synth.activations(321 + K % 5, M, K)
    y_ref, bound = oracle.fp8row_gemv(codes, scales, N, K, x)
    for off in (0, 1):
        assert_within(gemv(pn, torch, dev, codes, scales, N, K, x, off), y_ref, bound)


@pytest.mark.parametrize("N,K", [(37, 1040), (300, 5120)])
def test_gemv_lds_kernel_one_token(env, monkeypatch, N, K):
    """At one token the x-in-registers kernel is the default; the LDS kernel, forced."""
    pn, torch, dev = env
    monkeypatch.setenv("PN_GEMV_NO_XREG", "1")
    _, codes, scales = head_like(N, K, 325 + K % 13)
    x = synth.activations(326, 1, K)
    y_ref, bound = oracle.fp8row_gemv(codes, scales, N, K, x)
    assert_within(gemv(pn, torch, dev, codes, scales, N, K, x), y_ref, bound)


def test_gemv_one_hot_exact(env):
    pn, torch, dev = env
    N, K = 70, 2048
    _, codes, scales = head_like(N, K, 330)
    deq = oracle.fp8row_dequantize_rows(codes, scales, N, K)
    ks = [0, 15, 1024, 2047]
    x = np.zeros((4, K), np.float32)
    for m, k in enumerate(ks):
        x[m, k] = 1.0
    y = gemv(pn, torch, dev, codes, scales, N, K, x)
    for m, k in enumerate(ks):
        assert np.array_equal(y[m], deq[:, k])


@pytest.mark.slow
def test_head_shape_sampled_rows(env):
    """The head shape, 248,320 x 5,120 (1.27 GB of codes): seeded valid E4M3FN words and bf16
    multipliers, GEMV at M = 1..4 against the oracle on every 97th row."""
    pn, torch, dev = env
    N, K = 248320, 5120
    codes = torch.empty((N, K), dtype=torch.uint8, device=dev)
    scales = torch.empty(N, dtype=torch.int16, device=dev)
    step = 16384
    rows = np.arange(0, N, 97)
    c_ref = np.empty((len(rows), K), np.uint8)
    s_ref = np.empty(len(rows), np.uint16)
    for r0 in range(0, N, step):
        n = min(step, N - r0)
        c, sc = synth.e4m3_row_words(5000 + r0, n, K)
        codes[r0:r0 + n] = up(torch, dev, c)
        scales[r0:r0 + n] = up(torch, dev, sc.view(np.int16))
        sel = (rows >= r0) & (rows < r0 + n)
        c_ref[sel] = c[rows[sel] - r0]
        s_ref[sel] = sc[rows[sel] - r0]
    x = synth.activations(5001, 4, K)
    xd = up(torch, dev, x)
    y = torch.empty((4, N), dtype=torch.float32, device=dev)
    y_ref, bound = oracle.fp8row_gemv(c_ref, s_ref, len(rows), K, x)
    for M in (1, 2, 3, 4):
        pn.gemv_fp8row(codes, scales, N, K, xd[:M], y[:M], M=M)
        torch.cuda.synchronize()
        assert_within(y[:M].cpu().numpy()[:, rows], y_ref[:M], bound[:M])