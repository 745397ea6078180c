"""GPU parity of the NVFP4 W4A16 path through the C ABI against the CPU oracle: bit-exact global
scale, quantizer, validation and decode; GEMV within 1e-5 * sum |w x|."""
import numpy as np
import pytest

import oracle
import synth
from gpu_cases import nvfp4_quantized
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


def gemv(pn, torch, dev, codes, scales, g, N, K, xb):
    yd = torch.full((xb.shape[0], N), float("nan"), dtype=torch.float32, device=dev)
    pn.gemv_nvfp4(up(torch, dev, codes), up(torch, dev, scales), g, N, K,
                  up(torch, dev, xb.view(np.int16)), yd)
    torch.cuda.synchronize()
    return yd.cpu().numpy()


def test_validate_and_dequantize_bit_exact(env):
    pn, torch, dev = env
    N, K = 24, 256
    _, g, codes, scales = nvfp4_quantized(N, K, 511)
    scales = scales.copy()
    scales[1, 3] = 0x80
    scales[2, 0] = 0xB8
    scales[3, 7] = 0x7F
    scales[4, 15] = 0xFF
    scales[5, 2] = 0x00
    codes = codes.copy()
    codes[6, :] = np.arange(K // 2) % 256  # every code word
    ver = torch.full((N,), -1, dtype=torch.int32, device=dev)
    for gg in (g, 0.0, -1.0, float("inf"), float("nan")):
        pn.nvfp4_validate_rows(up(torch, dev, scales), gg, N, K, ver)
        torch.cuda.synchronize()
        assert np.array_equal(ver.cpu().numpy(), oracle.nvfp4_validate_rows(scales, gg, N, K))
    for gg in (g, 1.0, 1e-30, 3.0e36):
        out = torch.empty((N, K), dtype=torch.float32, device=dev)
        pn.nvfp4_dequantize_rows(up(torch, dev, codes), up(torch, dev, scales), gg, N, K, out)
        torch.cuda.synchronize()
        assert_bits_equal(out.cpu().numpy(), oracle.nvfp4_dequantize_rows(codes, scales, gg, N, K))


@pytest.mark.parametrize("M", [1, 2, 3, 4])
@pytest.mark.parametrize("N,K", [(64, 512), (37, 16 * 67), (5, 16)])
def test_gemv_small(env, M, N, K):
    pn, torch, dev = env
    _, g, codes, scales = nvfp4_quantized(N, K, 520 + K)
    xb = synth.activations_bf16(521, M, K)
    y = gemv(pn, torch, dev, codes, scales, g, N, K, xb)
    y_ref, bound = oracle.nvfp4_gemv(codes, scales, g, N, K, xb)
    assert_within(y, y_ref, bound)


def test_gemv_one_hot_exact(env):
    pn, torch, dev = env
    N, K = 40, 256
    _, g, codes, scales = nvfp4_quantized(N, K, 530)
    deq = oracle.nvfp4_dequantize_rows(codes, scales, g, N, K)
    ks = [0, 1, 16, 255]
    xb = np.zeros((4, K), np.uint16)
    for m, k in enumerate(ks):
        xb[m, k] = 0x3F80
    y = gemv(pn, torch, dev, codes, scales, g, N, K, xb)
    for m, k in enumerate(ks):
        # one product e2m1 * S, then * g: the same two roundings as the decode
        assert np.array_equal(y[m], deq[:, k])


@pytest.mark.slow
def test_config5_full_size(env):
    pn, torch, dev = env
    N, K = 17408, 5120
    w, g, codes, scales = nvfp4_quantized(N, K, 501)
    out = torch.empty((N, K), dtype=torch.float32, device=dev)
    pn.nvfp4_dequantize_rows(up(torch, dev, codes), up(torch, dev, scales), g, N, K, out)
    torch.cuda.synchronize()
    assert_bits_equal(out.cpu().numpy(), oracle.nvfp4_dequantize_rows(codes, scales, g, N, K))
    del out
    xb = synth.activations_bf16(502, 4, K)
    y_ref4, bound4 = oracle.nvfp4_gemv(codes, scales, g, N, K, xb)
    for M in (1, 2, 3, 4):
        y = gemv(pn, torch, dev, codes, scales, g, N, K, xb[:M])
        assert_within(y, y_ref4[:M], bound4[:M])


@pytest.mark.parametrize("M", [1, 2, 3, 4])
@pytest.mark.parametrize("N,K", [(1, 16 * 256), (37, 16 * 257), (300, 5120), (5, 16 * 321), (1031, 6144),
                                 (9, 16 * 385), (70, 16 * 64), (3, 16 * 5)])
def test_gemv_register_x_shapes(env, M, N, K):
    """The kernel that keeps x in registers (up to 6 groups per lane at 1-2 tokens: K <= 6144; 5 at
    3-4 tokens), at the 4 / 5 / 6 groups-per-lane boundaries, partly filled lanes, and past them
    (the LDS kernel)."""
    pn, torch, dev = env
    _, g, codes, scales = nvfp4_quantized(N, K, 540 + K % 97)
    xb = synth.activations_bf16(541 + K, M, K)
    y = gemv(pn, torch, dev, codes, scales, g, N, K, xb)
    y_ref, bound = oracle.nvfp4_gemv(codes, scales, g, N, K, xb)
    assert_within(y, y_ref, bound)


@pytest.mark.parametrize("M", [1, 2])
def test_gemv_one_hot_exact_few_tokens(env, M):
    pn, torch, dev = env
    N, K = 40, 5120
    _, g, codes, scales = nvfp4_quantized(N, K, 531)
    deq = oracle.nvfp4_dequantize_rows(codes, scales, g, N, K)
    ks = [17, 5119][:M]
    xb = np.zeros((M, K), np.uint16)
    for m, k in enumerate(ks):
        xb[m, k] = 0x3F80
    y = gemv(pn, torch, dev, codes, scales, g, N, K, xb)
    for m, k in enumerate(ks):
        assert np.array_equal(y[m], deq[:, k])


@pytest.mark.parametrize("M", [1, 2])
def test_gemv_lds_kernel_and_unaligned_x(env, monkeypatch, M):
    """The LDS kernel at 1-2 tokens: forced, and taken by itself when x is not 16-byte aligned."""
    pn, torch, dev = env
    N, K = 45, 5120
    _, g, codes, scales = nvfp4_quantized(N, K, 550)
    xb = synth.activations_bf16(551, M, K)
    y_ref, bound = oracle.nvfp4_gemv(codes, scales, g, N, K, xb)
    # x at a 2-byte offset inside a larger buffer
    buf = torch.zeros(M * K + 8, dtype=torch.int16, device=dev)
    buf[1:1 + M * K] = up(torch, dev, xb.view(np.int16).reshape(-1))
    xd = buf[1:1 + M * K].view(M, K)
    yd = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev)
    pn.gemv_nvfp4(up(torch, dev, codes), up(torch, dev, scales), g, N, K, xd, yd)
    torch.cuda.synchronize()
    assert_within(yd.cpu().numpy(), y_ref, bound)
    monkeypatch.setenv("PN_GEMV_NO_XREG", "1")
    y = gemv(pn, torch, dev, codes, scales, g, N, K, xb)
    assert_within(y, y_ref, bound)
