"""x that is 4-byte aligned but not 16-byte aligned, through every GEMV kernel family of the C ABI
(the header requires only 4-byte alignment of fp32 x, 2-byte of bf16 x). A kernel reads such x
with scalar loads at the addresses its vector loads would use, so each PN kernel must give the bits
it gives for aligned x, and every result must stay within the oracle's 1e-5 * sum |w x|
("PN weight format", "Value"; the sum y = W x itself)."""
import numpy as np
import pytest

import oracle
import synth
from gpu_cases import PN3T, PN4T, nvfp4_quantized, quantized
from test_gpu_pn import assert_within, dev_bytes

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_quantized_weight_pn3t_amd as pn
    return pn, torch, torch.device("cuda:0")


def gemv_x_at(pn, torch, dev, typ, Wd, N, K, x, offset_floats):
    """pn_gemv with x placed offset_floats floats into a 256-byte aligned device buffer."""
    M = x.shape[0]
    buf = torch.zeros(M * K + offset_floats, dtype=torch.float32, device=dev)
    xd = buf[offset_floats:offset_floats + M * K].view(M, K)
    xd.copy_(torch.from_numpy(np.ascontiguousarray(x, np.float32)))
    yd = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev)
    pn.gemv(typ, Wd, N, K, xd, yd)
    torch.cuda.synchronize()
    return yd.cpu().numpy()


# (type, N, blocks per row, M, forced piece size or None): the variant each case reaches
CASES = [
    (PN3T, 300, 64, 1, None),                  # vector units, 8-word pieces, one token
    (PN4T, 100, 40, 2, None),                  # vector units, 4-word pieces, two tokens
    (PN4T, 70, 272, 1, None),                  # vector units, long rows, one token
    (PN3T, 50, 70, 2, None),                   # vector units, two tokens
    (PN4T, 19, 130, 1, ("PN_GEMV_PIECE", "2")),  # vector units, 2-word pieces, forced
    (PN3T, 37, 64, 3, None),                   # vector units, 4-word pieces, three tokens
    (PN4T, 45, 128, 4, None),                  # vector units, 2-word pieces, four tokens
    (PN4T, 77, 96, 5, None),                   # matrix cores, W through LDS
    (PN3T, 33, 10, 5, None),                   # matrix cores, direct weight loads
    (PN4T, 20, 32, 9, None),                   # matrix cores, K-split layout
]


@pytest.mark.parametrize("typ,N,nb,M,force", CASES)
def test_gemv_x_unaligned_same_bits(env, monkeypatch, typ, N, nb, M, force):
    pn, torch, dev = env
    if force:
        monkeypatch.setenv(*force)
    G = oracle.PARAMS[typ][1]
    K = nb * G
    _, W = quantized(typ, N, K, 11000 + nb + M)
    x = synth.activations(11100 + nb + M, M, K)
    Wd = dev_bytes(torch, dev, W)
    y_ref, bound = oracle.gemv(typ, W, N, K, x)
    aligned = gemv_x_at(pn, torch, dev, typ, Wd, N, K, x, 0)
    for off in (1, 2, 3):
        y = gemv_x_at(pn, torch, dev, typ, Wd, N, K, x, off)
        assert np.array_equal(y.view(np.uint32), aligned.view(np.uint32)), f"x offset {off} floats"
    assert_within(aligned, y_ref, bound)


@pytest.mark.parametrize("M", [1, 4])
def test_gemv_nvfp4_x_unaligned(env, M):
    """bf16 x one word off 16-byte alignment goes to the general NVFP4 kernel: within the
    oracle's bound like the aligned call."""
    pn, torch, dev = env
    N, K = 37, 16 * 67
    _, g, codes, scales = nvfp4_quantized(N, K, 11200)
    xb = synth.activations_bf16(11201, M, K)
    y_ref, bound = oracle.nvfp4_gemv(codes, scales, g, N, K, xb)
    up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    buf = torch.zeros(M * K + 1, dtype=torch.int16, device=dev)
    xd = buf[1:1 + M * K].view(M, K)
    xd.copy_(torch.from_numpy(np.ascontiguousarray(xb).view(np.int16)))
    yd = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev)
    pn.gemv_nvfp4(up(codes), up(scales), g, N, K, xd, yd)
    torch.cuda.synchronize()
    assert_within(yd.cpu().numpy(), y_ref, bound)
