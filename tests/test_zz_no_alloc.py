"""pn_gemv_hadamard_noalloc (the entry point for callers that cannot allocate) against
pn_gemv_hadamard through the C ABI: two calls in a row, the second on a smaller input, each the
same bits as the allocating call (the same rotation and GEMV kernels on the same inputs), and both
within the oracle's bound. The size limit is checked on the host."""
import numpy as np
import pytest

import oracle
import synth
from gpu_cases import PN3T, PN4T, quantized
from test_gpu_hadamard import gamma
from test_gpu_pn import dev_bytes

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_quantized_weight_pn3t_amd as pn
    return pn, torch, torch.device("cuda:0")


def both(pn, torch, dev, typ, N, nb, M, B, seed):
    G = oracle.PARAMS[typ][1]
    K = nb * G
    _, W = quantized(typ, N, K, seed)
    x = synth.activations(seed + 1, M, K)
    Wd = dev_bytes(torch, dev, W)
    xd = torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    ya = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev)
    yn = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev)
    pn.gemv_hadamard(typ, Wd, N, K, xd, B, ya, M=M)
    pn.gemv_hadamard_noalloc(typ, Wd, N, K, xd, B, yn, M=M)
    torch.cuda.synchronize()
    ya, yn = ya.cpu().numpy(), yn.cpu().numpy()
    assert np.array_equal(ya.view(np.uint32), yn.view(np.uint32))
    # the GEMV's bound on the rotated x plus the rotation's own error carried through the weights
    y_ref, bound, rbound = oracle.gemv_hadamard(typ, W, N, K, x, B)
    err = np.abs(yn.astype(np.float64) - y_ref)
    assert np.all(np.isfinite(yn))
    assert np.all(err <= 1e-5 * bound + (1 + 1e-5) * gamma(B) * rbound)


def test_noalloc_matches_allocating_call_twice(env):
    pn, torch, dev = env
    # first the larger call, then a smaller one that reuses (part of) the same array
    both(pn, torch, dev, PN4T, 300, 272, 4, 1024, 14000)   # M * K = 69,632 floats
    both(pn, torch, dev, PN3T, 97, 16, 1, 256, 14010)       # M * K = 1,280 floats


def test_noalloc_size_limit(env):
    pn, torch, dev = env
    K = 65600  # 4 tokens x 65,600 floats: past the 262,144-float array
    x = torch.zeros((4, K), dtype=torch.float32, device=dev)
    y = torch.zeros((4, 8), dtype=torch.float32, device=dev)
    W = torch.zeros((8, pn.row_bytes(PN4T, K)), dtype=torch.uint8, device=dev)
    st = pn.lib().pn_gemv_hadamard_noalloc(PN4T, W.data_ptr(), 8, K, x.data_ptr(), 4, 64,
                                           y.data_ptr(), None)
    assert st == -2  # PN_ERR_SHAPE
    assert 4 * K > pn.NOALLOC_MAX_FLOATS
