"""GPU parity of the PN GEMV at several tokens through the C ABI against the CPU oracle ("PN weight
format", "Block layout" and "Value"; the sum y = W x itself): the matrix-core path (5-16 tokens) and
the vector-unit kernel at 2-4 tokens.

Tolerance as for every PN GEMV: |y - y_ref| <= 1e-5 * sum_k |w_k x_k| per output. The cases cover
ragged row counts (a last tile of 16 rows partly empty), both alignment parities of the weights,
x staged in several LDS phases (with the exponent lowered between phases), workgroups that walk
several groups of tiles, exact special inputs, determinism and a per-token dynamic range.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_cases import PN3T, PN4T, quantized
from test_gpu_pn import assert_within, dev_bytes, run_gemv

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_quantized_weight_pn3t_amd as pn
    return pn, torch, torch.device("cuda:0")


def case(typ, N, nb, seed):
    G = oracle.PARAMS[typ][1]
    K = nb * G
    _, W = quantized(typ, N, K, seed)
    return K, W


@pytest.mark.parametrize("typ,N,nb", [
    (PN3T, 1, 1), (PN3T, 17, 8), (PN3T, 37, 64), (PN4T, 45, 130), (PN4T, 300, 80),
    (PN3T, 4111, 3), (PN4T, 9, 1)])
@pytest.mark.parametrize("M", [3, 5, 8, 9, 16])
def test_gemv_tokens_shapes(env, typ, N, nb, M):
    pn, torch, dev = env
    K, W = case(typ, N, nb, 9000 + nb)
    x = synth.activations(9100 + nb + M, M, K)
    y_ref, bound = oracle.gemv(typ, W, N, K, x)
    for offset in (0, 2):
        y = run_gemv(pn, torch, dev, typ, dev_bytes(torch, dev, W, offset), N, K, x)
        assert_within(y, y_ref, bound)


@pytest.mark.parametrize("typ,N,nb,M", [(PN4T, 37, 272, 16), (PN3T, 29, 100, 12), (PN4T, 70, 200, 6)])
def test_gemv_tokens_phases(env, typ, N, nb, M):
    """x too large for LDS at once: staged in phases of blocks. Token magnitudes change between
    phases (small first, then large, and the reverse) so that the per-token exponent is lowered
    from phase to phase and the running sums are rescaled."""
    pn, torch, dev = env
    K, W = case(typ, N, nb, 9200 + nb)
    x = synth.activations(9300 + nb, M, K).astype(np.float64)
    ramp = np.linspace(-12.0, 12.0, K)
    for m in range(M):
        x[m] *= 2.0 ** (ramp if m % 2 == 0 else ramp[::-1])
    x = x.astype(np.float32)
    y_ref, bound = oracle.gemv(typ, W, N, K, x)
    y = run_gemv(pn, torch, dev, typ, dev_bytes(torch, dev, W), N, K, x)
    assert_within(y, y_ref, bound)


@pytest.mark.parametrize("N,M,nb", [(256 * 16 * 10 + 333, 5, 2), (256 * 16 * 10 + 333, 11, 2),
                                    (256 * 16 * 23 + 7, 6, 2), (256 * 16 * 10 + 333, 5, 8),
                                    (256 * 16 * 12 + 5, 11, 8)])
def test_gemv_tokens_tile_groups(env, N, M, nb):
    """More than nine tiles of 16 rows per workgroup: each workgroup walks several groups of
    tiles, the last group partly empty -- for both weight paths (rows of 8 blocks staged through
    LDS, rows of 2 blocks read directly)."""
    pn, torch, dev = env
    typ = PN3T
    K, W = case(typ, N, nb, 9400 + M + nb)
    x = synth.activations(9500 + M, M, K)
    y_ref, bound = oracle.gemv(typ, W, N, K, x)
    y = run_gemv(pn, torch, dev, typ, dev_bytes(torch, dev, W), N, K, x)
    assert_within(y, y_ref, bound)


@pytest.mark.parametrize("typ,K", [(PN3T, 640), (PN4T, 512)])
def test_gemv_tokens_exact_special_inputs(env, typ, K):
    """One-hot x gives the decoded column exactly, a block indicator gives d * sum(n - z) exactly,
    x = 0 gives 0 -- at 16 tokens at once."""
    pn, torch, dev = env
    N = 40
    _, W = quantized(typ, N, K, 77)
    Wd = dev_bytes(torch, dev, W)
    deq = oracle.dequantize_rows(typ, W, K)
    G = oracle.PARAMS[typ][1]
    ks = [0, 1, 2, 7, 9, 10, 19, 20, 39, G - 1, G, G + 21, 2 * G + 5, K - 20, K - 2, K - 1]
    x = np.zeros((len(ks), K), np.float32)
    for m, k in enumerate(ks):
        x[m, k] = 1.0
    y = run_gemv(pn, torch, dev, typ, Wd, N, K, x)
    for m, k in enumerate(ks):
        assert np.array_equal(y[m], deq[:, k]), (m, k)
    x = np.zeros((3, K), np.float32)
    x[0, G:2 * G] = 1.0
    x[1, 0:G] = -2.0
    x[2, K - G:] = 0.5
    y = run_gemv(pn, torch, dev, typ, Wd, N, K, x)
    y_ref, _ = oracle.gemv(typ, W, N, K, x)
    assert np.array_equal(y.astype(np.float64), y_ref)
    y = run_gemv(pn, torch, dev, typ, Wd, N, K, np.zeros((5, K), np.float32))
    assert np.all(y == 0)


def test_gemv_tokens_deterministic(env):
    pn, torch, dev = env
    N, K = 333, 5120
    _, W = quantized(PN3T, N, K, 91)
    Wd = dev_bytes(torch, dev, W)
    x = synth.activations(93, 7, K)
    a = run_gemv(pn, torch, dev, PN3T, Wd, N, K, x)
    b = run_gemv(pn, torch, dev, PN3T, Wd, N, K, x)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_gemv_tokens_dynamic_range(env):
    """Each token has its own exponent: tokens of very different scale in one call, and a token
    whose x has one large element per block (meeting code 0, so it counts in the bound). Scales
    stay where y is a normal fp32 number: below that the output grid itself is coarser than
    1e-5 of the sum (at x ~ 2^-140, y is subnormal and half its spacing exceeds the bound)."""
    pn, torch, dev = env
    typ, N, K = PN3T, 300, 5120
    _, W = quantized(typ, N, K, 8200)
    W = W.copy()
    blocks = W.reshape(N, K // 80, 34)
    blocks[:, :, 17] &= np.uint8(0xF1)  # element 37 of every block: code 0
    x = synth.activations(8300, 6, K).astype(np.float64)
    x[0] *= 1e-30
    x[1] *= 1e30
    x[2, 37::80] = 2.0 ** 19
    x[3] *= 2.0 ** -118  # exponent near the top of the staging range
    x[4, :] = 0.0
    x[4, 100] = 3.0
    x = x.astype(np.float32)
    y_ref, bound = oracle.gemv(typ, W, N, K, x)
    y = run_gemv(pn, torch, dev, typ, dev_bytes(torch, dev, W), N, K, x)
    assert_within(y, y_ref, bound)


@pytest.mark.parametrize("M", [5, 12])
@pytest.mark.parametrize("typ,N,nb", [(PN3T, 37, 64), (PN4T, 45, 128)])
def test_gemv_direct_weight_loads_forced(env, monkeypatch, typ, N, nb, M):
    """The direct-load kernel on shapes that the LDS-staged one would take (16-byte aligned
    weights, rows of a multiple of 8 blocks)."""
    pn, torch, dev = env
    monkeypatch.setenv("PN_GEMV_MFMA_DIRECT", "1")
    K, W = case(typ, N, nb, 9800 + nb)
    x = synth.activations(9900 + nb, M, K)
    y_ref, bound = oracle.gemv(typ, W, N, K, x)
    y = run_gemv(pn, torch, dev, typ, dev_bytes(torch, dev, W), N, K, x)
    assert_within(y, y_ref, bound)


@pytest.mark.parametrize("typ,N,nb", [(PN4T, 300, 80), (PN4T, 1024, 80), (PN4T, 77, 96),
                                      (PN3T, 37, 68), (PN3T, 515, 128), (PN4T, 9, 100)])
def test_gemv_two_tokens_medium_rows(env, typ, N, nb):
    """Two tokens on rows of 65-130 blocks (partial last chunks, odd block counts), W 4-byte
    aligned and at +2 bytes."""
    pn, torch, dev = env
    K, W = case(typ, N, nb, 9400 + nb)
    x = synth.activations(9500 + nb, 2, K)
    y_ref, bound = oracle.gemv(typ, W, N, K, x)
    for offset in (0, 2):
        y = run_gemv(pn, torch, dev, typ, dev_bytes(torch, dev, W, offset), N, K, x)
        assert_within(y, y_ref, bound)


def test_gemv_two_tokens_x_ramp(env):
    """Two tokens whose magnitudes ramp over 2^24 along K (every weight is decoded exactly, so no
    range of x is special)."""
    pn, torch, dev = env
    typ, N, nb = PN4T, 130, 96
    K, W = case(typ, N, nb, 9450)
    x = synth.activations(9451, 2, K).astype(np.float64)
    ramp = np.linspace(-12.0, 12.0, K)
    x[0] *= 2.0 ** ramp
    x[1] *= 2.0 ** ramp[::-1]
    x = x.astype(np.float32)
    y_ref, bound = oracle.gemv(typ, W, N, K, x)
    assert_within(run_gemv(pn, torch, dev, typ, dev_bytes(torch, dev, W), N, K, x), y_ref, bound)


@pytest.mark.parametrize("M,typ,N,nb", [(3, PN3T, 37, 64), (3, PN4T, 45, 128), (4, PN3T, 37, 64),
                                        (4, PN4T, 45, 128), (2, PN4T, 45, 128), (2, PN3T, 33, 80)])
def test_gemv_vector_kernels_few_tokens(env, typ, N, nb, M):
    """2-4 tokens on the vector-unit kernels, both alignment parities of W."""
    pn, torch, dev = env
    K, W = case(typ, N, nb, 9950 + nb)
    x = synth.activations(9960 + nb, M, K)
    y_ref, bound = oracle.gemv(typ, W, N, K, x)
    for offset in (0, 2):
        y = run_gemv(pn, torch, dev, typ, dev_bytes(torch, dev, W, offset), N, K, x)
        assert_within(y, y_ref, bound)

@pytest.mark.slow
def test_gemv_down_full_size_tokens(env):
    """Down (pn4t 5120x17408) at 1-4 tokens, every row against the oracle. Its K slices: one launch
    at one and two tokens (at two, 156.7 KB of x beside the partials in the 160 KB LDS), two of
    9 + 8 chunks at three and four."""
    pn, torch, dev = env
    N, K = 5120, 17408
    _, W = quantized(PN4T, N, K, 303)
    Wd = dev_bytes(torch, dev, W)
    x4 = synth.activations(9990, 4, K)
    y_ref, bound = oracle.gemv(PN4T, W, N, K, x4)
    for M in (1, 2, 3, 4):
        y = run_gemv(pn, torch, dev, PN4T, Wd, N, K, x4[:M])
        assert_within(y, y_ref[:M], bound[:M])
