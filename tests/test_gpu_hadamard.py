"""GPU parity of the Hadamard-rotated activations ("PN weight format", "Files that use PN": the model
rotates the activations that reach the PN weights) through the C ABI against the CPU oracle.

Reading (the page gives neither order nor normalisation): slices of B elements of each row of x,
each multiplied by the orthonormal Sylvester Walsh-Hadamard matrix H_B / sqrt(B).

Tolerances, derived from the arithmetic (stated in include/pn.h): the rotation runs in fp32 as
log2(B) butterfly stages and one scaling, so per element |x'_gpu - x'| <= g * mass with
g = (log2 B + 2) * 2^-24 and mass = sum of |x| over the slice / sqrt(B). The fused GEMV then obeys
the GEMV tolerance on the rotated x plus the rotation's error carried through the weights:
|y - y_ref| <= 1e-5 * sum_k |w_k x'_k| + (1 + 1e-5) * g * sum_k |w_k| mass_k.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_cases import PN3T, PN4T, quantized
from test_gpu_pn import dev_bytes, run_gemv

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_quantized_weight_pn3t_amd as pn
    return pn, torch, torch.device("cuda:0")


def gamma(B):
    return (int(B).bit_length() - 1 + 2) * 2.0 ** -24 * (1 + 1e-6)


def dev_f32(torch, dev, a, offset_floats=0):
    """a (fp32) on the device, starting offset_floats floats into its buffer (4-byte aligned)."""
    a = np.ascontiguousarray(a, np.float32)
    buf = torch.zeros(a.size + offset_floats, dtype=torch.float32, device=dev)
    view = buf[offset_floats:offset_floats + a.size].view(a.shape)
    view.copy_(torch.from_numpy(a))
    return buf, view


def rotate(pn, torch, dev, x, B, offset=0, in_place=False):
    _, xd = dev_f32(torch, dev, x, offset)
    if in_place:
        out = xd
    else:
        _, out = dev_f32(torch, dev, np.full(x.shape, np.nan, np.float32), offset)
    pn.hadamard_rows(xd, B, out, M=x.shape[0], K=x.shape[1])
    torch.cuda.synchronize()
    return out.cpu().numpy()


def assert_rotation(got, x, B):
    ref, mass = oracle.hadamard(x, B)
    assert np.all(np.isfinite(got))
    err = np.abs(got.astype(np.float64) - ref)
    tol = gamma(B) * mass
    worst = float(np.max(err / np.maximum(tol, 1e-300)))
    assert np.all(err <= tol), f"max |err| / tol = {worst:.3f}"


@pytest.mark.parametrize("M,K,B", [(3, 640, 2), (2, 640, 4), (1, 640, 8), (3, 640, 64), (2, 1280, 256),
                                   (2, 1536, 512), (1, 5120, 1024), (2, 17408, 1024), (3, 6144, 2048),
                                   (2, 8192, 4096), (1, 16384, 16384), (16, 17408, 1024)])
@pytest.mark.parametrize("offset", [0, 1])
def test_rotation_matches_oracle(env, M, K, B, offset):
    """Every slice size from 2 to 16384 (stages in registers, across lanes, and through LDS), x
    and out 16-byte aligned or not (offset by one float)."""
    pn, torch, dev = env
    x = synth.activations(5000 + B + M, M, K)
    assert_rotation(rotate(pn, torch, dev, x, B, offset), x, B)


@pytest.mark.parametrize("M,K,B", [(4, 17408, 1024), (3, 640, 16), (1, 16384, 16384)])
def test_rotation_in_place(env, M, K, B):
    pn, torch, dev = env
    x = synth.activations(5100 + B, M, K)
    assert_rotation(rotate(pn, torch, dev, x, B, in_place=True), x, B)


def test_rotation_many_workgroup_steps(env):
    """More slices than one pass of the grid: both kernels loop over their work."""
    pn, torch, dev = env
    x = synth.activations(5200, 16, 163840)
    assert_rotation(rotate(pn, torch, dev, x, 256), x, 256)
    x = synth.activations(5201, 64, 17408)
    assert_rotation(rotate(pn, torch, dev, x, 1024), x, 1024)


@pytest.mark.parametrize("B", [4, 256, 1024, 16384])
def test_rotation_exact_inputs(env, B):
    """Even log2 B: the scaling is a power of two, so small-integer x rotates exactly (every sum
    is an integer below 2^24), and a one-hot x gives one column of H_B / sqrt(B) exactly."""
    pn, torch, dev = env
    K = max(B, 1024)
    x = (synth.random_bytes(5300 + B, 2 * K).reshape(2, K).astype(np.int64) % 9 - 4).astype(np.float32)
    ref, _ = oracle.hadamard(x, B)
    got = rotate(pn, torch, dev, x, B)
    assert np.array_equal(got.astype(np.float64), ref)
    for j in (0, 1, B // 2 + 3, K - 1):
        x1 = np.zeros((1, K), np.float32)
        x1[0, j] = 1.0
        ref, _ = oracle.hadamard(x1, B)
        assert np.array_equal(rotate(pn, torch, dev, x1, B).astype(np.float64), ref), j


def gemv_hadamard(pn, torch, dev, typ, Wd, N, K, x, B, x_offset=0):
    _, xd = dev_f32(torch, dev, x, x_offset)
    x_before = xd.clone()
    M = x.shape[0]
    yd = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev)
    pn.gemv_hadamard(typ, Wd, N, K, xd, B, yd)
    torch.cuda.synchronize()
    assert torch.equal(xd, x_before), "the fused call modified x"
    return yd.cpu().numpy()


# (type, N, nb, B): slices B below 256 rotate in registers only, larger ones through LDS; rows from
# 8 to 272 blocks, some not a multiple of 8 (a lane-kernel remainder).
FUSED = [(PN3T, 300, 64, 1024), (PN3T, 77, 8, 128), (PN3T, 33, 16, 256), (PN4T, 45, 64, 4096),
         (PN4T, 260, 272, 1024), (PN4T, 70, 96, 2048), (PN3T, 41, 80, 256), (PN4T, 19, 130, 64),
         (PN4T, 9, 256, 16384), (PN3T, 25, 8, 4), (PN4T, 31, 130, 8), (PN3T, 13, 64, 512),
         (PN4T, 50, 76, 256)]


@pytest.mark.parametrize("M", [1, 2, 3, 4])
@pytest.mark.parametrize("typ,N,nb,B", FUSED)
def test_gemv_hadamard_matches_oracle(env, typ, N, nb, B, M):
    pn, torch, dev = env
    G = oracle.PARAMS[typ][1]
    K = nb * G
    _, W = quantized(typ, N, K, 5400 + nb)
    x = synth.activations(5500 + nb + M, M, K)
    y_ref, bound, rbound = oracle.gemv_hadamard(typ, W, N, K, x, B)
    for offset in (0, 2):
        Wd = dev_bytes(torch, dev, W, offset)
        y = gemv_hadamard(pn, torch, dev, typ, Wd, N, K, x, B)
        assert np.all(np.isfinite(y))
        tol = 1e-5 * bound + (1 + 1e-5) * gamma(B) * rbound
        err = np.abs(y.astype(np.float64) - y_ref)
        assert np.all(err <= tol), f"max |err| / tol = {float(np.max(err / tol)):.3f}"


# Shapes for the bit comparison with the two calls: (type, N, nb, B, M). 40000 rows give every CU
# several rows; pn4t 260 x 272 blocks has 17 chunks of 16 blocks (tail items); 80 blocks a short
# last chunk; 76 and 130 blocks a remainder past the last multiple of 8 blocks.
ROT_BITS = [(PN3T, 300, 64, 1024, 1), (PN3T, 300, 64, 1024, 4), (PN4T, 260, 272, 1024, 2),
            (PN4T, 50, 76, 256, 3), (PN4T, 33, 80, 1024, 4), (PN3T, 25, 8, 4, 3),
            (PN3T, 40000, 8, 64, 1), (PN4T, 70, 64, 512, 2), (PN3T, 16, 4, 2, 4),
            (PN4T, 19, 130, 64, 1), (PN3T, 77, 8, 128, 2)]


@pytest.mark.parametrize("typ,N,nb,B,M", ROT_BITS)
@pytest.mark.parametrize("x_offset", [0, 1])
def test_gemv_hadamard_equals_rotate_then_gemv(env, typ, N, nb, B, M, x_offset):
    """The call rotates x with the rotation kernel and runs the GEMV kernels on the result: its
    bits equal pn_hadamard_rows followed by pn_gemv, both within the oracle's tolerance. x 16-byte
    aligned or not (offset by one float)."""
    pn, torch, dev = env
    G = oracle.PARAMS[typ][1]
    K = nb * G
    _, W = quantized(typ, N, K, 5900 + nb)
    Wd = dev_bytes(torch, dev, W)
    x = synth.activations(5950 + nb + M, M, K)
    fused = gemv_hadamard(pn, torch, dev, typ, Wd, N, K, x, B, x_offset)
    xr = rotate(pn, torch, dev, x, B)
    two = run_gemv(pn, torch, dev, typ, Wd, N, K, xr)
    assert np.array_equal(fused.view(np.uint32), two.view(np.uint32))
    y_ref, bound, rbound = oracle.gemv_hadamard(typ, W, N, K, x, B)
    tol = 1e-5 * bound + (1 + 1e-5) * gamma(B) * rbound
    err = np.abs(fused.astype(np.float64) - y_ref)
    assert np.all(err <= tol), f"max |err| / tol = {float(np.max(err / tol)):.3f}"


def test_gemv_hadamard_one_hot_column(env):
    """x = one slice's Hadamard row (a +-1/32 pattern): its rotation is e_j exactly (the matrix is
    its own inverse), so y is the decoded column j of W exactly."""
    pn, torch, dev = env
    typ, N, K, B = PN3T, 64, 5120, 1024
    _, W = quantized(typ, N, K, 5800)
    deq = oracle.dequantize_rows(typ, W, K)
    Wd = dev_bytes(torch, dev, W)
    for j in (0, 5, 1023, 2048 + 77):
        e = np.zeros((1, K), np.float32)
        e[0, j] = 1.0
        xh, _ = oracle.hadamard(e, B)  # entries +-1/32, exact in fp32
        y = gemv_hadamard(pn, torch, dev, typ, Wd, N, K, xh.astype(np.float32), B)
        assert np.array_equal(y[0], deq[:, j]), j


def test_gemv_hadamard_long_rows(env):
    """Rows of 640 blocks (K = 40960, two slices of K for the GEMV) with x rotated in slices of 1024:
    the call equals the two calls, bit for bit."""
    pn, torch, dev = env
    typ, N, K = PN4T, 40, 64 * 640
    _, W = quantized(typ, N, K, 5990)
    Wd = dev_bytes(torch, dev, W)
    x = synth.activations(5991, 2, K)
    fused = gemv_hadamard(pn, torch, dev, typ, Wd, N, K, x, 1024)
    two = run_gemv(pn, torch, dev, typ, Wd, N, K, rotate(pn, torch, dev, x, 1024))
    assert np.array_equal(fused.view(np.uint32), two.view(np.uint32))


@pytest.mark.slow
@pytest.mark.parametrize("typ,N,K,seed,xseed", [(PN3T, 17408, 5120, 301, 304),
                                                (PN4T, 5120, 17408, 303, 305)])
def test_gemv_hadamard_full_size(env, typ, N, K, seed, xseed):
    """The model's gate and down shapes with x rotated in slices of 1024 (the bench's setting),
    one to four tokens, every row against the oracle."""
    pn, torch, dev = env
    _, W = quantized(typ, N, K, seed)
    Wd = dev_bytes(torch, dev, W)
    x2 = synth.activations(xseed, 4, K)
    y_ref, bound, rbound = oracle.gemv_hadamard(typ, W, N, K, x2, 1024)
    for M in (1, 2, 3, 4):
        y = gemv_hadamard(pn, torch, dev, typ, Wd, N, K, x2[:M], 1024)
        tol = 1e-5 * bound[:M] + (1 + 1e-5) * gamma(1024) * rbound[:M]
        err = np.abs(y.astype(np.float64) - y_ref[:M])
        assert np.all(err <= tol), f"M={M} max |err| / tol = {float(np.max(err / tol)):.3f}"


def test_gemv_hadamard_two_streams_in_flight(env):
    """Rotated-x calls on two streams with nothing synchronising them, large matrices (whose GEMV
    reads the rotated x for some 15 us) between small ones, one call that needs a larger workspace
    in the middle and one grouped call: every output has the bits of the same call made alone.
    Each stream's calls reuse that stream's workspace, so this holds only if the two streams'
    workspaces are apart and a grown one is released after the calls that read it."""
    pn, torch, dev = env
    B = 1024
    mats = {
        "down": (PN4T, 5120, 17408, 303),   # the full-size test's weights (cached)
        "gate": (PN3T, 17408, 5120, 301),
        "small": (PN3T, 300, 5120, 6101),
        "kv": (PN4T, 130, 5120, 6102),
        "long": (PN4T, 64, 81920, 6103),    # 4 x 81920 floats: past a 1 MiB workspace
    }
    Wd = {}
    for name, (typ, N, K, seed) in mats.items():
        Wd[name] = dev_bytes(torch, dev, quantized(typ, N, K, seed)[1])
    calls = [("down", 4), ("small", 1), ("gate", 2), ("down", 1), ("long", 4), ("small", 3),
             ("down", 2), ("long", 1), ("group", 2), ("gate", 1)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    xs, outs = [], []
    for i, (name, M) in enumerate(calls):
        K = 5120 if name == "group" else mats[name][2]
        x = synth.activations(6200 + i, M, K)
        _, xd = dev_f32(torch, dev, x)
        xs.append((x, xd))
        if name == "group":
            outs.append([torch.full((M, mats[p][1]), float("nan"), dtype=torch.float32, device=dev)
                         for p in ("small", "kv")])
        else:
            outs.append([torch.full((M, mats[name][1]), float("nan"), dtype=torch.float32,
                                    device=dev)])
    torch.cuda.synchronize()
    for i, (name, M) in enumerate(calls):
        s = streams[i % 2]
        xd = xs[i][1]
        if name == "group":
            parts = [(mats[p][0], Wd[p], mats[p][1], y) for p, y in zip(("small", "kv"), outs[i])]
            pn.gemv_group_hadamard(parts, 5120, xd, B, M=M, stream=s)
        else:
            typ, N, K, _ = mats[name]
            pn.gemv_hadamard(typ, Wd[name], N, K, xd, B, outs[i][0], M=M, stream=s)
    torch.cuda.synchronize()
    for i, (name, M) in enumerate(calls):
        x = xs[i][0]
        for p, y in zip(("small", "kv") if name == "group" else (name,), outs[i]):
            typ, N, K, _ = mats[p]
            alone = gemv_hadamard(pn, torch, dev, typ, Wd[p], N, K, x, B)
            assert np.array_equal(y.cpu().numpy().view(np.uint32), alone.view(np.uint32)), (i, p)


def test_gemv_hadamard_more_streams_than_slots(env):
    """24 streams (more than the 16 workspaces a device keeps, so some calls take a temporary of
    their own), one rotated-x call on each with nothing synchronising them: every output has the
    bits of the same call made alone."""
    pn, torch, dev = env
    typ, N, K, B = PN3T, 300, 5120, 1024
    Wd = dev_bytes(torch, dev, quantized(typ, N, K, 6101)[1])
    streams = [torch.cuda.Stream() for _ in range(24)]
    xs, ys = [], []
    for i in range(len(streams)):
        M = 1 + i % 4
        x = synth.activations(6300 + i, M, K)
        xs.append((x, dev_f32(torch, dev, x)[1]))
        ys.append(torch.full((M, N), float("nan"), dtype=torch.float32, device=dev))
    torch.cuda.synchronize()
    for i, s in enumerate(streams):
        pn.gemv_hadamard(typ, Wd, N, K, xs[i][1], B, ys[i], M=xs[i][0].shape[0], stream=s)
    torch.cuda.synchronize()
    for i in range(len(streams)):
        alone = gemv_hadamard(pn, torch, dev, typ, Wd, N, K, xs[i][0], B)
        assert np.array_equal(ys[i].cpu().numpy().view(np.uint32), alone.view(np.uint32)), i
