"""Several PN GEMVs that share x (pn_gemv_group) through the C ABI against the CPU oracle ("PN
weight format", "Value"; each part's sum y = W x itself): every part within 1e-5 * sum_k |w x| per
output, the same bits on every call and as one pn_gemv call per part, the parts' outputs
independent of one another. Cases: both types, rows short and long, tiny and empty parts, x off
16-byte alignment."""
import numpy as np
import pytest

import oracle
import synth
from gpu_cases import LAYER_SET, PN3T, PN4T, quantized
from test_gpu_pn import assert_within, dev_bytes, run_gemv

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_quantized_weight_pn3t_amd as pn
    return pn, torch, torch.device("cuda:0")


def run_group(pn, torch, dev, K, parts, x, x_offset=0, w_offsets=None):
    """parts: [(type, W bytes, N)] -> list of y (numpy), one pn_gemv_group call; w_offsets: a byte
    offset (0 or 2) per part for where its W starts in its buffer."""
    M = x.shape[0]
    buf = torch.zeros(M * K + x_offset, dtype=torch.float32, device=dev)
    xd = buf[x_offset:x_offset + M * K].view(M, K)
    xd.copy_(torch.from_numpy(np.ascontiguousarray(x, np.float32)))
    ys, args = [], []
    for j, (typ, W, N) in enumerate(parts):
        yd = torch.full((M, max(N, 1)), float("nan"), dtype=torch.float32, device=dev)
        off = w_offsets[j] if w_offsets else 0
        Wd = dev_bytes(torch, dev, W, off) if N else torch.zeros(1, dtype=torch.uint8, device=dev)
        ys.append(yd)
        args.append((typ, Wd, N, yd))
    pn.gemv_group(args, K, xd, M=M)
    torch.cuda.synchronize()
    return [y.cpu().numpy()[:, :N] for y, (_, _, N) in zip(ys, parts)]


# (K, [(type, N)]): K fixes each type's piece size (8, 4 or 2 words) and its chunks per row; the
# parts of both types run as one launch in every case here at 1-4 tokens
CASES = [
    (5120, [(PN3T, 600), (PN4T, 130), (PN4T, 129)]),            # q, k, v: 64-block pn3t rows (one
                                                                # chunk), 80-block pn4t (ragged)
    (5120, [(PN3T, 1000), (PN3T, 777)]),                        # gate, up: one type
    (3200, [(PN3T, 333), (PN4T, 65), (PN3T, 1), (PN4T, 7)]),    # tiny parts of both types
    (6400, [(PN3T, 140), (PN4T, 301)]),                         # long rows of both types
    (5120, [(PN3T, 0), (PN4T, 50), (PN3T, 9)]),                 # an empty part
    (5120, [(PN3T, 200), (PN4T, 64), (PN3T, 17), (PN4T, 300)]),  # four parts
]


def parts_for(K, spec, seed):
    out = []
    for j, (typ, N) in enumerate(spec):
        W = quantized(typ, N, K, seed + 17 * j)[1] if N else np.zeros((0,), np.uint8)
        out.append((typ, W, N))
    return out


@pytest.mark.parametrize("M", [1, 2, 3, 4])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_group_matches_oracle(env, case, M):
    pn, torch, dev = env
    K, spec = CASES[case]
    parts = parts_for(K, spec, 13000 + 100 * case)
    x = synth.activations(13500 + case + M, M, K)
    ys = run_group(pn, torch, dev, K, parts, x)
    again = run_group(pn, torch, dev, K, parts, x)
    for (typ, W, N), y, y2 in zip(parts, ys, again):
        assert np.array_equal(y.view(np.uint32), y2.view(np.uint32)), "not deterministic"
        if N:
            y_ref, bound = oracle.gemv(typ, W, N, K, x)
            assert_within(y, y_ref, bound)


@pytest.mark.parametrize("M", [1, 2, 3])
def test_group_x_unaligned_and_separate_calls(env, M):
    """x one float off 16-byte alignment gives the bits of aligned x, and the group gives the bits
    of one pn_gemv call per part."""
    pn, torch, dev = env
    K, spec = CASES[0]
    parts = parts_for(K, spec, 13000)
    x = synth.activations(13600 + M, M, K)
    a = run_group(pn, torch, dev, K, parts, x)
    b = run_group(pn, torch, dev, K, parts, x, x_offset=1)
    for ya, yb in zip(a, b):
        assert np.array_equal(ya.view(np.uint32), yb.view(np.uint32))
    for (typ, W, N), ya in zip(parts, a):
        y1 = run_gemv(pn, torch, dev, typ, dev_bytes(torch, dev, W), N, K, x)
        assert np.array_equal(ya.view(np.uint32), y1.view(np.uint32))
        y_ref, bound = oracle.gemv(typ, W, N, K, x)
        assert_within(ya, y_ref, bound)


# the cases above, and one whose pn4t rows hold an odd block count (15 blocks: rows of two
# alignments, which the parts of that type take as launches of their own)
BITS_CASES = CASES + [(960, [(PN3T, 50), (PN3T, 31), (PN4T, 40), (PN4T, 3)])]


@pytest.mark.parametrize("M", [1, 2, 3, 4])
@pytest.mark.parametrize("case", range(len(BITS_CASES)))
def test_group_same_bits_as_separate_calls(env, case, M):
    """Every case at 1-4 tokens, the parts' W at alternating 4-byte alignments (+0, +2 bytes): the
    group gives the bits of one pn_gemv call per part on the same bytes (the parts share one
    launch where the shapes allow it, each part with its own share of the workgroups and its
    type's own piece size), and every output is within the oracle's bound."""
    pn, torch, dev = env
    K, spec = BITS_CASES[case]
    parts = parts_for(K, spec, 14000 + 100 * case)
    offs = [2 * (j % 2) for j in range(len(parts))]
    x = synth.activations(14500 + case + M, M, K)
    ys = run_group(pn, torch, dev, K, parts, x, w_offsets=offs)
    for (typ, W, N), y, off in zip(parts, ys, offs):
        if not N:
            continue
        y1 = run_gemv(pn, torch, dev, typ, dev_bytes(torch, dev, W, off), N, K, x)
        assert np.array_equal(y.view(np.uint32), y1.view(np.uint32))
        y_ref, bound = oracle.gemv(typ, W, N, K, x)
        assert_within(y, y_ref, bound)


@pytest.mark.slow
@pytest.mark.parametrize("M", [1, 2, 3, 4])
@pytest.mark.parametrize("rows", [(6144, 1024), (17408,)])
def test_group_layer_q_k_v(env, M, rows):
    """The model's q (pn3t 6144x5120), k and v (pn4t 1024x5120) in one call, and its gate and up
    (pn3t 17408x5120 each) in one call, every row."""
    pn, torch, dev = env
    K = 5120
    spec = [(typ, N, seed) for N, KK, typ, seed in LAYER_SET if KK == K and N in rows]
    parts = [(typ, quantized(typ, N, K, seed)[1], N) for typ, N, seed in spec]
    assert len(parts) == (3 if rows == (6144, 1024) else 2)
    x = synth.activations(13700 + M, M, K)
    for (typ, W, N), y in zip(parts, run_group(pn, torch, dev, K, parts, x)):
        y_ref, bound = oracle.gemv(typ, W, N, K, x)
        assert_within(y, y_ref, bound)


def run_group_hadamard(pn, torch, dev, K, parts, x, B):
    M = x.shape[0]
    xd = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(dev)
    x_before = xd.clone()
    ys, args = [], []
    for typ, W, N in parts:
        yd = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev)
        ys.append(yd)
        args.append((typ, dev_bytes(torch, dev, W), N, yd))
    pn.gemv_group_hadamard(args, K, xd, B, M=M)
    torch.cuda.synchronize()
    assert torch.equal(xd, x_before), "the call modified x"
    return [y.cpu().numpy() for y in ys]


# (K, B, [(type, N)]): x rotated in slices of B ("Files that use PN"; the reading of pn_hadamard.h)
ROT_CASES = [
    (5120, 1024, [(PN3T, 600), (PN4T, 130), (PN4T, 129)]),   # 64-block pn3t + 80-block pn4t
    (5120, 256, [(PN3T, 300), (PN3T, 77)]),                  # two register parts
    (3200, 64, [(PN3T, 333), (PN4T, 65), (PN4T, 7)]),        # register bodies of both types
    (6400, 256, [(PN3T, 140), (PN4T, 301)]),                 # long rows of both types
    (17408, 1024, [(PN4T, 37), (PN4T, 20)]),                 # long rows, 17 chunks
]


@pytest.mark.parametrize("M", [1, 2, 3, 4])
@pytest.mark.parametrize("case", range(len(ROT_CASES)))
def test_group_hadamard_matches_oracle(env, case, M):
    from test_gpu_hadamard import gamma
    pn, torch, dev = env
    K, B, spec = ROT_CASES[case]
    parts = [(typ, quantized(typ, N, K, 14000 + 100 * case + 17 * j)[1], N)
             for j, (typ, N) in enumerate(spec)]
    x = synth.activations(14500 + case + M, M, K)
    ys = run_group_hadamard(pn, torch, dev, K, parts, x, B)
    again = run_group_hadamard(pn, torch, dev, K, parts, x, B)
    for (typ, W, N), y, y2 in zip(parts, ys, again):
        assert np.array_equal(y.view(np.uint32), y2.view(np.uint32)), "not deterministic"
        y_ref, bound, rbound = oracle.gemv_hadamard(typ, W, N, K, x, B)
        tol = 1e-5 * bound + (1 + 1e-5) * gamma(B) * rbound
        err = np.abs(y.astype(np.float64) - y_ref)
        assert np.all(err <= tol), f"max |err| / tol = {float(np.max(err / tol)):.3f}"


@pytest.mark.slow
@pytest.mark.parametrize("M", [1, 2, 3, 4])
def test_group_hadamard_layer_q_k_v(env, M):
    """The model's q, k and v over x rotated in slices of 1024, one call, every row."""
    from test_gpu_hadamard import gamma
    pn, torch, dev = env
    K, B = 5120, 1024
    spec = [(typ, N, seed) for N, KK, typ, seed in LAYER_SET if KK == K and N in (6144, 1024)]
    parts = [(typ, quantized(typ, N, K, seed)[1], N) for typ, N, seed in spec]
    x = synth.activations(14800 + M, M, K)
    for (typ, W, N), y in zip(parts, run_group_hadamard(pn, torch, dev, K, parts, x, B)):
        y_ref, bound, rbound = oracle.gemv_hadamard(typ, W, N, K, x, B)
        tol = 1e-5 * bound + (1 + 1e-5) * gamma(B) * rbound
        err = np.abs(y.astype(np.float64) - y_ref)
        assert np.all(err <= tol), f"max |err| / tol = {float(np.max(err / tol)):.3f}"


@pytest.mark.parametrize("M", [1, 2, 3, 4])
def test_group_same_bits_every_piece_size(env, monkeypatch, M):
    """Each piece size the registers allow at M tokens, forced in turn (PN_GEMV_PIECE): the group of
    both types (q, k and v shapes) still gives the bits of one pn_gemv call per part, and every
    output is within the oracle's bound."""
    pn, torch, dev = env
    K, spec = CASES[0]
    parts = parts_for(K, spec, 13000)
    x = synth.activations(14700 + M, M, K)
    for P in {1: (8, 4, 2), 2: (4, 2), 3: (4, 2), 4: (2,)}[M]:
        monkeypatch.setenv("PN_GEMV_PIECE", str(P))
        ys = run_group(pn, torch, dev, K, parts, x)
        for (typ, W, N), y in zip(parts, ys):
            y1 = run_gemv(pn, torch, dev, typ, dev_bytes(torch, dev, W), N, K, x)
            assert np.array_equal(y.view(np.uint32), y1.view(np.uint32)), P
            y_ref, bound = oracle.gemv(typ, W, N, K, x)
            assert_within(y, y_ref, bound)
