"""GPU parity of the PN path (pn3t / pn4t) through the C ABI against the CPU oracle.

Decode and validation must be bit-exact (NaN outputs compared by class: a NaN or infinite d only
occurs in invalid rows, whose decode the pages leave open; the IEEE product is the reading). The
GEMV must satisfy |y - y_ref| <= 1e-5 * sum_k |w_k x_k| per output (the accuracy contract of
pn_gemv in include/pn.h; the packed-BF16 post reports about 1e-6 agreement for its own kernel). The quantizer must be bit-exact.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_cases import LAYER_SET, PN3T, PN4T, config1, hand_blocks_pn3t, quantized

pytestmark = pytest.mark.gpu
TOL = 1e-5


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_quantized_weight_pn3t_amd as pn
    return pn, torch, torch.device("cuda:0")


def dev_bytes(torch, dev, W, offset=0):
    """Upload bytes, optionally at a +offset byte position inside a larger buffer."""
    flat = np.ascontiguousarray(W).reshape(-1)
    buf = torch.zeros(flat.size + 16, dtype=torch.uint8, device=dev)
    buf[offset:offset + flat.size] = torch.from_numpy(flat).to(dev)
    return buf[offset:offset + flat.size]


def assert_bits_equal(got, ref):
    got = np.ascontiguousarray(got, np.float32)
    ref = np.ascontiguousarray(ref, np.float32)
    both_nan = np.isnan(got) & np.isnan(ref)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    gb, rb = got.view(np.uint32), ref.view(np.uint32)
    bad = (gb != rb) & ~both_nan
    assert not bad.any(), f"{bad.sum()} mismatches, first at {np.argwhere(bad)[:5].tolist()}"


def run_gemv(pn, torch, dev, typ, Wd, N, K, x):
    xd = torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(dev)
    M = x.shape[0]
    yd = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev)
    pn.gemv(typ, Wd, N, K, xd, yd)
    torch.cuda.synchronize()
    return yd.cpu().numpy()


def assert_within(y, y_ref, bound, tol=TOL):
    err = np.abs(y.astype(np.float64) - y_ref)
    assert np.all(np.isfinite(y)), "non-finite output"
    ratio = err / np.maximum(bound, 1e-300)
    worst = float(np.max(np.where(bound > 0, ratio, 0.0)))
    assert np.all(err <= tol * bound), f"max |err|/bound = {worst:.3e}"
    return worst


# ---- config 1: pn3t 256 x 640, hand-built blocks -------------------------------------------------

@pytest.mark.parametrize("offset", [0, 2])
def test_config1_dequantize_and_validate(env, offset):
    pn, torch, dev = env
    W, valid = config1()
    N, K = W.shape[0], 640
    Wd = dev_bytes(torch, dev, W, offset)
    out = torch.empty((N, K), dtype=torch.float32, device=dev)
    pn.dequantize_rows(PN3T, Wd, N, K, out)
    ver = torch.full((N,), -1, dtype=torch.int32, device=dev)
    pn.validate_rows(PN3T, Wd, N, K, ver)
    torch.cuda.synchronize()
    assert_bits_equal(out.cpu().numpy(), oracle.dequantize_rows(PN3T, W, K))
    assert np.array_equal(ver.cpu().numpy(), oracle.validate_rows(PN3T, W, K))
    assert np.array_equal(ver.cpu().numpy().astype(bool), valid)


def test_config1_hand_blocks_decoded_values(env):
    """Each hand-built block's decode, with the expectations the pages state."""
    pn, torch, dev = env
    for desc, blk, ok in hand_blocks_pn3t():
        Wd = dev_bytes(torch, dev, blk)
        out = torch.empty(80, dtype=torch.float32, device=dev)
        pn.dequantize_row(PN3T, Wd, 80, out)
        ver = torch.full((1,), -1, dtype=torch.int32, device=dev)
        pn.validate_row(PN3T, Wd, 80, ver)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        assert_bits_equal(got, oracle.dequantize_rows(PN3T, blk, 80)[0])
        assert int(ver.item()) == int(ok), desc
        if desc == "code z with negative d":
            assert np.all(got.view(np.uint32) == 0x80000000)
        if desc == "canonical zero group":
            assert np.all(got.view(np.uint32) == 0)


@pytest.mark.parametrize("M", [1, 2, 3, 4])
@pytest.mark.parametrize("offset", [0, 2])
def test_config1_gemv(env, M, offset):
    pn, torch, dev = env
    W, valid = config1()
    N, K = W.shape[0], 640
    x = synth.activations(102, M, K)
    y = run_gemv(pn, torch, dev, PN3T, dev_bytes(torch, dev, W, offset), N, K, x)
    y_ref, bound = oracle.gemv(PN3T, W, N, K, x)
    assert_within(y[:, valid], y_ref[:, valid], bound[:, valid])


# ---- exact special cases ------------------------------------------------------------------------

@pytest.mark.parametrize("typ,K", [(PN3T, 640), (PN4T, 512)])
def test_gemv_exact_special_inputs(env, typ, K):
    pn, torch, dev = env
    N = 40
    _, W = quantized(typ, N, K, 77)
    Wd = dev_bytes(torch, dev, W)
    deq = oracle.dequantize_rows(typ, W, K)
    G = oracle.PARAMS[typ][1]
    # one-hot x: y is the decoded column, exactly
    ks = [0, 1, 9, G - 1, G, K - 1]
    x = np.zeros((len(ks[:4]), K), np.float32)
    for m, k in enumerate(ks[:4]):
        x[m, k] = 1.0
    y = run_gemv(pn, torch, dev, typ, Wd, N, K, x)
    for m, k in enumerate(ks[:4]):
        assert np.array_equal(y[m], deq[:, k])
    # block indicator: y = d * sum(n - z), exactly
    x = np.zeros((1, K), np.float32)
    x[0, G:2 * G] = 1.0
    y = run_gemv(pn, torch, dev, typ, Wd, N, K, x)
    y_ref, _ = oracle.gemv(typ, W, N, K, x)
    assert np.array_equal(y[0].astype(np.float64), y_ref[0])
    # x = 0: y = 0
    y = run_gemv(pn, torch, dev, typ, Wd, N, K, np.zeros((3, K), np.float32))
    assert np.all(y == 0)


def test_gemv_is_deterministic(env):
    pn, torch, dev = env
    N, K = 300, 5120
    _, W = quantized(PN3T, N, K, 91)
    Wd = dev_bytes(torch, dev, W)
    x = synth.activations(92, 4, K)
    a = run_gemv(pn, torch, dev, PN3T, Wd, N, K, x)
    b = run_gemv(pn, torch, dev, PN3T, Wd, N, K, x)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


# ---- ragged shapes, odd block counts, alignment -----------------------------------------------

@pytest.mark.parametrize("typ,N,nb", [
    (PN3T, 1, 1), (PN3T, 7, 3), (PN3T, 13, 65), (PN3T, 33, 127), (PN4T, 5, 1), (PN4T, 9, 63),
    (PN4T, 17, 129), (PN4T, 31, 272)])
@pytest.mark.parametrize("M", [1, 4])
def test_gemv_ragged(env, typ, N, nb, M):
    pn, torch, dev = env
    G = oracle.PARAMS[typ][1]
    K = nb * G
    _, W = quantized(typ, N, K, 1000 + nb)
    x = synth.activations(2000 + nb, M, K)
    y_ref, bound = oracle.gemv(typ, W, N, K, x)
    for offset in (0, 2):
        y = run_gemv(pn, torch, dev, typ, dev_bytes(torch, dev, W, offset), N, K, x)
        assert_within(y, y_ref, bound)


@pytest.mark.parametrize("typ,N,nb", [
    (PN4T, 1, 65), (PN4T, 2, 100), (PN4T, 3, 272), (PN3T, 5, 70), (PN4T, 600, 65),
    (PN3T, 515, 66), (PN4T, 1031, 130), (PN4T, 97, 301)])
@pytest.mark.parametrize("M", [1, 2])
def test_gemv_long_rows(env, typ, N, nb, M):
    """Rows of more than 64 blocks at 1-2 tokens: pieces of (row pair, block) that start and end
    inside row pairs, an odd last row, fewer row pairs than workgroups and more."""
    pn, torch, dev = env
    G = oracle.PARAMS[typ][1]
    K = nb * G
    _, W = quantized(typ, N, K, 7000 + nb)
    x = synth.activations(7100 + nb, M, K)
    y_ref, bound = oracle.gemv(typ, W, N, K, x)
    for offset in (0, 2):
        y = run_gemv(pn, torch, dev, typ, dev_bytes(torch, dev, W, offset), N, K, x)
        assert_within(y, y_ref, bound)


# piece sizes (words per lane) each token count may run: the x of a piece must fit the registers
PIECES = {1: (8, 4, 2), 2: (4, 2), 3: (4, 2), 4: (2,)}


@pytest.mark.parametrize("typ,N,nb", [(PN3T, 37, 64), (PN4T, 19, 40), (PN4T, 45, 128), (PN3T, 9, 72),
                                      (PN4T, 300, 272), (PN3T, 21, 33), (PN4T, 40, 17)])
@pytest.mark.parametrize("M", [1, 2, 3, 4])
def test_gemv_every_piece_size(env, monkeypatch, typ, N, nb, M):
    """Each piece size the registers allow at M tokens, forced in turn (PN_GEMV_PIECE), at both
    alignments of W: whole and partial last chunks, and odd block counts (rows of two
    alignments, run as two launches)."""
    pn, torch, dev = env
    G = oracle.PARAMS[typ][1]
    K = nb * G
    _, W = quantized(typ, N, K, 8000 + nb)
    x = synth.activations(8100 + nb, M, K)
    y_ref, bound = oracle.gemv(typ, W, N, K, x)
    for P in PIECES[M]:
        monkeypatch.setenv("PN_GEMV_PIECE", str(P))
        for offset in (0, 2):
            y = run_gemv(pn, torch, dev, typ, dev_bytes(torch, dev, W, offset), N, K, x)
            assert_within(y, y_ref, bound)


def set_codes(W, typ, N, nb, elems, codes):
    """Rewrites, in every row, the code of element elems[b] of block b to codes[b]: code t of word i
    sits at bit BITS*(t>>1) + 16*(t&1) of the little-endian word at block byte 2 + 4i ("PN weight
    format", "Block layout")."""
    bits, G, cpw, _ = oracle.PARAMS[typ]
    blk = W.reshape(N, nb, 34)
    for b in range(nb):
        i, t = divmod(int(elems[b]), cpw)
        shift = bits * (t >> 1) + 16 * (t & 1)
        o = 2 + 4 * i
        word = sum(blk[:, b, o + q].astype(np.uint32) << np.uint32(8 * q) for q in range(4))
        mask = np.uint32(((1 << bits) - 1) << shift)
        word = (word & ~mask) | np.uint32(int(codes[b]) << shift)
        for q in range(4):
            blk[:, b, o + q] = ((word >> np.uint32(8 * q)) & np.uint32(0xFF)).astype(np.uint8)


@pytest.mark.parametrize("typ,nb", [(PN3T, 64), (PN4T, 80), (PN3T, 27), (PN4T, 272)])
@pytest.mark.parametrize("M", [1, 2, 3, 4])
@pytest.mark.parametrize("mag", [2.0 ** 12, 2.0 ** 16, 2.0 ** 19])
def test_gemv_dominant_x_on_code_near_z(env, monkeypatch, typ, nb, M, mag):
    """One x per block far larger than the rest (|x| in [1, 2) elsewhere), meeting a weight whose
    code is z (w = 0), z + 1 or z - 1: the bound 1e-5 * sum |w x| must hold however small the
    other products are against the large x ("PN weight format", "Value": each weight is exact, so
    code z contributes exactly nothing). Every piece size the token count allows, forced in turn;
    the element and the code offset vary from block to block, and over the tokens."""
    pn, torch, dev = env
    bits, G, cpw, z = oracle.PARAMS[typ]
    N, K = 48, nb * G
    _, W = quantized(typ, N, K, 8300 + nb)
    W = W.copy()
    elems = (np.arange(nb) * 37 + 11) % G
    offs = np.array([0, 1, -1])[np.arange(nb) % 3]
    set_codes(W, typ, N, nb, elems, z + offs)
    u = synth.uniform(8301 + nb, M * K).reshape(M, K)
    sgn = np.where(synth.uniform(8302 + nb, M * K).reshape(M, K) < 0.5, -1.0, 1.0)
    x = (1.0 + u) * sgn
    for m in range(M):
        x[m, np.arange(nb) * G + elems] = mag * (-1.0) ** m
    x = x.astype(np.float32)
    y_ref, bound = oracle.gemv(typ, W, N, K, x)
    for P in PIECES[M]:
        monkeypatch.setenv("PN_GEMV_PIECE", str(P))
        y = run_gemv(pn, torch, dev, typ, dev_bytes(torch, dev, W), N, K, x)
        assert_within(y, y_ref, bound)


@pytest.mark.parametrize("typ,nb", [(PN3T, 1), (PN3T, 3), (PN4T, 129)])
def test_decode_validate_ragged(env, typ, nb):
    pn, torch, dev = env
    G = oracle.PARAMS[typ][1]
    N, K = 11, nb * G
    _, W = quantized(typ, N, K, 3000 + nb)
    W = W.copy()
    W[3, 1] = 0x7C  # d of block 0 in row 3 becomes infinite
    if typ == PN3T:
        W[5, 34 * (nb - 1) + 33] |= 0x80  # bit 31 of the last word of row 5
    for offset in (0, 2):
        Wd = dev_bytes(torch, dev, W, offset)
        out = torch.empty((N, K), dtype=torch.float32, device=dev)
        pn.dequantize_rows(typ, Wd, N, K, out)
        ver = torch.full((N,), -1, dtype=torch.int32, device=dev)
        pn.validate_rows(typ, Wd, N, K, ver)
        torch.cuda.synchronize()
        assert_bits_equal(out.cpu().numpy(), oracle.dequantize_rows(typ, W, K))
        assert np.array_equal(ver.cpu().numpy(), oracle.validate_rows(typ, W, K))


def test_gemv_large_k_phases(env):
    """K large enough that x is staged in several LDS phases (M = 4)."""
    pn, torch, dev = env
    typ, N, K = PN3T, 24, 80 * 700
    _, W = quantized(typ, N, K, 4100)
    x = synth.activations(4101, 4, K)
    y = run_gemv(pn, torch, dev, typ, dev_bytes(torch, dev, W), N, K, x)
    y_ref, bound = oracle.gemv(typ, W, N, K, x)
    assert_within(y, y_ref, bound)


def test_empty_inputs_are_noops(env):
    pn, torch, dev = env
    _, W = quantized(PN3T, 8, 640, 5)
    Wd = dev_bytes(torch, dev, W)
    x = torch.ones((1, 640), dtype=torch.float32, device=dev)
    y = torch.full((1, 8), 7.0, dtype=torch.float32, device=dev)
    pn.gemv(PN3T, Wd, 0, 640, x, y)
    pn.gemv(PN3T, Wd, 8, 640, x, y, M=0)
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)
    with pytest.raises(pn.PNError):
        pn.gemv(PN3T, Wd, 8, 650, x, y)
    with pytest.raises(pn.PNError):
        pn.gemv(PN3T, Wd, 8, 640, x, y, M=17)  # rejected by the host check, before any launch


def test_invalid_rows_are_memory_safe(env):
    pn, torch, dev = env
    W, valid = config1()
    x = synth.activations(5, 4, 640)
    y = run_gemv(pn, torch, dev, PN3T, dev_bytes(torch, dev, W), 256, 640, x)
    assert np.all(np.isfinite(y[:, valid]))


# ---- config 2: pn4t 5120 x 6144, Laplace + outliers ------------------------------------------

@pytest.mark.slow
def test_config2_dequantize_and_gemv(env):
    pn, torch, dev = env
    N, K = 5120, 6144
    _, W = quantized(PN4T, N, K, 201, "laplace")
    Wd = dev_bytes(torch, dev, W)
    out = torch.empty((N, K), dtype=torch.float32, device=dev)
    pn.dequantize_rows(PN4T, Wd, N, K, out)
    torch.cuda.synchronize()
    assert_bits_equal(out.cpu().numpy(), oracle.dequantize_rows(PN4T, W, K))
    del out
    x = synth.activations(203, 1, K)
    y = run_gemv(pn, torch, dev, PN4T, Wd, N, K, x)
    y_ref, bound = oracle.gemv(PN4T, W, N, K, x)
    print("config2 worst err/bound", assert_within(y, y_ref, bound))


# ---- config 3: the MLP at M = 1 (full size) ----------------------------------------------------

@pytest.mark.slow
@pytest.mark.parametrize("name,typ,N,K,seed,xseed", [
    ("gate", PN3T, 17408, 5120, 301, 304), ("up", PN3T, 17408, 5120, 302, 304),
    ("down", PN4T, 5120, 17408, 303, 305)])
def test_config3_mlp_gemv(env, name, typ, N, K, seed, xseed):
    pn, torch, dev = env
    _, W = quantized(typ, N, K, seed)
    x = synth.activations(xseed, 1, K)
    y = run_gemv(pn, torch, dev, typ, dev_bytes(torch, dev, W), N, K, x)
    y_ref, bound = oracle.gemv(typ, W, N, K, x)
    print(name, "worst err/bound", assert_within(y, y_ref, bound))


@pytest.mark.slow
def test_config3_stacked_gate_up_every_row(env):
    """The launch the bench times: gate (seed 301) and up (seed 302) stacked by rows into one pn3t
    34816 x 5120 matrix at M = 1, every row against the oracle."""
    pn, torch, dev = env
    K = 5120
    _, Wg = quantized(PN3T, 17408, K, 301)
    _, Wu = quantized(PN3T, 17408, K, 302)
    W = np.concatenate([Wg, Wu])
    N = W.shape[0]
    x = synth.activations(304, 1, K)
    y = run_gemv(pn, torch, dev, PN3T, dev_bytes(torch, dev, W), N, K, x)
    y_ref, bound = oracle.gemv(PN3T, W, N, K, x)
    print("stacked gate+up worst err/bound", assert_within(y, y_ref, bound))


@pytest.mark.parametrize("typ,N,K,offset", [(PN3T, 24613, 5120, 0), (PN3T, 24613, 5120, 2),
                                             (PN4T, 36100, 4096, 0), (PN4T, 36101, 4096, 2)])
def test_gemv_one_token_ticket_groups(env, typ, N, K, offset):
    """One token on rows of one chunk (64 blocks) with enough rows per workgroup that its waves
    take their groups of rows from a counter as they free up (at least 3 groups per wave on 256
    compute units): ragged row counts, both alignments of W, every row against the oracle, and
    the same bits on a second call. The rows repeat a 2048-row oracle-quantized matrix."""
    pn, torch, dev = env
    _, Wb = quantized(typ, 2048, K, 950 + typ)
    W = np.ascontiguousarray(np.tile(Wb, ((N + 2047) // 2048, 1))[:N])
    x = synth.activations(960 + typ, 1, K)
    Wd = dev_bytes(torch, dev, W, offset)
    y = run_gemv(pn, torch, dev, typ, Wd, N, K, x)
    y2 = run_gemv(pn, torch, dev, typ, Wd, N, K, x)
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))
    y_ref, bound = oracle.gemv(typ, W, N, K, x)
    assert_within(y, y_ref, bound)


# ---- config 4: the decoder-layer set at M = 1..4 -------------------------------------------------

@pytest.mark.slow
@pytest.mark.parametrize("idx", range(len(LAYER_SET)))
def test_config4_layer_set(env, idx):
    pn, torch, dev = env
    N, K, typ, seed = LAYER_SET[idx]
    _, W = quantized(typ, N, K, seed)
    Wd = dev_bytes(torch, dev, W)
    x4 = synth.activations(409, 4, K)
    y_ref4, bound4 = oracle.gemv(typ, W, N, K, x4)
    for M in (1, 2, 3, 4):
        y = run_gemv(pn, torch, dev, typ, Wd, N, K, x4[:M])
        assert_within(y, y_ref4[:M], bound4[:M])


# ---- the reference quantizer on the GPU ----------------------------------------------------------

def adversarial_groups(typ):
    bits, G, cpw, z = oracle.PARAMS[typ]
    rows = []
    rows.append(np.zeros(G))
    rows.append(np.full(G, -0.0))
    rows.append(np.where(np.arange(G) == 3, 1e-9, 0.0))           # all candidates round to 0
    rows.append(np.where(np.arange(G) == 0, 3.0e38, 1.0))         # every candidate overflows
    rows.append(np.where(np.arange(G) == 5, np.nan, 0.5))
    rows.append(np.where(np.arange(G) == 7, -np.inf, 0.5))
    rows.append(np.linspace(-1, 1, G))                            # |min| == max
    rows.append(np.linspace(-1, 0.5, G))
    rows.append((np.arange(G) % 9 - 4) * 0.5 + 0.25)              # exact half-way codes
    rows.append(np.full(G, 6.1e-5))                               # subnormal-range scales
    rows.append(np.full(G, 65504.0 * 4))                          # near fp16 overflow
    rows.append(synth.normal_f32(77, G, 1e-4).astype(np.float64))
    rows.append(np.where(np.arange(G) % 2 == 0, 1.0, -1.0))
    return np.array(rows, dtype=np.float32)


@pytest.mark.parametrize("typ", [PN3T, PN4T])
def test_quantizer_bit_exact_adversarial(env, typ):
    pn, torch, dev = env
    G = oracle.PARAMS[typ][1]
    w = adversarial_groups(typ)
    # one row of 4 identical blocks per case, plus random rows
    w = np.concatenate([np.tile(w, (1, 4)), synth.gaussian_weights(55, 40, 4 * G),
                        synth.laplace_outlier_weights(56, 57, 40, 4 * G, 0.015, 0.01, 8.0)])
    W_ref, st_ref = oracle.quantize_rows(typ, w)
    wd = torch.from_numpy(w).to(dev)
    Wd = torch.zeros(W_ref.shape, dtype=torch.uint8, device=dev)
    st = torch.full((w.shape[0],), -1, dtype=torch.int32, device=dev)
    pn.quantize_rows(typ, wd, Wd, st)
    torch.cuda.synchronize()
    assert np.array_equal(Wd.cpu().numpy(), W_ref)
    assert np.array_equal(st.cpu().numpy(), st_ref)


@pytest.mark.slow
@pytest.mark.parametrize("typ,N,K,seed", [(PN3T, 17408, 5120, 301), (PN4T, 5120, 17408, 303),
                                          (PN4T, 5120, 6144, 201)])
def test_quantizer_bit_exact_full_size(env, typ, N, K, seed):
    pn, torch, dev = env
    w, W_ref = quantized(typ, N, K, seed, "laplace" if seed == 201 else "normal")
    wd = torch.from_numpy(w).to(dev)
    Wd = torch.zeros(W_ref.shape, dtype=torch.uint8, device=dev)
    pn.quantize_rows(typ, wd, Wd)
    torch.cuda.synchronize()
    got = Wd.cpu().numpy()
    mism = np.argwhere(got != W_ref)
    assert mism.size == 0, f"{len(mism)} bytes differ, first {mism[:4].tolist()}"
