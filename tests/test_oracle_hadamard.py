"""Pins of the oracle's Hadamard rotation of the activations ("PN weight format", "Files that use
PN": the model rotates the activations that reach the PN weights with a Hadamard transform).

The page fixes neither the order nor the normalisation; the reading is the orthonormal
Sylvester-ordered Walsh-Hadamard matrix on consecutive slices of B elements (B a power of two
dividing K). What pins the oracle other than itself: scipy's own construction of the Sylvester
matrix, the textbook H_2 and H_4 written out by hand, the involution and norm preservation of an
orthonormal symmetric matrix, and, for the rotated GEMV, a dense product over the decoded weights.
"""
import numpy as np
import pytest
import scipy.linalg

import oracle
import synth
from gpu_cases import PN3T, PN4T, quantized


def slices_ref(x, B):
    H = scipy.linalg.hadamard(B).astype(np.float64) / np.sqrt(B)
    M, K = x.shape
    xs = x.astype(np.float64).reshape(M, K // B, B)
    return np.einsum("ij,mbj->mbi", H, xs).reshape(M, K)


@pytest.mark.parametrize("B,K", [(2, 6), (4, 8), (8, 64), (64, 320), (256, 1280), (1024, 2048),
                                 (1024, 5120)])
def test_matches_library_sylvester(B, K):
    x = synth.activations(700 + B, 3, K)
    out, mass = oracle.hadamard(x, B)
    ref = slices_ref(x, B)
    assert np.all(np.abs(out - ref) <= 1e-12 * mass)


def test_textbook_h2_h4():
    h2 = np.array([[1, 1], [1, -1]], dtype=np.float64) / np.sqrt(2.0)
    h4 = np.array([[1, 1, 1, 1],
                   [1, -1, 1, -1],
                   [1, 1, -1, -1],
                   [1, -1, -1, 1]], dtype=np.float64) / 2.0
    x = np.array([[3.0, -1.0, 0.5, 8.0]], dtype=np.float32)
    out2, _ = oracle.hadamard(x, 2)
    assert np.allclose(out2[0], np.concatenate([h2 @ x[0, :2], h2 @ x[0, 2:]]), rtol=0, atol=1e-15)
    out4, _ = oracle.hadamard(x, 4)
    assert np.array_equal(out4[0], h4 @ x[0].astype(np.float64))  # halves and small integers: exact


@pytest.mark.parametrize("B", [2, 16, 128, 1024])
def test_involution_and_norm(B):
    K = 4 * B if B < 1024 else 2048
    x = synth.activations(800 + B, 2, K).astype(np.float64)
    out, mass = oracle.hadamard(x, B)
    back, _ = oracle.hadamard(out, B)
    assert np.all(np.abs(back - x) <= 1e-12 * np.abs(x).sum())
    n0 = np.linalg.norm(x.reshape(2, -1, B), axis=2)
    n1 = np.linalg.norm(out.reshape(2, -1, B), axis=2)
    assert np.allclose(n0, n1, rtol=1e-13, atol=0)
    # mass: the slice's sum of |x| over sqrt(B), the same for every element of the slice
    ref = np.repeat(np.abs(x).reshape(2, -1, B).sum(axis=2) / np.sqrt(B), B, axis=1)
    assert np.allclose(mass, ref, rtol=1e-14, atol=0)


def test_one_hot_gives_a_column():
    B, K = 64, 128
    for j in (0, 1, 37, 63, 64 + 5):
        x = np.zeros((1, K), np.float32)
        x[0, j] = 1.0
        out, _ = oracle.hadamard(x, B)
        H = scipy.linalg.hadamard(B) / 8.0
        col = np.zeros(K)
        base = (j // B) * B
        col[base:base + B] = H[:, j - base]
        assert np.array_equal(out[0], col)  # entries +-1/8, exact


def test_rejects_bad_block():
    x = np.zeros((1, 96), np.float32)
    for B in (0, 3, 12, 64, 192):
        with pytest.raises(ValueError):
            oracle.hadamard(x, B)


@pytest.mark.parametrize("typ,N,K,B", [(PN3T, 9, 640, 128), (PN4T, 7, 512, 512), (PN3T, 5, 1280, 256)])
def test_rotated_gemv_matches_dense(typ, N, K, B):
    _, W = quantized(typ, N, K, 910 + B)
    x = synth.activations(920 + B, 3, K)
    y, bound, rbound = oracle.gemv_hadamard(typ, W, N, K, x, B)
    deq = oracle.dequantize_rows(typ, W, K).astype(np.float64)
    xr = slices_ref(x, B)
    y_ref = xr @ deq.T
    assert np.all(np.abs(y - y_ref) <= 1e-12 * bound)
    assert np.allclose(bound, np.abs(xr) @ np.abs(deq).T, rtol=1e-12, atol=0)
    mass = np.repeat(np.abs(x.astype(np.float64)).reshape(3, -1, B).sum(axis=2) / np.sqrt(B), B, axis=1)
    assert np.allclose(rbound, mass @ np.abs(deq).T, rtol=1e-12, atol=0)
    # the unrotated GEMV of the rotated x agrees too (same decode, same sum)
    y2, b2 = oracle.gemv(typ, W, N, K, xr.astype(np.float32))
    assert np.all(np.abs(y2 - y) <= 1e-6 * bound + 1e-12)
