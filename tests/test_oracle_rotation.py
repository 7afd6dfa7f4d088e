"""Pins of the oracle's fixed rotation (hadamard_rotate, reading R12: the
Sylvester-ordered Hadamard matrix, block-diagonal, scaled to be orthogonal;
[OptRot] abstract and Figure 1: a fusible rotation applied before GPTQ)."""
import math

import numpy as np
import pytest
import scipy.linalg

import oracle as O


def test_sylvester_order_4_by_hand():
    # H_2 = [[1, 1], [1, -1]], H_4 = [[H_2, H_2], [H_2, -H_2]] written out
    H4 = np.array([[1, 1, 1, 1],
                   [1, -1, 1, -1],
                   [1, 1, -1, -1],
                   [1, -1, -1, 1]], dtype=np.float64)
    np.testing.assert_array_equal(O.hadamard_matrix(4), H4)
    np.testing.assert_array_equal(O.hadamard_matrix(1), np.ones((1, 1)))


@pytest.mark.parametrize("b", [2, 8, 64, 512])
def test_matches_the_library_hadamard(b):
    np.testing.assert_array_equal(O.hadamard_matrix(b), scipy.linalg.hadamard(b))


@pytest.mark.parametrize("n,block", [(64, 0), (96, 32), (256, 16), (1024, 0)])
def test_rotation_is_orthogonal_and_an_involution(n, block):
    rng = np.random.default_rng(n + block)
    M = rng.standard_normal((5, n))
    b = O.default_rotation_block(n) if block <= 0 else block
    R = O.hadamard_rotate(np.eye(n), block)
    np.testing.assert_allclose(R @ R.T, np.eye(n), atol=1e-13)
    np.testing.assert_allclose(R, R.T, atol=0)  # Sylvester Hadamard blocks are symmetric
    Mr = O.hadamard_rotate(M, block)
    np.testing.assert_allclose(Mr, M @ R, atol=1e-12)
    np.testing.assert_allclose(np.linalg.norm(Mr, axis=1), np.linalg.norm(M, axis=1), rtol=1e-13)
    np.testing.assert_allclose(O.hadamard_rotate(Mr, block), M, atol=1e-12)
    # block-diagonal: a row living in one segment stays in it
    e = np.zeros((1, n))
    e[0, b + 3 if n > b else 3] = 1.0
    er = O.hadamard_rotate(e, block)
    seg = (b + 3) // b if n > b else 0
    assert np.count_nonzero(er) == b
    assert np.all(er[0, seg * b:(seg + 1) * b] != 0)
    # a single spike becomes flat: every entry of its segment is +-1/sqrt(b)
    np.testing.assert_allclose(np.abs(er[0, seg * b:(seg + 1) * b]), 1 / math.sqrt(b), rtol=1e-14)


def test_default_blocks():
    assert O.default_rotation_block(4096) == 4096
    assert O.default_rotation_block(11008) == 256   # 11008 = 2^8 * 43
    assert O.default_rotation_block(49152) == 4096  # capped
    assert O.default_rotation_block(12) == 4
    with pytest.raises(ValueError):
        O.hadamard_rotate(np.ones((1, 48)), 32)  # 32 does not divide 48


def test_fusible_layer_output_and_hessian():
    """X' W'^T = X W^T, H' = R^T H R, and the layer loss of a quantized
    rotated weight measured in either basis is the same."""
    rng = np.random.default_rng(3)
    m, n, T = 12, 64, 300
    W = rng.normal(0, 0.02, (m, n))
    X = rng.standard_normal((T, n)) * rng.lognormal(0, 1, n)
    R = O.hadamard_rotate(np.eye(n))
    Wr, Xr = O.hadamard_rotate(W), O.hadamard_rotate(X)
    np.testing.assert_allclose(Xr @ Wr.T, X @ W.T, atol=1e-12)
    H, Hr = O.hessian([X]), O.hessian([Xr])
    np.testing.assert_allclose(Hr, R.T @ H @ R, rtol=1e-10, atol=1e-9 * np.abs(H).max())
    Hd, _ = O.damp(Hr, 0.01)
    U, info = O.inverse_cholesky_upper(Hd)
    assert info == 0
    g = O.gptq_quantize(Wr, U, 4, 16, 16)
    back = g["What"] @ R.T  # the quantized layer in the original basis
    assert O.layer_loss(Wr, g["What"], Hr) == pytest.approx(O.layer_loss(W, back, H), rel=1e-9)


def test_rotation_spreads_outliers():
    """A weight matrix with a few large entries becomes far more incoherent
    after the rotation ([OptRot] Theorem 3.1 bounds the error by mu_W)."""
    rng = np.random.default_rng(4)
    W = rng.normal(0, 0.02, (64, 256))
    W[rng.integers(0, 64, 8), rng.integers(0, 256, 8)] = 1.0
    mu, mur = O.weight_incoherence(W), O.weight_incoherence(O.hadamard_rotate(W))
    assert mur < 0.5 * mu
    assert O.weight_incoherence(np.ones((4, 4))) == pytest.approx(1.0)
