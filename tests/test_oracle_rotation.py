"""Pins for the oracle's random-sign Hadamard rotation."""
import numpy as np
import scipy.linalg

import oracle


def test_page_worked_example(golden):
    g = golden("hadamard_trick1.txt")
    m = int(g["block"][0])
    x = np.array(g["input"])[None, :]
    y = oracle.rotate_rows(x, m, np.array(g["signs"]))[0]
    assert np.allclose(y, g["output"], rtol=0, atol=1e-12)
    assert np.isclose(np.sum(x * x), g["sum_of_squares"][0], atol=1e-12)
    assert np.isclose(np.sum(y * y), g["sum_of_squares"][0], atol=1e-12)


def test_sylvester_is_the_natural_order_hadamard():
    for m in (1, 2, 4, 8, 16, 64, 256):
        assert np.array_equal(oracle.sylvester(m), scipy.linalg.hadamard(m).astype(np.float64))


def _dense_R(n, m, signs):
    blocks = [scipy.linalg.hadamard(m) @ np.diag(signs[k * m:(k + 1) * m]) for k in range(n // m)]
    return scipy.linalg.block_diag(*blocks) / np.sqrt(m)


def test_blockwise_application_matches_dense_matrix():
    rng = np.random.default_rng(2)
    n, m = 32, 8
    signs = rng.choice([-1.0, 1.0], size=n)
    R = _dense_R(n, m, signs)
    M = rng.standard_normal((5, n))
    assert np.allclose(oracle.rotation_matrix(n, m, signs), R, atol=1e-15)
    assert np.allclose(oracle.rotate_rows(M, m, signs), M @ R.T, atol=1e-13)
    assert np.allclose(oracle.rotate_rows_inverse(M, m, signs), M @ R, atol=1e-13)
    H = rng.standard_normal((n, n))
    H = H + H.T
    assert np.allclose(oracle.rotate_sym(H, m, signs), R @ H @ R.T, atol=1e-12)


def test_rotation_invariants():
    rng = np.random.default_rng(3)
    n, m = 64, 16
    signs = rng.choice([-1.0, 1.0], size=n)
    R = oracle.rotation_matrix(n, m, signs)
    assert np.allclose(R @ R.T, np.eye(n), atol=1e-14)
    W = rng.standard_normal((6, n))
    X = rng.standard_normal((40, n))
    # the layer output is unchanged: W x = (W R^T)(R x)
    Wr = oracle.rotate_rows(W, m, signs)
    Xr = oracle.rotate_rows(X, m, signs)
    assert np.allclose(W @ X.T, Wr @ Xr.T, atol=1e-12)
    # rotating H0 equals the second moment of the rotated inputs
    H0 = oracle.second_moment(X)
    assert np.allclose(oracle.rotate_sym(H0, m, signs), oracle.second_moment(Xr), atol=1e-12)
    # lengths kept; inverse undoes the forward map
    assert np.allclose(np.sum(Wr * Wr, axis=1), np.sum(W * W, axis=1))
    assert np.allclose(oracle.rotate_rows_inverse(Wr, m, signs), W, atol=1e-13)


def test_rotation_spreads_an_outlier():
    x = np.zeros((1, 16))
    x[0, 3] = 4.0
    y = oracle.rotate_rows(x, 16, np.ones(16))
    assert np.allclose(np.abs(y), 1.0)
