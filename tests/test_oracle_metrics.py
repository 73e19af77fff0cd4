"""Pins for the measures the parity tests compare with (proxy loss, ledger)."""
import numpy as np

import oracle


def test_proxy_loss_hand_computed_2x2():
    """W - W_hat = [[1, 1], [-1, 0]] with H0 = [[2, 1], [1, 3]]: row 1 gives 2 + 2 + 3 = 7,
    row 2 gives 2, total 9 (worked by hand)."""
    W = np.array([[1.0, 2.0], [0.0, 1.0]])
    W_hat = np.array([[0.0, 1.0], [1.0, 1.0]])
    H0 = np.array([[2.0, 1.0], [1.0, 3.0]])
    assert oracle.proxy_loss(W, W_hat, H0) == 9.0


def test_proxy_loss_is_output_error_energy():
    """tr(dW H0 dW^T) with H0 = X^T X / N is the mean squared output error ||X dW^T||^2 / N."""
    rng = np.random.default_rng(5)
    X = rng.standard_normal((40, 6))
    W = rng.standard_normal((3, 6))
    W_hat = W + 0.1 * rng.standard_normal((3, 6))
    H0 = oracle.second_moment(X)
    direct = np.sum((X @ (W - W_hat).T) ** 2) / 40
    assert np.isclose(oracle.proxy_loss(W, W_hat, H0), direct, rtol=1e-12)


def test_grid_distance_hand_computed():
    """T = [1, 2] against one block of level +1 (code 2 of 2 bits) at scale 1: residual [0, 1],
    relative distance 1 / sqrt(5)."""
    d = oracle.grid_distance(np.array([[1.0, 2.0]]), np.array([[2, 2]]), np.array([[1.0]]), 2, 2)
    assert abs(d - 1.0 / np.sqrt(5.0)) < 1e-15


def test_code_disagreement_hand_computed():
    assert oracle.code_disagreement(np.array([[0, 1, 2, 3]]), np.array([[0, 1, 3, 3]])) == 0.25
    assert oracle.code_disagreement(np.zeros((3, 5)), np.zeros((3, 5))) == 0.0


def test_projection_ulp_moves_hand_computed():
    """Two weights, one block each.  Level +1 at s = 0.10034: its fp16 scale is 1644 * 2^-14 =
    0.100341796875, which is 205.5 bf16 quanta (2^-11) -- a tie, rounded to the even 206 -- while
    s itself is 205.496 quanta, rounded to 205: the projection moves this weight by one bf16 ulp.
    Level -3 at s = 0.2: fp16(0.2) = 0.199951171875, so -0.599853515625 (153.56 quanta of 2^-8)
    against -0.6 (153.6 quanta): both round to 154, no move.  Share 1/2."""
    s_raw = np.array([[0.10034, 0.2]])
    s16 = oracle.fp16_rne(s_raw)
    assert s16[0, 0] == 1644 * 2.0 ** -14 and s16[0, 1] == 0.199951171875
    codes = np.array([[2, 0]])                        # levels +1 and -3 with L = 3
    assert oracle.projection_ulp_moves(codes, s16, s_raw, 2, 1) == 0.5
    assert oracle.projection_ulp_moves(codes, s16, s16, 2, 1) == 0.0


def test_grid_representation_keeps_a_grid_point():
    """Weights already on the grid (every block holds a level +-L, scales fp16): the nearest codes
    are the codes and the joint solve returns the scales (zero residual at the prior's centre)."""
    rng = np.random.default_rng(9)
    rows, n, g = 4, 32, 8
    codes = rng.integers(0, 4, size=(rows, n))
    codes[:, ::g] = 3
    s = oracle.fp16_rne(rng.uniform(0.1, 0.4, size=(rows, n // g)))
    X = rng.standard_normal((4 * n, n))
    H = X.T @ X / (4 * n) + 0.05 * np.eye(n)
    T = oracle.dequant(codes, s, 2, g)
    c2, s16, s_raw = oracle.grid_representation(T, s, 2, g, H, 0.01)
    assert np.array_equal(c2, codes) and np.array_equal(s16, s)
    assert oracle.grid_distance(T, c2, s16, 2, g) == 0.0
