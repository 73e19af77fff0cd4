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
