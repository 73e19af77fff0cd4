"""Pins for the oracle's second moment and damping (closed forms, brute force, invariants)."""
import numpy as np

import oracle


def test_second_moment_hand_example():
    X = np.array([[1.0, 2.0], [3.0, 4.0]])
    # (1/2) * [[1+9, 2+12], [2+12, 4+16]]
    assert np.array_equal(oracle.second_moment(X), np.array([[5.0, 7.0], [7.0, 10.0]]))


def test_second_moment_is_mean_of_outer_products():
    rng = np.random.default_rng(0)
    X = rng.integers(-4, 5, size=(7, 5)).astype(np.float64)
    acc = [[0.0] * 5 for _ in range(5)]
    for row in X.tolist():
        for i in range(5):
            for j in range(5):
                acc[i][j] += row[i] * row[j]
    brute = np.array(acc) / 7.0
    assert np.array_equal(oracle.second_moment(X), brute)


def test_second_moment_invariants():
    rng = np.random.default_rng(1)
    X = rng.standard_normal((50, 12))
    H0 = oracle.second_moment(X)
    assert np.array_equal(H0, H0.T)
    assert np.linalg.eigvalsh(H0).min() > -1e-12
    assert np.isclose(np.trace(H0), np.sum(X * X) / 50, rtol=1e-13)


def test_damping_hand_example():
    H, delta = oracle.damp(np.array([[5.0, 7.0], [7.0, 10.0]]), 0.01)
    assert np.isclose(delta, 0.075)
    assert np.allclose(H, [[5.075, 7.0], [7.0, 10.075]], rtol=0, atol=1e-15)


def test_damping_uses_stored_dimension_and_reaches_padding():
    H0 = oracle.pad_square(np.array([[5.0, 7.0], [7.0, 10.0]]), 4)
    H, delta = oracle.damp(H0, 0.01)
    assert np.isclose(delta, 0.01 * 15.0 / 4)
    assert np.allclose(np.diag(H), [5.0 + delta, 10.0 + delta, delta, delta])
    assert np.all(H[2:, :2] == 0) and np.all(H[:2, 2:] == 0)


def test_chunked_second_moment_and_single_entries_match_the_hand_sum():
    rng = np.random.default_rng(2)
    X = rng.integers(-3, 4, size=(9, 4)).astype(np.float64)
    brute = np.zeros((4, 4))
    for row in X.tolist():
        for i in range(4):
            for j in range(4):
                brute[i, j] += row[i] * row[j]
    H0 = oracle.second_moment_chunks([X[:2], X[2:7], X[7:]])
    assert np.array_equal(H0, brute / 9.0)
    pairs = [(0, 0), (3, 1), (2, 3)]
    assert np.array_equal(oracle.sum_of_products(X, pairs), [brute[i, j] for i, j in pairs])
