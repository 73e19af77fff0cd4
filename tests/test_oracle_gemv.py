"""Pins for the oracle's packed-module product (container layout of the Wringer model cards)."""
import numpy as np

import oracle


def _module(rng, rows, n, bits, g):
    L = 2 ** bits - 1
    codes = rng.integers(0, L + 1, size=(rows, n))
    scales = oracle.fp16_rne(rng.uniform(1e-3, 3e-2, size=(rows, n // g)))
    return codes, scales, oracle.pack(codes, scales, bits, g)


def test_without_rotation_explicit_loops():
    rng = np.random.default_rng(50)
    rows, n, bits, g = 3, 16, 2, 8
    codes, scales, buf = _module(rng, rows, n, bits, g)
    X = rng.integers(-4, 5, size=(2, 12)).astype(np.float64)
    Y = oracle.packed_gemv(buf, rows, n, bits, g, 0, None, X)
    for b in range(2):
        for r in range(rows):
            acc = sum((2 * codes[r, j] - 3) * scales[r, j // g] * X[b, j] for j in range(12))
            assert np.isclose(Y[b, r], acc, rtol=1e-14, atol=1e-18)


def test_rotated_input_equals_the_materialized_weights_times_the_input():
    """W_q R x computed two ways: rotating the input (the product) or materializing the weights in
    the input basis (rows v -> R^T v) and multiplying with the unrotated input."""
    rng = np.random.default_rng(51)
    for rows, n, n_in, bits, g, m in [(5, 512, 500, 2, 64, 128), (4, 1024, 1024, 3, 32, 1024), (3, 96, 90, 4, 32, 32)]:
        codes, scales, buf = _module(rng, rows, n, bits, g)
        signs = rng.choice([-1.0, 1.0], size=n)
        X = rng.normal(size=(3, n_in))
        Y = oracle.packed_gemv(buf, rows, n, bits, g, m, signs, X)
        Wm = oracle.materialize_exact(buf, rows, n, bits, g, m, signs, n_in)
        assert np.allclose(Y, X @ Wm.T, rtol=1e-12, atol=1e-14)
