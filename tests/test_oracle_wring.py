"""Pins for the oracle's wring: target, nearest-point recode, fixed point."""
import numpy as np

import oracle


def _setup(rng, rows=4, n=16, g=8, bits=2):
    L = 2 ** bits - 1
    A_ = rng.standard_normal((4 * n, n))
    H = A_.T @ A_ / (4 * n) + 0.05 * np.eye(n)
    codes = rng.integers(0, L + 1, size=(rows, n))
    scales = oracle.fp16_rne(rng.uniform(0.1, 0.5, size=(rows, n // g)))
    return H, codes, scales, L


def test_target_formula_explicit_loops():
    rng = np.random.default_rng(30)
    H, codes, scales, L = _setup(rng, rows=3, n=8, g=4)
    B = rng.standard_normal((3, 2))
    A = rng.standard_normal((2, 8))
    alpha = 5.0
    Wp = oracle.wring_target(codes, scales, 2, 4, B, A, alpha)
    for i in range(3):
        for j in range(8):
            expect = (2 * codes[i, j] - 3) * scales[i, j // 4] + alpha / 2 * sum(B[i, k] * A[k, j] for k in range(2))
            assert np.isclose(Wp[i, j], expect, rtol=1e-14, atol=1e-15)


def test_recode_is_the_nearest_grid_point():
    rng = np.random.default_rng(31)
    for bits in (2, 3):
        H, codes, scales, L = _setup(rng, bits=bits)
        B = 0.3 * rng.standard_normal((4, 3))
        A = 0.3 * rng.standard_normal((3, 16))
        out = oracle.wring(codes, scales, bits, 8, B, A, 3.0, H, 0.01)
        srep = np.repeat(scales, 8, axis=1)
        lev = np.arange(-L, L + 1, 2)
        brute = np.argmin(np.abs(out["target"][:, :, None] - lev[None, None, :] * srep[:, :, None]), axis=2)
        assert np.array_equal(out["codes"], brute)


def test_zero_adapter_is_a_fixed_point():
    rng = np.random.default_rng(32)
    H, codes, scales, L = _setup(rng)
    out = oracle.wring(codes, scales, 2, 8, np.zeros((4, 3)), np.zeros((3, 16)), 3.0, H, 0.01)
    assert np.array_equal(out["codes"], codes)
    assert np.array_equal(out["scales"], scales)


def test_wring_fits_the_watered_target_better_than_the_old_point():
    """The new codes/scales sit closer to W' (in the H metric) than the dequantised old point plus nothing."""
    rng = np.random.default_rng(33)
    H, codes, scales, L = _setup(rng, rows=8, n=32)
    B = 0.4 * rng.standard_normal((8, 4))
    A = 0.4 * rng.standard_normal((4, 32))
    out = oracle.wring(codes, scales, 2, 8, B, A, 4.0, H, 0.01)
    new = oracle.proxy_loss(out["target"], oracle.dequant(out["codes"], out["scales"], 2, 8), H)
    old = oracle.proxy_loss(out["target"], oracle.dequant(codes, scales, 2, 8), H)
    assert new < old
