"""Pins for the odd grid, nearest rounding and fp16 projection."""
import numpy as np
import pytest

import oracle


def test_levels_are_signed_odd_and_symmetric():
    assert sorted(oracle.level_of(np.arange(4), 3).tolist()) == [-3, -1, 1, 3]
    assert oracle.level_of(np.arange(8), 7).tolist() == [-7, -5, -3, -1, 1, 3, 5, 7]
    assert oracle.levels_count(2) == 3 and oracle.levels_count(3) == 7
    with pytest.raises(ValueError):
        oracle.levels_count(1)


@pytest.mark.parametrize("L", [3, 7])
def test_nearest_code_is_bruteforce_argmin(L):
    rng = np.random.default_rng(4)
    t = rng.uniform(-L - 3, L + 3, size=4000)
    lev = np.arange(-L, L + 1, 2)
    brute = np.argmin(np.abs(t[:, None] - lev[None, :]), axis=1)
    assert np.array_equal(oracle.nearest_code(t, L), brute)


def test_nearest_code_ties_and_clamp():
    assert oracle.level_of(oracle.nearest_code(0.0, 3), 3) == 1       # tie between -1 and 1 goes up
    assert oracle.level_of(oracle.nearest_code(2.0, 3), 3) == 3
    assert oracle.level_of(oracle.nearest_code(-2.0, 3), 3) == -1
    assert oracle.nearest_code(100.0, 3) == 3 and oracle.nearest_code(-100.0, 3) == 0


def test_fp16_rne_hand_cases():
    f = oracle.fp16_rne
    assert f(1 + 2.0 ** -11) == 1.0                       # tie -> even mantissa
    assert f(1 + 3 * 2.0 ** -11) == 1 + 2.0 ** -9         # tie -> even mantissa (up)
    assert f(1 + 2.0 ** -11 + 2.0 ** -30) == 1 + 2.0 ** -10   # just above the tie
    assert f(2.0 ** -25) == 0.0                           # subnormal tie -> 0
    assert f(3 * 2.0 ** -25) == 2.0 ** -23
    assert f(-(1 + 3 * 2.0 ** -11)) == -(1 + 2.0 ** -9)
    assert f(1.0e6) == 65504.0 and f(-1.0e6) == -65504.0


def test_fp16_rne_is_nearest():
    rng = np.random.default_rng(5)
    x = rng.uniform(1e-4, 10.0, size=2000)
    r = oracle.fp16_rne(x).astype(np.float16)
    up = np.nextafter(r, np.float16(np.inf)).astype(np.float64)
    dn = np.nextafter(r, np.float16(-np.inf)).astype(np.float64)
    d = np.abs(x - r.astype(np.float64))
    assert np.all(d <= np.abs(x - up)) and np.all(d <= np.abs(x - dn))


def test_dequant_hand_example():
    codes = np.array([[0, 1, 2, 3, 3, 2, 1, 0]])
    scales = np.array([[0.5, 2.0]])
    w = oracle.dequant(codes, scales, 2, 4)
    assert np.array_equal(w, [[-1.5, -0.5, 0.5, 1.5, 6.0, 2.0, -2.0, -6.0]])
