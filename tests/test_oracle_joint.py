"""Pins for the oracle's joint least-squares scale solve with a prior."""
import numpy as np
import pytest
import scipy.optimize

import oracle


def _problem(rng, rows=3, n=16, g=4, bits=2):
    L = 2 ** bits - 1
    A = rng.standard_normal((5 * n, n))
    A = A + 0.8 * A[:, :1]
    H = A.T @ A / (5 * n)
    H = H + 0.01 * np.trace(H) / n * np.eye(n)
    codes = rng.integers(0, L + 1, size=(rows, n))
    T = rng.standard_normal((rows, n))
    s0 = rng.uniform(0.2, 1.0, size=(rows, n // g))
    return H, codes, T, s0, L


def _dense_Q(lev, g):
    n = lev.shape[0]
    Q = np.zeros((n, n // g))
    for j in range(n):
        Q[j, j // g] = lev[j]
    return Q


def _objective(s, Q, H, t, s0, lam):
    G = Q.T @ H @ Q
    mu = np.trace(G) / Q.shape[1]
    d = t - Q @ s
    return d @ H @ d + lam * mu * np.sum((s - s0) ** 2)


def test_row_gram_equals_QtHQ():
    rng = np.random.default_rng(20)
    H, codes, _, _, L = _problem(rng)
    lev = oracle.level_of(codes[0], L).astype(float)
    Q = _dense_Q(lev, 4)
    assert np.allclose(oracle.row_gram(lev, H, 4), Q.T @ H @ Q, atol=1e-13)


@pytest.mark.parametrize("lam", [0.01, 0.5])
def test_solution_has_zero_gradient(lam):
    rng = np.random.default_rng(21)
    H, codes, T, s0, L = _problem(rng)
    _, s = oracle.joint_scales(codes, 2, 4, H, T, s0, lam)
    for r in range(codes.shape[0]):
        Q = _dense_Q(oracle.level_of(codes[r], L).astype(float), 4)
        f = lambda x: _objective(x, Q, H, T[r], s0[r], lam)
        eps = 1e-6
        grad = np.array([(f(s[r] + eps * e) - f(s[r] - eps * e)) / (2 * eps) for e in np.eye(s.shape[1])])
        grad0 = np.array([(f(s0[r] + eps * e) - f(s0[r] - eps * e)) / (2 * eps) for e in np.eye(s.shape[1])])
        assert np.linalg.norm(grad) < 1e-7 * np.linalg.norm(grad0)


def test_matches_a_numerical_minimiser():
    rng = np.random.default_rng(22)
    H, codes, T, s0, L = _problem(rng, rows=2)
    _, s = oracle.joint_scales(codes, 2, 4, H, T, s0, 0.01)
    for r in range(2):
        Q = _dense_Q(oracle.level_of(codes[r], L).astype(float), 4)
        res = scipy.optimize.minimize(lambda x: _objective(x, Q, H, T[r], s0[r], 0.01), s0[r],
                                      method="BFGS", options={"gtol": 1e-12})
        assert np.allclose(res.x, s[r], rtol=1e-5, atol=1e-7)


def test_ridge_special_case_identity_H_one_block():
    rng = np.random.default_rng(23)
    n = 8
    codes = rng.integers(0, 4, size=(1, n))
    lev = 2 * codes[0] - 3
    t = rng.standard_normal((1, n))
    s0 = np.array([[0.7]])
    lam = 0.01
    mu = float(lev @ lev)
    expect = (lev @ t[0] + lam * mu * 0.7) / (lev @ lev + lam * mu)
    _, s = oracle.joint_scales(codes, 2, n, np.eye(n), t, s0, lam)
    assert np.isclose(s[0, 0], expect, rtol=1e-14)


def test_lambda_zero_is_weighted_least_squares():
    rng = np.random.default_rng(24)
    H, codes, T, s0, L = _problem(rng, rows=1)
    C = np.linalg.cholesky(H).T                   # H = C^T C
    Q = _dense_Q(oracle.level_of(codes[0], L).astype(float), 4)
    ls = np.linalg.lstsq(C @ Q, C @ T[0], rcond=None)[0]
    _, s = oracle.joint_scales(codes, 2, 4, H, T, s0, 0.0)
    assert np.allclose(s[0], ls, rtol=1e-10)


def test_dequantised_target_is_a_fixed_point():
    rng = np.random.default_rng(25)
    H, codes, _, s0, L = _problem(rng)
    s0 = oracle.fp16_rne(s0)
    T = oracle.dequant(codes, s0, 2, 4)
    s16, s = oracle.joint_scales(codes, 2, 4, H, T, s0, 0.01)
    assert np.allclose(s, s0, rtol=1e-12)
    assert np.array_equal(s16, s0)


def test_projection_is_fp16_rne_of_the_solution():
    rng = np.random.default_rng(26)
    H, codes, T, s0, L = _problem(rng)
    s16, s = oracle.joint_scales(codes, 2, 4, H, T, s0, 0.01)
    assert np.array_equal(s16, s.astype(np.float16).astype(np.float64))


def test_joint_scales_do_not_increase_the_weighted_error():
    """f(s*) <= f(s0) = (t - Q s0)^T H (t - Q s0) and the error term at s* is below f(s*)."""
    rng = np.random.default_rng(27)
    H, codes, T, s0, L = _problem(rng)
    _, s = oracle.joint_scales(codes, 2, 4, H, T, s0, 0.01)
    e_new = oracle.proxy_loss(T, oracle.dequant(codes, s, 2, 4), H)
    e_old = oracle.proxy_loss(T, oracle.dequant(codes, s0, 2, 4), H)
    assert e_new <= e_old
