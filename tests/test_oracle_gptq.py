"""Pins for the oracle's GPTQ / LDLQ sweep: the page's toy, closed-form compensation, LDLQ, diagonal H."""
import itertools

import numpy as np
import pytest

import oracle


def _spd(n, rng, corr=0.9):
    A = rng.standard_normal((4 * n, n))
    A = A + corr * A[:, :1]                      # strongly correlated inputs
    H = A.T @ A / (4 * n)
    return H + 0.01 * np.trace(H) / n * np.eye(n)


def test_page_toy_unit_feedback(golden):
    g = golden("feedback_toy_trick2.txt")
    H = np.array(g["H_unit_feedback"]).reshape(3, 3)
    q, pre = oracle.integer_feedback_round(np.array(g["weights"]), H)
    assert np.array_equal(q, g["feedback_rounding"])
    assert np.allclose(pre, g["feedback_pre_values"], atol=1e-12)


def test_page_toy_near_equal_inputs(golden):
    g = golden("feedback_toy_trick2.txt")
    H = np.ones((3, 3)) + 1e-6 * np.eye(3)
    q, pre = oracle.integer_feedback_round(np.array(g["weights"]), H)
    assert np.array_equal(q, g["feedback_rounding"])
    assert np.allclose(pre, g["near_equal_pre_values"], atol=1e-5)
    assert abs(np.sum(q) - 1.2) < abs(np.sum(g["plain_rounding"]) - 1.2)


def test_page_toy_uncorrelated_inputs_give_plain_rounding(golden):
    g = golden("feedback_toy_trick2.txt")
    q, _ = oracle.integer_feedback_round(np.array(g["weights"]), np.diag([1.0, 2.0, 3.0]))
    assert np.array_equal(q, g["plain_rounding"])


def test_factor_is_upper_cholesky_of_inverse():
    rng = np.random.default_rng(6)
    H = _spd(20, rng)
    U = oracle.upper_cholesky_of_inverse(H)
    assert np.allclose(np.tril(U, -1), 0) and np.all(np.diag(U) > 0)
    assert np.allclose(U.T @ U @ H, np.eye(20), atol=1e-10)


@pytest.mark.parametrize("bits", [2, 3])
def test_diagonal_H_reduces_to_plain_rounding(bits):
    rng = np.random.default_rng(7)
    rows, n, g = 9, 48, 16
    L = 2 ** bits - 1
    W = rng.standard_normal((rows, n))
    H = np.diag(rng.uniform(0.5, 2.0, size=n))
    out = oracle.gptq_sweep(W, H, bits, g)
    # plain rounding with absmax fp16 scales of the untouched weights, by brute force over the levels
    s = np.array([[np.float16(np.max(np.abs(W[r, b * g:(b + 1) * g])) / L) for b in range(n // g)]
                  for r in range(rows)], dtype=np.float64)
    lev = np.arange(-L, L + 1, 2)
    srep = np.repeat(s, g, axis=1)
    rtn = np.argmin(np.abs(W[:, :, None] - lev[None, None, :] * srep[:, :, None]), axis=2)
    assert np.array_equal(out["scales"], s)
    assert np.array_equal(out["codes"], rtn)


def _obs_compensation(W, H, Qvals, k):
    """Values of columns k.. after optimally compensating the quantized columns 0..k-1 (closed form)."""
    F = slice(k, None)
    Qs = slice(0, k)
    if k == 0:
        return W[:, F].copy()
    D = W[:, Qs] - Qvals[:, Qs]
    return W[:, F] + np.linalg.solve(H[F, F], H[F, Qs] @ D.T).T


@pytest.mark.parametrize("bits", [2, 3])
def test_sweep_values_are_the_optimal_compensation(bits):
    rng = np.random.default_rng(8)
    rows, n, g = 4, 24, 8
    L = 2 ** bits - 1
    W = rng.standard_normal((rows, n))
    H = _spd(n, rng)
    out = oracle.gptq_sweep(W, H, bits, g)
    Qvals = oracle.dequant(out["codes"], out["scales"], bits, g)
    for k in range(n):
        v = _obs_compensation(W, H, Qvals, k)
        s = out["scales"][:, k // g]
        assert np.allclose(out["t"][:, k] * s, v[:, 0], rtol=1e-9, atol=1e-11)
        if k % g == 0:
            expect = np.array([np.float16(x) for x in np.max(np.abs(v[:, :g]), axis=1) / L], dtype=np.float64)
            assert np.array_equal(s, expect)


def test_ldlq_pull_form_gives_the_same_codes():
    """LDLQ: H = M D M^T with M unit upper; q_k = Q(w_k + sum_{j<k} (w_j - q_j) M_jk)."""
    rng = np.random.default_rng(9)
    rows, n, g, bits = 16, 48, 16, 2
    L = 3
    W = 0.02 * rng.standard_normal((rows, n))
    H = _spd(n, rng)
    out = oracle.gptq_sweep(W, H, bits, g)
    J = np.eye(n)[::-1]
    V = J @ np.linalg.cholesky(J @ H @ J) @ J          # H = V V^T, V upper
    M = V / np.diag(V)[None, :]                        # unit upper, D = diag(V)^2
    assert np.allclose(M @ np.diag(np.diag(V) ** 2) @ M.T, H, atol=1e-12)
    srep = np.repeat(out["scales"], g, axis=1)
    q = np.zeros_like(W)
    codes = np.zeros((rows, n), dtype=np.int64)
    for k in range(n):
        v = W[:, k] + (W[:, :k] - q[:, :k]) @ M[:k, k]
        lev = np.arange(-L, L + 1, 2)
        c = np.argmin(np.abs(v[:, None] - lev[None, :] * srep[:, k:k + 1]), axis=1)
        codes[:, k] = c
        q[:, k] = lev[c] * srep[:, k]
    assert np.array_equal(codes, out["codes"])


def test_per_row_bits_match_row_by_row_sweeps():
    rng = np.random.default_rng(10)
    rows, n, g = 6, 32, 8
    W = rng.standard_normal((rows, n))
    H = _spd(n, rng)
    bits = np.array([2, 3, 2, 3, 3, 2])
    out = oracle.gptq_sweep(W, H, bits, g)
    for r in range(rows):
        one = oracle.gptq_sweep(W[r:r + 1], H, int(bits[r]), g)
        assert np.array_equal(one["codes"][0], out["codes"][r])
        assert np.array_equal(one["scales"][0], out["scales"][r])


def test_zero_block_gets_zero_scale_and_dequantises_to_zero():
    rng = np.random.default_rng(11)
    W = rng.standard_normal((2, 16))
    W[0, :8] = 0.0
    H = np.eye(16)
    out = oracle.gptq_sweep(W, H, 2, 8)
    assert out["scales"][0, 0] == 0.0
    assert np.all(out["codes"][0, :8] == 2)
    assert np.all(oracle.dequant(out["codes"], out["scales"], 2, 8)[0, :8] == 0.0)


def test_sweep_loss_not_below_bruteforce_minimum():
    """Sanity bound: over all 4^6 code vectors with the sweep's scales, none beats the global minimum."""
    rng = np.random.default_rng(12)
    n, g = 6, 6
    W = rng.standard_normal((1, n))
    H = _spd(n, rng)
    out = oracle.gptq_sweep(W, H, 2, g)
    s = out["scales"][0, 0]
    best = min(oracle.proxy_loss(W, np.array([[(2 * c - 3) * s for c in cs]]), H)
               for cs in itertools.product(range(4), repeat=n))
    got = oracle.proxy_loss(W, oracle.dequant(out["codes"], out["scales"], 2, g), H)
    assert best <= got + 1e-15
    rtn = oracle.nearest_code(W / s, 3)
    assert got <= oracle.proxy_loss(W, oracle.dequant(rtn, out["scales"], 2, g), H) + 1e-12
