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


def _tiny_wring_case(seed=44):
    """n = 8, group 4, 2 bits: a seeded row quantized as the pipeline does (GPTQ sweep, joint scales
    against W), then a rank-2 adapter of std 0.08 (relative to the weights about the size of the
    workloads' rank-128 adapters); returns what the wring starts from."""
    rng = np.random.default_rng(seed)
    n, g, bits = 8, 4, 2
    Xc = rng.standard_normal((64, n))
    Xc[:, 3] *= 4.0                                   # one strong channel, as in the calibration model
    H, _ = oracle.damp(Xc.T @ Xc / 64, 0.01)
    w = 0.02 * rng.standard_t(5, size=(1, n))
    g0 = oracle.gptq_sweep(w, H, bits, g)
    s1, _ = oracle.joint_scales(g0["codes"], bits, g, H, w, g0["scales"], 0.01)
    B = 0.08 * rng.standard_normal((1, 2))
    A = 0.08 * rng.standard_normal((2, n))
    return H, g0["codes"], s1, B, A, n, g, bits


def _f16_step(x, k):
    """The fp16 value k representable steps away from the fp16 value x (x > 0)."""
    bits = np.float16(x).view(np.int16).astype(np.int32) + k
    return float(np.int16(bits).view(np.float16))


def _objective_lstsq_stack(H, lev, g, t, s0, lam):
    """min over s of (t - Q s)^T H (t - Q s) + lam mu ||s - s0||^2 via least squares on the stacked
    system [C Q; sqrt(lam mu) I] s ~ [C t; sqrt(lam mu) s0] with H = C^T C, solved by QR; for a
    batch of level vectors lev (K x n).  Returns (objective values, minimisers)."""
    K, n = lev.shape
    nb = n // g
    C = np.linalg.cholesky(H).T
    Q = np.zeros((K, n, nb))
    for b in range(nb):
        Q[:, b * g:(b + 1) * g, b] = lev[:, b * g:(b + 1) * g]
    CQ = np.einsum("ij,kjb->kib", C, Q)
    mu = np.einsum("kib,kib->k", CQ, CQ) / nb            # trace(Q^T H Q) / nb
    M = np.concatenate([CQ, np.sqrt(lam * mu)[:, None, None] * np.eye(nb)[None]], axis=1)
    rhs = np.concatenate([np.broadcast_to(C @ t, (K, n)), np.sqrt(lam * mu)[:, None] * s0[None, :]], axis=1)
    Qm, Rm = np.linalg.qr(M)
    s = np.linalg.solve(Rm, np.einsum("kib,ki->kb", Qm, rhs)[..., None])[..., 0]
    d = t[None, :] - np.einsum("kjb,kb->kj", Q, s)
    f = np.einsum("kj,jl,kl->k", d, H, d) + lam * mu * np.sum((s - s0[None, :]) ** 2, axis=1)
    return f, s


def test_projected_scales_are_the_best_fp16_neighbours_on_a_tiny_block():
    """Brute force over fp16 scales: on the seeded n = 8, g = 4, 2-bit wring, every combination
    of +-3 fp16 steps around the fp16-rounded joint scales is evaluated on the objective
    (t - Q s)^T H (t - Q s) + lam mu ||s - s0||^2; the rounded solution attains the least
    value among those 49 points.  (An observation on this case, not a theorem: with coupled
    blocks the best fp16 point need not be the rounding of the real optimum.)  A dropped prior,
    a wrong sign on it or a transposed Q would move the solution by many fp16 steps."""
    H, c0, s0, B, A, n, g, bits = _tiny_wring_case()
    out = oracle.wring(c0, s0, bits, g, B, A, 2.0, H, 0.01)
    t = out["target"][0]
    lev = oracle.level_of(out["codes"][0], 3).astype(float)
    Q = _dense_Q(lev, g)
    best, arg = np.inf, None
    for i in range(-3, 4):
        for j in range(-3, 4):
            s = np.array([_f16_step(out["scales"][0, 0], i), _f16_step(out["scales"][0, 1], j)])
            v = _objective(s, Q, H, t, s0[0], 0.01)
            if v < best:
                best, arg = v, (i, j)
    assert arg == (0, 0)


def test_wring_is_a_zero_gradient_but_not_global_optimum_by_enumeration():
    """All 4^8 code vectors of the tiny block, each with its own least-squares scales (QR of the
    stacked system, not the oracle's closed form): the wring's codes are one of them, their
    objective value equals the enumerated one, the oracle's unrounded scales are that code
    vector's minimiser (zero gradient), and some other code vector does strictly better -- the
    wring's nearest-point codes are a valid local choice, not the global optimum."""
    import itertools
    H, c0, s0, B, A, n, g, bits = _tiny_wring_case()
    out = oracle.wring(c0, s0, bits, g, B, A, 2.0, H, 0.01)
    assert (out["codes"] != c0).any()                 # the recode moved some codes
    t = out["target"][0]
    allc = np.array(list(itertools.product(range(4), repeat=n)))
    f, s = _objective_lstsq_stack(H, 2 * allc - 3, g, t, s0[0], 0.01)
    idx = int(np.flatnonzero((allc == out["codes"][0]).all(axis=1))[0])
    assert np.allclose(s[idx], out["scales_unrounded"][0], rtol=1e-10)
    lev = oracle.level_of(out["codes"][0], 3).astype(float)
    assert np.isclose(_objective(out["scales_unrounded"][0], _dense_Q(lev, g), H, t, s0[0], 0.01), f[idx], rtol=1e-10)
    assert f[idx] >= f.min()
    assert f.min() < f[idx] * (1 - 1e-6)
    # every code vector's least-squares scales have zero gradient: spot-check the oracle's closed form
    pick = np.random.default_rng(3).choice(len(allc), 64, replace=False)
    _, s_or = oracle.joint_scales(allc[pick], bits, g, H, np.broadcast_to(t, (64, n)),
                                  np.broadcast_to(s0[0], (64, 2)), 0.01)
    assert np.allclose(s_or, s[pick], rtol=1e-9, atol=1e-14)
