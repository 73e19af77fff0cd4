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


def test_gptq_finisher_with_identity_h_is_absmax_rounding_then_block_ridge():
    """H = I: no error feedback, so the sweep rounds each weight to the nearest level on the
    block's absmax fp16 scale; the joint solve separates into one ridge problem per block,
    s_b = (q_b . t_b + lam mu s0_b) / (q_b . q_b + lam mu), mu = sum_b q_b . q_b / nb."""
    rng = np.random.default_rng(34)
    rows, n, g, bits, lam = 5, 24, 8, 2, 0.01
    L = 2 ** bits - 1
    codes0 = rng.integers(0, L + 1, size=(rows, n))
    s_in = oracle.fp16_rne(rng.uniform(0.1, 0.5, size=(rows, n // g)))
    B = 0.3 * rng.standard_normal((rows, 3))
    A = 0.3 * rng.standard_normal((3, n))
    out = oracle.wring_gptq(codes0, s_in, bits, g, B, A, 3.0, np.eye(n), lam)
    Wp = out["target"]
    for i in range(rows):
        q = np.zeros(n)
        s0 = np.zeros(n // g)
        for b in range(n // g):
            s0[b] = float(np.float16(max(abs(Wp[i, j]) for j in range(b * g, b * g + g)) / L))
            for j in range(b * g, b * g + g):
                c = min(max(int(np.floor((Wp[i, j] / s0[b] + L) / 2 + 0.5)), 0), L)
                assert out["codes"][i, j] == c
                q[j] = 2 * c - L
        assert np.array_equal(out["sweep_scales"][i], s0)
        qq = [sum(q[j] ** 2 for j in range(b * g, b * g + g)) for b in range(n // g)]
        qt = [sum(q[j] * Wp[i, j] for j in range(b * g, b * g + g)) for b in range(n // g)]
        mu = sum(qq) / (n // g)
        for b in range(n // g):
            ridge = (qt[b] + lam * mu * s0[b]) / (qq[b] + lam * mu)
            assert np.isclose(out["scales_unrounded"][i, b], ridge, rtol=1e-12)
            assert out["scales"][i, b] == float(np.float16(ridge))


def test_gptq_finisher_keeps_a_grid_point_with_extreme_levels():
    """W' = Q s0 exactly and every block holds a level +-L: the sweep makes no error (so no
    feedback) and reproduces the absmax scales s0; the joint residual vanishes at s0, where
    the prior is centred, so codes and scales come back unchanged for any SPD H."""
    rng = np.random.default_rng(35)
    for bits in (2, 3):
        H, codes, scales, L = _setup(rng, rows=6, n=32, g=8, bits=bits)
        codes[:, ::8] = rng.choice([0, L], size=(6, 4))
        out = oracle.wring_gptq(codes, scales, bits, 8, np.zeros((6, 2)), np.zeros((2, 32)), 2.0, H, 0.01)
        assert np.array_equal(out["codes"], codes)
        assert np.array_equal(out["sweep_scales"], scales)
        assert np.array_equal(out["scales"], scales)


def test_scale_search_is_the_best_candidate_by_enumeration():
    """Each block's result is the candidate with the least squared error over all 32 candidate
    scales and, for that scale, over every code vector (brute force on 4-weight blocks: the
    nearest level per weight is the error-minimising code for a fixed scale)."""
    import itertools
    rng = np.random.default_rng(37)
    for bits in (2, 3):
        L = 2 ** bits - 1
        for _ in range(6):
            w = rng.normal(0, 1, size=4)
            s, c, e, k = oracle.scale_search_block(w, L)
            amax = np.max(np.abs(w))
            best = np.inf
            for kk in range(32):
                sk = float(np.float16((1 - kk / 64) * amax / L))
                for cc in itertools.product(range(L + 1), repeat=4):
                    best = min(best, float(np.sum((w - sk * (2 * np.array(cc) - L)) ** 2)))
            assert np.isclose(e, best, rtol=1e-12, atol=1e-15)
            assert np.isclose(np.sum((w - s * (2 * c - L)) ** 2), e, rtol=1e-12)


def test_scale_search_keeps_the_absmax_scale_when_it_is_exact():
    """A block already on the grid at its absmax scale (a level +-L present) has zero error at
    k = 0, the first candidate, which a tie keeps."""
    rng = np.random.default_rng(38)
    H, codes, scales, L = _setup(rng, rows=3, n=24, g=8)
    codes[:, ::8] = L
    out = oracle.wring_scale_search(codes, scales, 2, 8, np.zeros((3, 2)), np.zeros((2, 24)), 2.0)
    assert np.array_equal(out["codes"], codes) and np.array_equal(out["scales"], scales)
    assert np.all(out["k"] == 0) and np.all(out["errors"] == 0)
