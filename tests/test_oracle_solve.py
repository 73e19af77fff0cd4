"""End-to-end oracle checks on a tiny layer, and the threshold-distance helper."""
import numpy as np

import oracle


def test_threshold_distance_hand_cases():
    t = np.array([0.1, 1.9, -2.3, 2.0, -0.05, 5.0])
    d = oracle.threshold_distance(t, 3)
    assert np.allclose(d, [0.1, 0.1, 0.3, 0.0, 0.05, 3.0])


def test_solve_module_pipeline_small():
    rng = np.random.default_rng(50)
    rows, n0, N, g, m = 16, 48, 400, 16, 16
    W = 0.02 * rng.standard_normal((rows, n0))
    X = rng.standard_normal((N, n0)) @ rng.standard_normal((n0, n0)) * 0.3
    signs = rng.choice([-1.0, 1.0], size=64)
    B = 0.01 * rng.standard_normal((rows, 4))
    A = 0.01 * rng.standard_normal((4, 64))
    out = oracle.solve_module(W, X, 2, g, 0.01, 0.01, B, A, 4.0, had_block=m, signs=signs, n_store=64)
    # rotation of the padded second moment equals the second moment of the rotated padded inputs
    Xp = np.zeros((N, 64))
    Xp[:, :n0] = X
    assert np.allclose(out["H0"], oracle.second_moment(oracle.rotate_rows(Xp, m, signs)), atol=1e-12)
    assert np.allclose(out["H"] - out["H0"], out["delta"] * np.eye(64), atol=1e-15)
    # joint scales fit W at least as well as the sweep's own scales (up to the fp16 projection)
    H = out["H"]
    e_gptq = oracle.proxy_loss(out["W"], oracle.dequant(out["gptq_codes"], out["gptq_scales"], 2, g), H)
    e_joint = oracle.proxy_loss(out["W"], oracle.dequant(out["gptq_codes"], out["joint_scales"], 2, g), H)
    assert e_joint <= e_gptq * 1.001
    c, s = oracle.unpack(out["packed"], rows, 64, 2, g)
    assert np.array_equal(c, out["codes"]) and np.array_equal(s, out["scales"])
    assert out["packed"].shape[0] == rows * 64 * 2 // 8 + 2 * rows * 4
