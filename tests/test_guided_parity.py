"""CPU checks of the guided parity comparison used by the full-size GPU tests.

A stand-in for the GPU result is the oracle itself run on a slightly perturbed H (the size of the
GPU's accumulation error); the guided comparison must accept it, and must reject a result with a
code changed away from any tie.
"""
import numpy as np
import pytest
import torch

import oracle
from parity import guided_check


def _problem(seed, rows=12, n=256, g=32):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((4 * n, n)) @ rng.standard_normal((n, n)) * 0.1
    X[:, :3] *= 20
    H0 = oracle.second_moment(X)
    H, _ = oracle.damp(H0, 0.01)
    W = 0.02 * rng.standard_normal((rows, n))
    B = 0.01 * rng.standard_normal((rows, 8))
    A = 0.01 * rng.standard_normal((8, n))
    E = rng.standard_normal((n, n)) * 2e-5       # entrywise relative error, 100x what the fp32 split sums give
    Hp = H * (1.0 + (E + E.T) / 2)
    return W, H, H0, Hp, B, A, g


def _as_gpu(res):
    keys = ("gptq_codes", "gptq_scales", "joint_scales", "codes", "scales")
    return {k: torch.from_numpy(np.asarray(res[k])) for k in keys}


def test_guided_check_accepts_a_perturbed_h_run():
    W, H, H0, Hp, B, A, g = _problem(1)
    other = oracle.solve_rows(W, Hp, 2, g, 0.01, B, A, 8.0)
    ref, st = guided_check(_as_gpu(other), W, H, H0, 2, g, 0.01, B, A, 8.0, 2e-2, max_forced_frac=1e-2,
                           max_scale_ulps=2)
    assert not st["unexplained"]
    assert st["codes_forced"] + st["scales_forced"] > 0     # the perturbation does move some decisions


def test_guided_check_rejects_a_code_away_from_ties():
    W, H, H0, Hp, B, A, g = _problem(2)
    other = oracle.solve_rows(W, H, 2, g, 0.01, B, A, 8.0)
    t = other["gptq_t"][3]
    k = int(np.argmax(oracle.threshold_distance(t, 3)))      # the column farthest from a threshold
    codes = other["gptq_codes"].copy()
    codes[3, k] = (codes[3, k] + 2) % 4
    other = dict(other, gptq_codes=codes)
    with pytest.raises(AssertionError):
        guided_check(_as_gpu(other), W, H, H0, 2, g, 0.01, B, A, 8.0, 2e-2)
