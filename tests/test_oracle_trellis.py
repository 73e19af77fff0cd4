"""Pins for the oracle's trellis-coded quantizer (Pingala-8 post, "Trick 3: trellis coding")."""
import itertools

import numpy as np

import oracle


def _toy_values(g):
    return np.array([[[g["state0_values"][0]], [g["state0_values"][1]]],
                     [[g["state1_values"][0]], [g["state1_values"][1]]]])


def test_page_toy_best_path_and_greedy(golden):
    g = golden("trellis_toy_trick3.txt")
    vals = _toy_values(g)
    best = oracle.trellis_viterbi(g["targets"], vals, 0)
    assert np.allclose(best["recon"][0], g["best_picks"])
    assert np.array_equal(best["states"][0, :3], np.array(g["best_states"], dtype=int))
    assert round(float(best["cost"][0]), 2) == g["best_error"][0]
    gr = oracle.trellis_greedy(g["targets"], vals, 0)
    assert np.allclose(gr["recon"][0], g["greedy_picks"])
    assert np.array_equal(gr["states"][0, :3], np.array(g["greedy_states"], dtype=int))
    assert round(float(gr["cost"][0]), 2) == g["greedy_error"][0]
    # plain 1-bit rounding with the same 3 bits sits between the two
    t = np.array(g["targets"])
    plain = np.where(t >= 0, g["plain_values"][1], g["plain_values"][0])
    pe = float(np.sum((t - plain) ** 2))
    assert round(pe, 2) == g["plain_error"][0]
    assert best["cost"][0] < pe < gr["cost"][0]


def _brute(T, vals, start):
    """Every branch sequence from the start state; each step takes the nearest coset value."""
    S = vals.shape[0]
    best = np.inf
    for us in itertools.product((0, 1), repeat=len(T)):
        s, c = start, 0.0
        for t, u in zip(T, us):
            c += np.min((t - vals[s, u]) ** 2)
            s = ((s << 1) | u) % S
        best = min(best, c)
    return best


def test_viterbi_cost_is_the_brute_force_minimum():
    rng = np.random.default_rng(40)
    for S, C, n, start in [(2, 1, 9, 0), (4, 1, 8, 1), (4, 2, 7, 0), (8, 2, 9, 3), (8, 1, 10, 0)]:
        vals = np.sort(rng.uniform(-2, 2, size=(S, 2, C)), axis=2)
        for _ in range(4):
            T = rng.normal(0, 1.2, size=n)
            out = oracle.trellis_viterbi(T, vals, start)
            assert np.isclose(out["cost"][0], _brute(T, vals, start), rtol=1e-12, atol=1e-14)


def test_codes_decode_to_the_path_and_its_cost():
    rng = np.random.default_rng(41)
    vals = np.sort(rng.uniform(-2, 2, size=(8, 2, 2)), axis=2)
    T = rng.normal(0, 1.2, size=(5, 40))
    out = oracle.trellis_viterbi(T, vals, 0)
    rec = oracle.trellis_decode(out["codes"], vals, 0)
    assert np.array_equal(rec, out["recon"])
    assert np.allclose(np.sum((T - rec) ** 2, axis=1), out["cost"], rtol=1e-12)
    # the searched path is never worse than greedy rounding along the trellis
    assert np.all(out["cost"] <= oracle.trellis_greedy(T, vals, 0)["cost"] + 1e-12)


def test_targets_on_a_reachable_path_cost_zero():
    rng = np.random.default_rng(42)
    vals = np.sort(rng.uniform(-2, 2, size=(4, 2, 2)), axis=2)
    codes = rng.integers(0, 4, size=(3, 30))
    T = oracle.trellis_decode(codes, vals, 2)
    out = oracle.trellis_viterbi(T, vals, 2)
    assert np.allclose(out["cost"], 0.0, atol=1e-24)
    assert np.array_equal(oracle.trellis_decode(out["codes"], vals, 2), T)
