"""GPU parity of wr_trellis_quantize (Pingala-8 post, "Trick 3: trellis coding") against the oracle.

Several paths can be optimal up to rounding (the GPU searches in fp32, the oracle in fp64), so
the tests compare what is unique and check the rest is valid: the GPU's codes must decode to
its reconstruction, its reported cost must be that path's fp64 sum of squared errors, and that
cost must equal the oracle's optimum within 1e-6 relative (the GPU cannot beat it).
"""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def wr():
    from post_bit_weight_amd import _lib
    return _lib


@pytest.fixture(scope="module")
def ctx(wr):
    return wr.Context(0)


def _run(wr, ctx, T, log2s, vals, start=0):
    rows, n = T.shape
    ld = (n + 3) // 4 * 4
    Tp = torch.zeros(rows, ld, dtype=torch.float32, device="cuda")
    Tp[:, :n] = torch.as_tensor(T, dtype=torch.float32)
    Td = Tp[:, :n]
    v = torch.as_tensor(vals, dtype=torch.float32).contiguous().cuda()
    codes = torch.empty(rows, n, dtype=torch.uint8, device="cuda")
    recon = torch.empty(rows, n, dtype=torch.float32, device="cuda")
    cost = torch.empty(rows, dtype=torch.float64, device="cuda")
    wr.wr_trellis_quantize(ctx, Td, log2s, v, codes, recon, cost, start_state=start)
    torch.cuda.synchronize()
    return codes.cpu().numpy().astype(np.int64), recon.cpu().numpy(), cost.cpu().numpy()


def _check(T32, vals32, start, codes, recon, cost, ref):
    T = T32.astype(np.float64)
    vals = vals32.astype(np.float64)
    dec = oracle.trellis_decode(codes, vals, start)
    assert np.array_equal(dec, recon.astype(np.float64))
    path = np.sum((T - dec) ** 2, axis=1)
    assert np.allclose(cost, path, rtol=1e-12, atol=0)
    opt = ref["cost"]
    assert np.all(cost >= opt * (1 - 1e-12)) and np.all(cost <= opt * (1 + 1e-6)), np.max(cost / opt - 1)
    return float(np.mean(codes == ref["codes"]))


def test_page_toy(wr, ctx, golden):
    g = golden("trellis_toy_trick3.txt")
    vals = np.array([[[g["state0_values"][0]], [g["state0_values"][1]]],
                     [[g["state1_values"][0]], [g["state1_values"][1]]]], dtype=np.float32)
    T = np.array([g["targets"]], dtype=np.float32)
    codes, recon, cost = _run(wr, ctx, T, 1, vals)
    assert np.allclose(recon[0], g["best_picks"])
    assert round(float(cost[0]), 2) == g["best_error"][0]
    assert codes[0].tolist() == [0, 1, 1]  # branch bits; the bit written is the next state


@pytest.mark.parametrize("log2s,C,rows,n,start", [(1, 1, 37, 1000, 0), (2, 2, 37, 2560, 1), (3, 2, 37, 2560, 0),
                                                   (3, 4, 20, 777, 5), (4, 2, 33, 1024, 9), (4, 1, 9, 65, 0),
                                                   (2, 4, 70, 31, 3), (3, 2, 10, 96, 2), (3, 2, 11, 161, 0),
                                                   (2, 2, 5, 1, 0)])
def test_random_trellises_match_the_oracle(wr, ctx, log2s, C, rows, n, start):
    rng = np.random.default_rng(log2s * 100 + C * 10 + rows)
    S = 1 << log2s
    vals = np.sort(rng.uniform(-3, 3, size=(S, 2, C)), axis=2).astype(np.float32)
    T = rng.normal(0, 1.5, size=(rows, n)).astype(np.float32)
    codes, recon, cost = _run(wr, ctx, T, log2s, vals, start)
    ref = oracle.trellis_viterbi(T.astype(np.float64), vals.astype(np.float64), start)
    same = _check(T, vals, start, codes, recon, cost, ref)
    assert same >= 0.99, same


@pytest.mark.parametrize("log2s,C,n", [(3, 2, 96), (3, 2, 101), (3, 2, 31), (3, 2, 1), (3, 2, 2), (3, 2, 33),
                                         (3, 2, 2559), (4, 2, 161), (4, 4, 64), (3, 1, 70)])
def test_coset_by_low_bit_trellis_matches_the_oracle(wr, ctx, log2s, C, n):
    """Tables whose coset depends only on the predecessor's low bit and the branch bit, like the
    workload trellis: every branch into a state carries one coset, so the forward kernel computes
    each metric once.  Lengths with an odd number of whole 32-step chunks, a ragged chunk, fewer
    than 32 steps and a single step."""
    rng = np.random.default_rng(log2s * 1000 + C * 100 + n)
    S = 1 << log2s
    base = np.sort(rng.uniform(-3, 3, size=(2, 2, C)), axis=2)
    vals = np.stack([base[p & 1] for p in range(S)]).astype(np.float32)
    T = rng.normal(0, 1.5, size=(13, n)).astype(np.float32)
    codes, recon, cost = _run(wr, ctx, T, log2s, vals, 0)
    ref = oracle.trellis_viterbi(T.astype(np.float64), vals.astype(np.float64), 0)
    _check(T, vals, 0, codes, recon, cost, ref)


def test_workload_trellis_full_size_sampled_rows(wr, ctx):
    """The bench workload: 25600 x 2560 targets (Student-t, std 1.5 level units), the 8-state
    2-bit trellis; the oracle on 24 sampled rows (rows are independent)."""
    from post_bit_weight_amd import synth
    rows, n = 25600, 2560
    T = synth.student_t((rows, n), seed=20261230, std=1.5, device="cuda")
    vals = synth.trellis8_values()
    codes = torch.empty(rows, n, dtype=torch.uint8, device="cuda")
    recon = torch.empty(rows, n, dtype=torch.float32, device="cuda")
    cost = torch.empty(rows, dtype=torch.float64, device="cuda")
    wr.wr_trellis_quantize(ctx, T, 3, vals.cuda(), codes, recon, cost)
    torch.cuda.synchronize()
    sel = np.sort(np.r_[0, rows - 1, np.random.default_rng(3).choice(np.arange(1, rows - 1), 22, replace=False)])
    t = torch.as_tensor(sel, device="cuda")
    Ts = T[t].cpu().numpy()
    ref = oracle.trellis_viterbi(Ts.astype(np.float64), vals.numpy().astype(np.float64), 0)
    same = _check(Ts, vals.numpy(), 0, codes[t].cpu().numpy().astype(np.int64), recon[t].cpu().numpy(),
                  cost[t].cpu().numpy(), ref)
    assert same >= 0.99, same
    # the post's point, on average over long sequences: the searched 2-bit path fits better than
    # plain 2-bit rounding to the four odd levels -3, -1, 1, 3
    plain2 = np.sum((Ts - np.clip(2 * np.floor(Ts / 2) + 1, -3, 3)) ** 2, axis=1)
    assert np.mean(cost[t].cpu().numpy()) < np.mean(plain2)


def test_bad_arguments(wr, ctx):
    T = torch.zeros(4, 6, dtype=torch.float32, device="cuda")
    v = torch.zeros(2, 2, 1, dtype=torch.float32, device="cuda")
    codes = torch.empty(4, 6, dtype=torch.uint8, device="cuda")
    with pytest.raises(RuntimeError):  # ld 6 is not a multiple of 4
        wr.wr_trellis_quantize(ctx, T, 1, v, codes)
    T8 = torch.zeros(4, 8, dtype=torch.float32, device="cuda")
    c8 = torch.empty(4, 8, dtype=torch.uint8, device="cuda")
    with pytest.raises(RuntimeError):  # start state outside 0 .. S-1
        wr.wr_trellis_quantize(ctx, T8, 1, v, c8, start_state=2)
