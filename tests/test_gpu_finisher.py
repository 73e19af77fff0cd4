"""GPU parity of the GPTQ-codes finisher (wr_wring_solve with WR_RECODE_GPTQ) against the oracle.

The v0.2 finisher of the Qwen3-4B card ("GPTQ codes + joint scales", section "Why the solver
changed") and the Agents-A1 card's finisher: the GPTQ sweep of the watered target
W' = dequant(codes, scales) + (alpha / r) B A with the damped H, then the joint scales against
W' with the prior at the sweep's scales.  Both sides use the same fp32 H, so codes may differ
only where the oracle's pre-rounding value sits within TIE of a decision threshold (the rest of
such a row is a different valid rounding), scales agree within one fp16 ulp on rows whose codes
agree, and the proxy losses within 1e-4.
"""
import ctypes as c

import numpy as np
import pytest
import torch

import oracle
from parity import TIE, code_parity, f16_bits, scale_ulps

pytestmark = pytest.mark.gpu



@pytest.fixture(scope="module")
def wr():
    from post_bit_weight_amd import _lib
    return _lib


@pytest.fixture(scope="module")
def ctx(wr):
    return wr.Context(0)


def _run(wr, ctx, H32, codes, scales, bits, g, lam, B, A, alpha):
    rows, n = codes.shape
    c_t = torch.from_numpy(codes.astype(np.uint8)).cuda()
    s_t = torch.from_numpy(scales.astype(np.float16)).cuda()
    info = torch.zeros(1, dtype=torch.int32, device="cuda")
    bits_t = torch.full((rows,), bits, dtype=torch.uint8, device="cuda")
    wr.wr_wring_solve(ctx, torch.from_numpy(H32).cuda(), bits_t, g, lam, c_t, s_t, info,
                      B=B.contiguous().cuda(), A=A.contiguous().cuda(), alpha=alpha, recode="gptq")
    return c_t.cpu().numpy().astype(np.int64), s_t.cpu().numpy().astype(np.float64), int(info.item())


def _compare(codes, scales, ref, H0, bits, g):
    L = 2 ** bits - 1
    cp = code_parity(codes, ref["codes"], ref["t"], L)
    assert cp["frac"] <= 1e-3 and cp["worst_first"] <= TIE, cp
    ok = cp["identical_rows"]
    assert scale_ulps(scales[ok], ref["scales"][ok]).max(initial=0) <= 1
    same = ok & (scale_ulps(scales, ref["scales"]).max(axis=1) == 0)
    lg = oracle.proxy_loss(ref["target"][same], oracle.dequant(codes, scales, bits, g)[same], H0)
    lr = oracle.proxy_loss(ref["target"][same], oracle.dequant(ref["codes"], ref["scales"], bits, g)[same], H0)
    assert abs(lg - lr) <= 1e-4 * lr
    return cp


def _first_solve(W, H, bits, g, lam):
    g0 = oracle.gptq_sweep(W, H, bits, g)
    s1, _ = oracle.joint_scales(g0["codes"], bits, g, H, W, g0["scales"], lam)
    return g0["codes"], s1


def test_gptq_finisher_toy(wr, ctx):
    """The toy layer: W 256 x 512 fp32, H from 4096 fp32 rows, group 32, rank-8 fp32 adapter."""
    from post_bit_weight_amd import synth
    W = synth.gaussian((256, 512), 0.02, seed=101)
    X = synth.SpectralSource(512, seed=102, n_outliers=5).chunk(0, 4096, dtype=torch.float32)
    B = synth.gaussian((256, 8), 0.01, seed=103)
    A = synth.gaussian((8, 512), 0.01, seed=104)
    H0 = oracle.second_moment(X.double().numpy())
    H32 = oracle.damp(H0, 0.01)[0].astype(np.float32)
    Hd = H32.astype(np.float64)
    codes0, s1 = _first_solve(W.double().numpy(), Hd, 2, 32, 0.01)
    codes, scales, info = _run(wr, ctx, H32, codes0, s1, 2, 32, 0.01, B, A, 8.0)
    assert info == 0
    ref = oracle.wring_gptq(codes0, s1, 2, 32, B.double().numpy(), A.double().numpy(), 8.0, Hd, 0.01)
    _compare(codes, scales, ref, H0, 2, 32)


def test_gptq_finisher_q_proj_slice(wr, ctx):
    """128 rows of the q_proj shape: n 2560, bf16 W and rank-128 bf16 adapter (alpha 128),
    group 64, H from 16384 spectral calibration rows."""
    from post_bit_weight_amd import synth
    rows, n, g, r = 128, 2560, 64, 128
    X = synth.SpectralSource(n, seed=20261210, outlier_frac=0.01).chunk(0, 16384, dtype=torch.bfloat16)
    W = synth.student_t((rows, n), seed=20261211, dtype=torch.bfloat16)
    B = synth.gaussian((rows, r), 0.01, seed=20261212, dtype=torch.bfloat16)
    A = synth.gaussian((r, n), 0.01, seed=20261213, dtype=torch.bfloat16)
    H0 = oracle.second_moment(X.double().numpy())
    H32 = oracle.damp(H0, 0.01)[0].astype(np.float32)
    Hd = H32.astype(np.float64)
    codes0, s1 = _first_solve(W.double().numpy(), Hd, 2, g, 0.01)
    codes, scales, info = _run(wr, ctx, H32, codes0, s1, 2, g, 0.01, B, A, float(r))
    assert info == 0
    ref = oracle.wring_gptq(codes0, s1, 2, g, B.double().numpy(), A.double().numpy(), float(r), Hd, 0.01)
    cp = _compare(codes, scales, ref, H0, 2, g)
    print(f"codes differing {cp['frac']:.2e}, rows with a tie {len(cp['rows'])}")


def test_gptq_finisher_grid_point_is_fixed(wr, ctx):
    """A grid point whose blocks each hold a level +-L, zero adapter: exact fixed point."""
    rng = np.random.default_rng(36)
    rows, n, g = 64, 512, 64
    Xr = rng.standard_normal((2048, n))
    H32 = (Xr.T @ Xr / 2048 + 0.05 * np.eye(n)).astype(np.float32)
    codes0 = rng.integers(0, 4, size=(rows, n))
    codes0[:, ::g] = rng.choice([0, 3], size=(rows, n // g))
    s0 = oracle.fp16_rne(rng.uniform(0.005, 0.02, size=(rows, n // g)))
    codes, scales, info = _run(wr, ctx, H32, codes0, s0, 2, g, 0.01, torch.zeros(rows, 16, dtype=torch.bfloat16),
                               torch.zeros(16, n, dtype=torch.bfloat16), 16.0)
    assert info == 0 and np.array_equal(codes, codes0) and np.array_equal(f16_bits(scales), f16_bits(s0))


def test_gptq_and_nearest_flags_exclude_each_other(wr, ctx):
    rows, n, g = 8, 128, 64
    H = torch.eye(n, dtype=torch.float32, device="cuda")
    codes = torch.zeros(rows, n, dtype=torch.uint8, device="cuda")
    scales = torch.ones(rows, n // g, dtype=torch.float16, device="cuda")
    bits = torch.full((rows,), 2, dtype=torch.uint8, device="cuda")
    info = torch.zeros(1, dtype=torch.int32, device="cuda")
    lib = wr.load()
    p = lambda t: c.c_void_p(t.data_ptr())
    rc = lib.wr_wring_solve(ctx.handle, None, wr.WR_F32, 0, None, None, 0, 0.0, wr.WR_F32, p(H), n, rows, n, p(bits),
                            g, 0.01, wr.WR_RECODE_NEAREST | wr.WR_RECODE_GPTQ, p(codes), p(scales), p(info))
    assert rc == wr.WR_EINVAL


@pytest.mark.parametrize("finisher", ["nearest", "gptq"])
def test_two_fill_and_wring_rounds(wr, ctx, finisher):
    """Two rounds (the Agents-A1 card ran two fill-and-wring rounds): the second wring starts from
    the first one's codes and scales with a second adapter.  pipeline.quantize chains them; each
    round is compared with the oracle started from the GPU's own input to that round."""
    from post_bit_weight_amd import pipeline, synth
    rows, n, g, r = 96, 1024, 64, 64
    X = synth.SpectralSource(n, seed=20261220, outlier_frac=0.01).chunk(0, 8192, dtype=torch.bfloat16)
    W = synth.student_t((rows, n), seed=20261221, dtype=torch.bfloat16)
    ad = [(synth.gaussian((rows, r), 0.01, seed=20261222 + 2 * k, dtype=torch.bfloat16),
           synth.gaussian((r, n), 0.01, seed=20261223 + 2 * k, dtype=torch.bfloat16)) for k in range(2)]
    H0 = oracle.second_moment(X.double().numpy())
    H32 = oracle.damp(H0, 0.01)[0].astype(np.float32)
    Hd = H32.astype(np.float64)
    out = pipeline.quantize(ctx, W.cuda(), torch.from_numpy(H32).cuda(), 2, g, 0.01,
                            adapters=[(B.cuda(), A.cuda()) for B, A in ad], keep_stages=True, finisher=finisher)
    torch.cuda.synchronize()
    assert (out["dev_info"].cpu().numpy() == 0).all()
    inputs = [(out["gptq_codes"], out["joint_scales"]), (out["round1_codes"], out["round1_scales"])]
    results = [(out["round1_codes"], out["round1_scales"]), (out["codes"], out["scales"])]
    fn = oracle.wring_gptq if finisher == "gptq" else oracle.wring
    for k in range(2):
        c_in = inputs[k][0].cpu().numpy().astype(np.int64)
        s_in = inputs[k][1].cpu().numpy().astype(np.float64)
        ref = fn(c_in, s_in, 2, g, ad[k][0].double().numpy(), ad[k][1].double().numpy(), float(r), Hd, 0.01)
        got_c = results[k][0].cpu().numpy().astype(np.int64)
        got_s = results[k][1].cpu().numpy().astype(np.float64)
        _compare(got_c, got_s, ref, H0, 2, g)


def test_gptq_finisher_q_proj_full_size_sampled_rows(wr, ctx):
    """The bench workload end to end on the GPU (H from 131072 calibration rows by the library,
    first solve, then the GPTQ-codes finisher on all 4096 rows); the oracle's finisher on 48
    sampled rows from the GPU's first-solve codes and scales with the same H (rows are
    independent given H)."""
    from post_bit_weight_amd import pipeline, synth
    rows, n, N, g, r = 4096, 2560, 131072, 64, 128
    src = synth.SpectralSource(n, seed=20261204, device="cuda", outlier_frac=0.01)
    X = torch.cat([src.chunk(k, 16384) for k in range(N // 16384)])
    W = synth.student_t((rows, n), seed=20261205, device="cuda", dtype=torch.bfloat16)
    B = synth.gaussian((rows, r), 0.01, seed=20261206, device="cuda", dtype=torch.bfloat16)
    A = synth.gaussian((r, n), 0.01, seed=20261207, device="cuda", dtype=torch.bfloat16)
    S, total = pipeline.accumulate_hessian(ctx, [X], n)
    H, _ = pipeline.finalize_hessian(ctx, S, total, 0.01, n)
    del X
    bits_t = torch.full((rows,), 2, dtype=torch.uint8, device="cuda")
    c1 = torch.empty(rows, n, dtype=torch.uint8, device="cuda")
    s1 = torch.empty(rows, n // g, dtype=torch.float16, device="cuda")
    info = torch.zeros(3, dtype=torch.int32, device="cuda")
    wr.wr_gptq_sweep(ctx, W, H, bits_t, g, 128, c1, s1, info[0:1])
    wr.wr_wring_solve(ctx, H, bits_t, g, 0.01, c1, s1, info[1:2], target=W)
    c2, s2 = c1.clone(), s1.clone()
    wr.wr_wring_solve(ctx, H, bits_t, g, 0.01, c2, s2, info[2:3], B=B, A=A, alpha=float(r), recode="gptq")
    torch.cuda.synchronize()
    assert (info.cpu().numpy() == 0).all()
    sel = np.sort(np.r_[0, rows - 1, np.random.default_rng(11).choice(np.arange(1, rows - 1), 46, replace=False)])
    t = torch.as_tensor(sel, device="cuda")
    Hd = H.cpu().double().numpy()
    ref = oracle.wring_gptq(c1[t].cpu().numpy().astype(np.int64), s1[t].cpu().numpy().astype(np.float64), 2, g,
                            B[t].double().cpu().numpy(), A.double().cpu().numpy(), float(r), Hd, 0.01)
    cp = _compare(c2[t].cpu().numpy().astype(np.int64), s2[t].cpu().numpy().astype(np.float64), ref, Hd, 2, g)
    print(f"codes differing {cp['frac']:.2e}, rows with a tie {len(cp['rows'])}")


def _search_check(codes, scales, ref, bits, g):
    """The searched finisher: each block's GPU scale gives an error within rounding of the oracle's
    least one (both evaluated in fp64 on the oracle's W'), the GPU's codes are the nearest levels
    at that scale except within 1e-4 level units of a threshold, and at least 99 % of scales equal
    the oracle's."""
    L = 2 ** bits - 1
    Wp = ref["target"]
    rows, n = Wp.shape
    nb = n // g
    s_rep = np.repeat(scales, g, axis=1)
    lev = 2 * codes - L
    err = ((Wp - s_rep * lev) ** 2).reshape(rows, nb, g).sum(axis=2)
    best = ref["errors"]
    assert np.all(err <= best * (1 + 1e-5) + 1e-18), np.max(err / np.maximum(best, 1e-30))
    t = np.divide(Wp, s_rep, out=np.zeros_like(Wp), where=s_rep > 0)
    near = oracle.nearest_code(t, L)
    bad = (near != codes) & (oracle.threshold_distance(t, L) > 1e-4)
    assert not bad.any(), int(bad.sum())
    same = np.mean(f16_bits(scales) == f16_bits(ref["scales"]))
    assert same >= 0.99, same
    return same


def _run_search(wr, ctx, codes, scales, bits, g, B, A, alpha):
    rows, n = codes.shape
    c_t = torch.from_numpy(codes.astype(np.uint8)).cuda()
    s_t = torch.from_numpy(scales.astype(np.float16)).cuda()
    info = torch.zeros(1, dtype=torch.int32, device="cuda")
    bits_t = torch.full((rows,), bits, dtype=torch.uint8, device="cuda")
    wr.wr_wring_solve(ctx, None, bits_t, g, 0.0, c_t, s_t, info, B=B.contiguous().cuda(), A=A.contiguous().cuda(),
                      alpha=alpha, recode="search")
    return c_t.cpu().numpy().astype(np.int64), s_t.cpu().numpy().astype(np.float64), int(info.item())


@pytest.mark.parametrize("shape", ["toy", "q_proj_slice"])
def test_scale_search_finisher(wr, ctx, shape):
    """The toy layer (fp32, group 32, rank 8) and a q_proj-shaped slice (bf16, group 64, rank 128),
    from the oracle's first-solve codes and scales."""
    from post_bit_weight_amd import synth
    if shape == "toy":
        rows, n, g, r, dt = 256, 512, 32, 8, torch.float32
        W = synth.gaussian((rows, n), 0.02, seed=101)
        X = synth.SpectralSource(n, seed=102, n_outliers=5).chunk(0, 4096, dtype=torch.float32)
    else:
        rows, n, g, r, dt = 128, 2560, 64, 128, torch.bfloat16
        W = synth.student_t((rows, n), seed=20261211, dtype=dt)
        X = synth.SpectralSource(n, seed=20261210, outlier_frac=0.01).chunk(0, 16384, dtype=dt)
    B = synth.gaussian((rows, r), 0.01, seed=103, dtype=dt)
    A = synth.gaussian((r, n), 0.01, seed=104, dtype=dt)
    Hd = oracle.damp(oracle.second_moment(X.double().numpy()), 0.01)[0].astype(np.float32).astype(np.float64)
    codes0, s1 = _first_solve(W.double().numpy(), Hd, 2, g, 0.01)
    codes, scales, info = _run_search(wr, ctx, codes0, s1, 2, g, B, A, float(r))
    assert info == 0
    ref = oracle.wring_scale_search(codes0, s1, 2, g, B.double().numpy(), A.double().numpy(), float(r))
    same = _search_check(codes, scales, ref, 2, g)
    print(f"scales equal to the oracle's: {same:.4f}")
