"""The measures of a module (grid distance, solver disagreement, one-ulp moves of the fp16
projection) computed by the library against the oracle's measures of the same arrays, and the
watered target and the unprojected scales the library exposes for them against the oracle."""
import numpy as np
import pytest
import torch

import oracle
from parity import f16_bits

pytestmark = pytest.mark.gpu


def _setup(rows=96, n=512, g=64, seed=601):
    from post_bit_weight_amd import _lib as wr
    from post_bit_weight_amd import pipeline, synth
    ctx = wr.Context(0)
    X = synth.SpectralSource(n, seed=seed, outlier_frac=0.01).chunk(0, 6000, dtype=torch.bfloat16)
    W = synth.student_t((rows, n), seed=seed + 1, dtype=torch.bfloat16).cuda()
    B = synth.gaussian((rows, 16), 0.01, seed=seed + 2, dtype=torch.bfloat16).cuda()
    A = synth.gaussian((16, n), 0.01, seed=seed + 3, dtype=torch.bfloat16).cuda()
    bits = torch.as_tensor(np.where(np.arange(rows) % 3 == 0, 3, 2).astype(np.uint8)).cuda()
    S, total = pipeline.accumulate_hessian(ctx, [X.cuda()], n)
    H, _ = pipeline.finalize_hessian(ctx, S, total, 0.01, n)
    codes = torch.empty(rows, n, dtype=torch.uint8, device="cuda")
    scales = torch.empty(rows, n // g, dtype=torch.float16, device="cuda")
    info = torch.zeros(2, dtype=torch.int32, device="cuda")
    wr.wr_gptq_sweep(ctx, W, H, bits, g, 128, codes, scales, info[0:1])
    wr.wr_wring_solve(ctx, H, bits, g, 0.01, codes, scales, info[1:2], target=W)
    torch.cuda.synchronize()
    assert (info.cpu().numpy() == 0).all()
    return wr, ctx, H, W, B, A, bits, codes, scales, g


def test_target_trace_and_stats_match_the_oracle():
    wr, ctx, H, W, B, A, bits, codes, scales, g = _setup()
    rows, n = W.shape
    b = bits.cpu().numpy().astype(np.int64)
    c1 = codes.cpu().numpy().astype(np.int64)
    s1 = scales.cpu().numpy().astype(np.float64)
    Bh, Ah = B.double().cpu().numpy(), A.double().cpu().numpy()
    info = torch.zeros(1, dtype=torch.int32, device="cuda")
    # the watered target
    Tf = torch.empty(rows, n, dtype=torch.float32, device="cuda")
    wr.wr_wring_target(ctx, bits, g, Tf, info, codes=codes, scales=scales, B=B, A=A, alpha=16.0)
    Tref = oracle.wring_target(c1, s1, b, g, Bh, Ah, 16.0)
    T = Tf.double().cpu().numpy()
    assert int(info.item()) == 0
    assert np.abs(T - Tref).max() <= 2 ** -22 * np.abs(Tref).max()
    # the wring with its unprojected scales traced, against the oracle's unrounded joint scales
    raw = torch.empty(rows, n // g, dtype=torch.float32, device="cuda")
    cn, sn = codes.clone(), scales.clone()
    wr.wr_set_scale_trace(ctx, raw)
    wr.wr_wring_solve(ctx, H, bits, g, 0.01, cn, sn, info, B=B, A=A, alpha=16.0, recode=True)
    wr.wr_set_scale_trace(ctx, None)
    torch.cuda.synchronize()
    Hg = H.cpu().double().numpy()
    ref = oracle.wring(c1, s1, b, g, Bh, Ah, 16.0, Hg, 0.01)
    cn_h, sn_h, raw_h = cn.cpu().numpy().astype(np.int64), sn.cpu().numpy().astype(np.float64), raw.cpu().numpy()
    same = (cn_h == ref["codes"]).all(axis=1)
    assert same.mean() >= 0.95
    rel = np.abs(raw_h[same] - ref["scales_unrounded"][same]) / np.abs(ref["scales_unrounded"][same])
    assert rel.max() <= 1e-5, rel.max()
    assert np.abs(f16_bits(raw_h.astype(np.float64)) - f16_bits(sn_h)).max() <= 1   # the projection of the trace
    # a trace smaller than the call is refused before any launch
    small = torch.empty(8, dtype=torch.float32, device="cuda")
    wr.wr_set_scale_trace(ctx, small)
    with pytest.raises(wr.WringerError):
        wr.wr_wring_solve(ctx, H, bits, g, 0.01, cn.clone(), sn.clone(), info, B=B, A=A, alpha=16.0, recode=True)
    wr.wr_set_scale_trace(ctx, None)
    # the sums, against the oracle's measures of the same arrays
    out = torch.zeros(4, dtype=torch.float64, device="cuda")
    wr.wr_quant_stats(ctx, cn, sn, bits, g, out, T=Tf, codes_ref=codes, scales_raw=raw)
    o = out.cpu().numpy()
    dist = oracle.grid_distance(T, cn_h, sn_h, b, g)
    assert abs(np.sqrt(o[0] / o[1]) - dist) <= 1e-12 * dist
    assert abs(o[1] - np.sum(T * T)) <= 1e-12 * o[1]
    assert o[2] == np.sum(cn_h != c1) == round(oracle.code_disagreement(cn_h, c1) * rows * n)
    moves = oracle.projection_ulp_moves(cn_h, sn_h, raw_h.astype(np.float64), b, g)
    assert o[3] == round(moves * rows * n)
    print(f"grid distance {dist:.4f}, codes recoded {o[2] / (rows * n):.4f}, projection moves {moves:.4f}")


def test_module_measures_match_the_oracle():
    """The module's measures (parent and filled grid distance, solver disagreement with and without
    the adapter, projection moves) against the oracle's measures of the library's own arrays,
    and the parent distance against the oracle's grid representation on the same H."""
    from post_bit_weight_amd import measures
    wr, ctx, H, W, B, A, bits, codes, scales, g = _setup(rows=64, n=384, seed=611)
    m = measures.module_measures(ctx, H, W, bits, g, 0.01, codes, scales, B, A, 16.0)
    torch.cuda.synchronize()
    for k, v in m.items():
        assert np.isfinite(v) and v >= 0.0, (k, v)
    b = bits.cpu().numpy().astype(np.int64)
    Wh = W.double().cpu().numpy()
    Hg = H.cpu().double().numpy()
    s1 = scales.cpu().numpy().astype(np.float64)
    cp, sp, _ = oracle.grid_representation(Wh, s1, b, g, Hg, 0.01)
    ref_parent = oracle.grid_distance(Wh, cp, sp, b, g)
    assert abs(m["grid_distance_parent"] - ref_parent) <= 1e-3 * ref_parent
    assert m["grid_distance_filled"] < m["grid_distance_parent"]
    assert 0.0 < m["solver_disagreement_zero_adapter"] < 0.5
    print({k: round(v, 5) for k, v in m.items()}, f"oracle parent distance {ref_parent:.5f}")
