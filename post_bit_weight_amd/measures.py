"""The measures the model cards report on their solves, computed by the library for one module.

* grid distance (Wringer Qwen3-4B card, "Why the solver changed": 0.46 for the parent weights,
  0.07 for the filled ones): ||T - T_grid||_F / ||T||_F with T_grid the nearest-point codes of T on
  the current fp16 scales and joint scales against T -- for the parent, T = the weights with the
  first solve's scales; for the filled weights, T = W' = dequant + (alpha / r) B A, whose grid
  representation is the wring's result;
* solver disagreement (same section: 18 % at zero training, 1.7 % after the fill): the share of
  codes on which the GPTQ finisher and the nearest-point finisher differ, with a zero adapter
  ("zero training") and with the module's adapter;
* projection moves (Agents-A1 card, "Honest caveats": 2.95 %): the share of stored-basis weights
  (2c - L) s whose bf16 rounding changes when the fp16 scales of the wring replace the unprojected
  solution of its scale solve.

All arithmetic runs in libwringer.so (wr_wring_solve, wr_wring_target, wr_set_scale_trace,
wr_quant_stats); this module allocates device memory, sequences the calls and divides the
resulting sums.  The module's own codes and scales are not touched (copies are solved).
"""

import torch

from . import _lib as wr


def module_measures(ctx, H, W, bits, group, lam, codes1, scales1, B, A, alpha):
    """H: damped H (n x n fp32); W: the module's weights in the stored basis (rows x n); bits: per-row
    uint8; codes1/scales1: the first solve's codes and scales (GPTQ + joint scales against W)."""
    rows, n = W.shape
    dev = W.device
    nb = n // group
    info = torch.zeros(1, dtype=torch.int32, device=dev)
    out = torch.zeros(4, dtype=torch.float64, device=dev)
    res = {}

    def copy():
        return codes1.clone(), scales1.clone()

    def stats(T, codes, scales, codes_ref=None, raw=None):
        wr.wr_quant_stats(ctx, codes, scales, bits, group, out, T=T, codes_ref=codes_ref, scales_raw=raw)
        return out.cpu().tolist()

    def check():
        if int(info.item()) != 0:
            raise RuntimeError(f"dev_info {int(info.item())} in the measures")

    Wf = W if W.dtype == torch.float32 else W.float()
    # parent: nearest-point codes of W on the first solve's scales, joint scales against W
    c, s = copy()
    wr.wr_wring_solve(ctx, H, bits, group, lam, c, s, info, target=Wf, recode=True)
    check()
    d2, t2, _, _ = stats(Wf, c, s)
    res["grid_distance_parent"] = (d2 / t2) ** 0.5
    # zero training: GPTQ finisher against the nearest-point finisher with no adapter (the latter
    # returns the first solve's codes: a fixed point)
    c, s = copy()
    wr.wr_wring_solve(ctx, H, bits, group, lam, c, s, info, recode="gptq")
    check()
    _, _, diff, _ = stats(None, c, s, codes_ref=codes1)
    res["solver_disagreement_zero_adapter"] = diff / (rows * n)
    # filled: W' and its grid representation (the wring, with the unprojected scales traced)
    Tf = torch.empty(rows, n, dtype=torch.float32, device=dev)
    wr.wr_wring_target(ctx, bits, group, Tf, info, codes=codes1, scales=scales1, B=B, A=A, alpha=alpha)
    check()
    raw = torch.empty(rows, nb, dtype=torch.float32, device=dev)
    cn, sn = copy()
    wr.wr_set_scale_trace(ctx, raw)
    try:
        wr.wr_wring_solve(ctx, H, bits, group, lam, cn, sn, info, B=B, A=A, alpha=alpha, recode=True)
    finally:
        wr.wr_set_scale_trace(ctx, None)
    check()
    cg, sg = copy()
    wr.wr_wring_solve(ctx, H, bits, group, lam, cg, sg, info, B=B, A=A, alpha=alpha, recode="gptq")
    check()
    d2, t2, diff, moved = stats(Tf, cn, sn, codes_ref=cg, raw=raw)
    res["grid_distance_filled"] = (d2 / t2) ** 0.5
    res["solver_disagreement_filled"] = diff / (rows * n)
    res["projection_ulp_moves"] = moved / (rows * n)
    return res
