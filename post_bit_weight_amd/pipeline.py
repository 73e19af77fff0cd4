"""Sequence the library calls that quantize one linear layer (or several layers sharing H).

Order (Wringer model cards, "Recipe"; Wringer news article, second paragraph):
H accumulation and damping -> optional Hadamard rotation -> GPTQ codes and
scales -> joint scales against the weights -> wring against
W_hat + (alpha / r) B A (nearest-point codes, joint scales) -> packing.
Every step runs in libwringer.so; torch only allocates device memory and pads
the weights into the stored (rotated) dimension.
"""

import torch

from . import _lib as wr


def accumulate_hessian(ctx, chunks, n, S=None):
    """S (n x n fp64) = sum over chunks of X^T X; returns (S, total_rows)."""
    if S is None:
        S = torch.empty(n, n, dtype=torch.float64, device=ctx.device)
    total = 0
    first = True
    for X in chunks:
        wr.wr_hessian_accumulate(ctx, X, S, zero=first)
        first = False
        total += X.shape[0]
    if first:
        wr.wr_hessian_accumulate(ctx, torch.empty(0, n, dtype=torch.bfloat16, device=ctx.device), S, zero=True)
    return S, total


def finalize_hessian(ctx, S, total_rows, damp_frac, n_store, had_block=None, signs=None):
    H = torch.empty(n_store, n_store, dtype=torch.float32, device=ctx.device)
    delta = torch.empty(1, dtype=torch.float32, device=ctx.device)
    wr.wr_hessian_finalize(ctx, S, total_rows, damp_frac, H, delta, had_block or 0, signs)
    return H, delta


def prepare_weights(ctx, W, n_store, had_block=None, signs=None):
    """The weights in the stored basis: zero-padded to n_store and rotated when had_block is set."""
    rows, n0 = W.shape
    if not had_block and n_store == n0:
        return W
    Wp = torch.zeros(rows, n_store, dtype=torch.float32, device=ctx.device)
    Wp[:, :n0] = W
    if had_block:
        wr.wr_hadamard_rotate(ctx, Wp, had_block, signs, wr.WR_ROT_ROWS)
    return Wp


def quantize(ctx, Wst, H, bits, group, lam=0.01, B=None, A=None, alpha=None, lazy_batch=128, keep_stages=False):
    """GPTQ sweep, joint scales, wring.  bits: int or a per-row uint8 tensor.  Returns a dict of tensors."""
    rows, n = Wst.shape
    if isinstance(bits, int):
        bits_t = torch.full((rows,), bits, dtype=torch.uint8, device=ctx.device)
    else:
        bits_t = bits
    codes = torch.empty(rows, n, dtype=torch.uint8, device=ctx.device)
    scales = torch.empty(rows, n // group, dtype=torch.float16, device=ctx.device)
    info = torch.zeros(3, dtype=torch.int32, device=ctx.device)
    out = {}
    wr.wr_gptq_sweep(ctx, Wst, H, bits_t, group, lazy_batch, codes, scales, info[0:1])
    if keep_stages:
        out["gptq_codes"], out["gptq_scales"] = codes.clone(), scales.clone()
    wr.wr_wring_solve(ctx, H, bits_t, group, lam, codes, scales, info[1:2], target=Wst)
    if keep_stages:
        out["joint_scales"] = scales.clone()
    if B is not None:
        wr.wr_wring_solve(ctx, H, bits_t, group, lam, codes, scales, info[2:3], B=B, A=A,
                          alpha=alpha if alpha is not None else A.shape[0], recode=True)
    out.update(codes=codes, scales=scales, dev_info=info, bits=bits_t)
    return out


def pack(ctx, codes, scales, bits, group):
    rows, n = codes.shape
    buf = torch.empty(wr.packed_nbytes(rows, n, bits, group), dtype=torch.uint8, device=ctx.device)
    wr.wr_pack(ctx, codes, scales, bits, group, buf)
    return buf


def solve_module(ctx, W, chunks, bits, group, damp_frac=0.01, lam=0.01, B=None, A=None, alpha=None,
                 had_block=None, signs=None, n_store=None, lazy_batch=128, keep_stages=False):
    """The whole solve for one module W (rows x n0) with calibration chunks (each N_k x n0)."""
    rows, n0 = W.shape
    n = n_store or n0
    S, total = accumulate_hessian(ctx, chunks, n0)
    H, delta = finalize_hessian(ctx, S, total, damp_frac, n, had_block, signs)
    Wst = prepare_weights(ctx, W, n, had_block, signs)
    out = quantize(ctx, Wst, H, bits, group, lam, B, A, alpha, lazy_batch, keep_stages)
    if isinstance(bits, int):
        out["packed"] = pack(ctx, out["codes"], out["scales"], bits, group)
    out.update(H=H, delta=delta, S=S, W=Wst)
    return out
