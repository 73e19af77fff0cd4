"""The whole per-module solve in the pages' order (oracle, test infrastructure only).

H accumulation and damping -> optional rotation -> GPTQ codes and scales ->
joint scales against the weights -> wring against W' = W_hat + (alpha/r) B A
(nearest-point codes, joint scales) -> pack.  Sources: Wringer news article
(second paragraph) and the model cards' "Recipe" sections for the order; the
Pingala-8 post's "Trick 1" for the rotation.
"""

import numpy as np

from .hessian import second_moment, pad_square, damp
from .rotation import rotate_rows, rotate_sym
from .gptq import gptq_sweep
from .joint import joint_scales
from .wring import wring
from .pack import pack


def solve_rows(W, H, bits, group, lam, B=None, A=None, alpha=None):
    """GPTQ codes and scales -> joint scales against W -> wring against W_hat + (alpha/r) B A, for
    the rows of W (stored basis) given the damped H.  Rows are independent given H, so any subset of
    a layer's rows gives the same result as the whole layer restricted to that subset."""
    g = gptq_sweep(W, H, bits, group)
    s1, _ = joint_scales(g["codes"], bits, group, H, W, g["scales"], lam)
    w = wring(g["codes"], s1, bits, group, B, A, alpha, H, lam)
    return {
        "gptq_codes": g["codes"], "gptq_scales": g["scales"], "gptq_t": g["t"],
        "joint_scales": s1,
        "codes": w["codes"], "scales": w["scales"], "target": w["target"], "wring_t": w["t"],
    }


def solve_module(W, X, bits, group, damp_frac, lam, B=None, A=None, alpha=None,
                 had_block=None, signs=None, n_store=None):
    """Run the solve for one linear layer W (rows x n0) with calibration rows X (N x n0).

    With a rotation, W and X live in the zero-padded stored dimension n_store
    (a multiple of had_block) and B, A are given in the rotated basis.
    """
    W = np.asarray(W, dtype=np.float64)
    rows, n0 = W.shape
    n = n0 if n_store is None else int(n_store)
    H0 = pad_square(second_moment(X), n)
    Wn = np.zeros((rows, n))
    Wn[:, :n0] = W
    if had_block:
        H0 = rotate_sym(H0, had_block, signs)
        Wn = rotate_rows(Wn, had_block, signs)
    H, delta = damp(H0, damp_frac)
    out = {"H0": H0, "H": H, "delta": delta, "W": Wn}
    out.update(solve_rows(Wn, H, bits, group, lam, B, A, alpha))
    if np.ndim(bits) == 0:
        out["packed"] = pack(out["codes"], out["scales"], int(bits), group)
    return out
