"""The wring: re-solve codes and scales against the adapter-watered target (oracle, test infrastructure only).

Wringer news article (second paragraph): the wring takes ``Wq + BA/r`` as the
new target and re-solves the integer codes and scales, after which the adapter
is dropped.  Qwen3-4B model card, "Recipe" (v0.3): nearest-point rounding of
the watered weights onto the same grid, then the same joint closed-form scale
solve with the watered weights as target.

Readings: the adapter term is (alpha / r) B A (the usual LoRA scaling; with
alpha = r it is B A); the "same grid" is the current fp16 scales; the prior of
the scale solve is centred on those scales.

The earlier finisher (v0.2 of the Qwen3-4B card, "GPTQ codes + joint scales"
in its "Why the solver changed"; the Agents-A1 card's finisher) re-solves the
codes of the watered target with the GPTQ sweep instead (``wring_gptq``).
Reading: the sweep runs on W' with the damped H exactly as the first solve does
(its own absmax block scales), and the joint solve's prior is centred on the
sweep's scales, the ones its codes were rounded against.

A third finisher of the same comparison ("nearest-point codes + block scale
search", Qwen3-4B card, "Why the solver changed") searches each block's scale
instead of solving for it (``wring_scale_search``).  Reading (the card gives no
search grid): candidates s_k = fp16(alpha_k max|w'| / L) with alpha_k = 1 - k/64,
k = 0 .. 31 (the absmax scale and 31 smaller ones down to about half of it);
each candidate's codes are the nearest levels of w'/s_k; the candidate with
the smallest squared error sum_j (w'_j - s_k (2 c_j - L))^2 of the block is
kept (the smaller k on a tie); no joint solve follows.
"""

import numpy as np

from .gptq import gptq_sweep
from .grid import dequant, fp16_rne, levels_count, nearest_code
from .joint import joint_scales


def wring_target(codes, scales, bits, group, B, A, alpha):
    """W' = dequant(codes, scales) + (alpha / r) B A, in float64."""
    W_hat = dequant(codes, scales, bits, group)
    if B is None or A is None:
        return W_hat
    B = np.asarray(B, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    r = A.shape[0]
    return W_hat + (float(alpha) / r) * (B @ A)


def wring(codes, scales, bits, group, B, A, alpha, H, lam):
    """Nearest-point recode of W' on the current scales, then joint scales against W'.

    Returns dict(codes, scales, scales_unrounded, target, t).
    """
    codes = np.asarray(codes, dtype=np.int64)
    rows, n = codes.shape
    Wp = wring_target(codes, scales, bits, group, B, A, alpha)
    L = np.broadcast_to(levels_count(bits), (rows,)).reshape(rows, 1)
    s = np.repeat(np.asarray(scales, dtype=np.float64), group, axis=1)
    t = np.divide(Wp, s, out=np.zeros_like(Wp), where=s > 0)
    c_new = nearest_code(t, L)
    s_new, s_raw = joint_scales(c_new, bits, group, H, Wp, scales, lam)
    return {"codes": c_new, "scales": s_new, "scales_unrounded": s_raw, "target": Wp, "t": t}


def wring_gptq(codes, scales, bits, group, B, A, alpha, H, lam):
    """GPTQ sweep of W' with H, then joint scales against W' with the prior at the sweep's scales.

    Returns dict(codes, scales, scales_unrounded, target, t, sweep_scales).
    """
    Wp = wring_target(codes, scales, bits, group, B, A, alpha)
    g = gptq_sweep(Wp, H, bits, group)
    s_new, s_raw = joint_scales(g["codes"], bits, group, H, Wp, g["scales"], lam)
    return {"codes": g["codes"], "scales": s_new, "scales_unrounded": s_raw, "target": Wp, "t": g["t"],
            "sweep_scales": g["scales"]}


SEARCH_CANDIDATES = 32


def scale_search_block(w, L):
    """Best candidate for one block w (1-D): returns (scale, codes, error, k)."""
    w = np.asarray(w, dtype=np.float64)
    amax = np.max(np.abs(w))
    best = None
    for k in range(SEARCH_CANDIDATES):
        s = float(fp16_rne((1.0 - k / 64.0) * amax / L))
        t = w / s if s > 0 else np.zeros_like(w)
        c = nearest_code(t, L)
        err = float(np.sum((w - s * (2 * c - L)) ** 2))
        if best is None or err < best[2]:
            best = (s, c, err, k)
    return best


def wring_scale_search(codes, scales, bits, group, B, A, alpha):
    """Nearest-point codes with a searched scale per block of W' (no joint solve).

    Returns dict(codes, scales, target, errors (rows x nb), k (rows x nb))."""
    codes = np.asarray(codes, dtype=np.int64)
    rows, n = codes.shape
    nb = n // group
    Wp = wring_target(codes, scales, bits, group, B, A, alpha)
    L = np.broadcast_to(levels_count(bits), (rows,))
    c_new = np.zeros((rows, n), dtype=np.int64)
    s_new = np.zeros((rows, nb))
    errs = np.zeros((rows, nb))
    ks = np.zeros((rows, nb), dtype=np.int64)
    for r in range(rows):
        for b in range(nb):
            s, c, e, k = scale_search_block(Wp[r, b * group:(b + 1) * group], int(L[r]))
            c_new[r, b * group:(b + 1) * group] = c
            s_new[r, b], errs[r, b], ks[r, b] = s, e, k
    return {"codes": c_new, "scales": s_new, "target": Wp, "errors": errs, "k": ks}
