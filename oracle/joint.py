"""Joint least-squares block scales with a prior (oracle, test infrastructure only).

Wringer model cards, "Recipe": block scales are solved by a joint
least-squares closed form with a prior (lambda = 0.01); "Why the solver
changed": the same joint closed-form scale solve finishes the wring.  Agents-A1
card, "Honest caveats": scales are projected to fp16 at solve time.

For one row with codes c (levels l_j = 2 c_j - L), target t and current scales
s0, the scales minimise

    f(s) = (t - Q s)^T H (t - Q s) + lambda * mu * ||s - s0||^2,

where Q is n x nb with Q[j, block(j)] = l_j, so Q s is the dequantised row.
Closed form: with G = Q^T H Q, h = Q^T H t and mu = trace(G) / nb,

    s = (G + lambda mu I)^-1 (h + lambda mu s0),   then s <- fp16(s).

Readings: the prior is centred on the scales the codes were rounded against
and weighted by lambda * mu (mu = trace(G)/nb makes lambda unitless); H is the
damped matrix.
"""

import numpy as np

from .grid import fp16_rne, levels_count, level_of


def row_gram(levels_row, H, group):
    """G[b, c] = sum_{j in b, l in c} l_j H[j, l] l_l  (= Q^T H Q) for one row."""
    lev = np.asarray(levels_row, dtype=np.float64)
    n = lev.shape[0]
    nb = n // group
    K = lev[:, None] * H * lev[None, :]
    return K.reshape(nb, group, nb, group).sum(axis=(1, 3))


def joint_scales(codes, bits, group, H, target, s0, lam):
    """Per-row joint scales.  Returns (scales_fp16, scales_unrounded), each rows x nb float64."""
    codes = np.asarray(codes, dtype=np.int64)
    H = np.asarray(H, dtype=np.float64)
    T = np.asarray(target, dtype=np.float64)
    S0 = np.asarray(s0, dtype=np.float64)
    rows, n = codes.shape
    if n % group != 0:
        raise ValueError("n must be a multiple of the group size")
    nb = n // group
    L = np.broadcast_to(levels_count(bits), (rows,))
    out = np.zeros((rows, nb), dtype=np.float64)
    for r in range(rows):
        lev = level_of(codes[r], L[r]).astype(np.float64)
        G = row_gram(lev, H, group)
        h = (lev * (H @ T[r])).reshape(nb, group).sum(axis=1)
        mu = np.trace(G) / nb
        A = G + lam * mu * np.eye(nb)
        out[r] = np.linalg.solve(A, h + lam * mu * S0[r])
    return fp16_rne(out), out
