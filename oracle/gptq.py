"""GPTQ / LDLQ column sweep with error feedback (oracle, test infrastructure only).

Pingala-8 post, "Trick 2: round with error feedback": columns of the weight
matrix are quantized one at a time and each column's error is pushed onto the
columns not yet quantized in proportions set by H (LDLQ); the [0.4, 0.4, 0.4]
toy shows the mechanism; a diagonal H reduces it to plain rounding.  Wringer
model cards ("Recipe"): starting codes are solved by GPTQ per layer with a full
second-order matrix onto a fixed signed grid with fp16 block scales.

The sweep used here is the GPTQ push form, for each row independently and the
columns in natural order (no reordering is described):

    U = upper Cholesky factor of H^-1 (H^-1 = U^T U)
    for k = 0 .. n-1:
        at a block start: s = fp16(max_{j in block} |w~_j| / L), from the
                          current, feedback-updated values
        t = w~_k / s;  c_k = nearest code;  q_k = (2 c_k - L) s
        e = (w~_k - q_k) / U_kk;   w~_j -= e U_kj  for all j > k

Readings: the scale of a block is fixed when the sweep reaches the block (the
pages only say block scales); an all-zero block gets s = 0 and the middle
upper code, which dequantises to 0.
"""

import numpy as np
import scipy.linalg

from .grid import fp16_rne, levels_count, nearest_code


def upper_cholesky_of_inverse(H):
    """Upper-triangular U with H^-1 = U^T U (H symmetric positive definite)."""
    H = np.asarray(H, dtype=np.float64)
    n = H.shape[0]
    cf = scipy.linalg.cho_factor(H, lower=True)        # raises LinAlgError when H is not PD
    Hinv = scipy.linalg.cho_solve(cf, np.eye(n))
    Hinv = 0.5 * (Hinv + Hinv.T)
    return np.linalg.cholesky(Hinv).T


def feedback_sweep(W, U, round_column):
    """Error-feedback sweep over the columns of W (rows x n) in natural order.

    ``round_column(k, Wt)`` returns the quantized values q of column k given the
    current feedback-updated matrix Wt (it may read other columns, e.g. to fix
    a block scale at a block start).  The error of each column is pushed onto
    all later columns through row k of U.  Returns (Q, pre) where Q holds the
    quantized values and pre the values each column had when it was rounded.
    """
    Wt = np.array(W, dtype=np.float64, copy=True)
    rows, n = Wt.shape
    Q = np.empty_like(Wt)
    pre = np.empty_like(Wt)
    for k in range(n):
        pre[:, k] = Wt[:, k]
        q = round_column(k, Wt)
        Q[:, k] = q
        e = (Wt[:, k] - q) / U[k, k]
        Wt[:, k + 1:] -= np.outer(e, U[k, k + 1:])
    return Q, pre


def integer_feedback_round(w, H):
    """Error feedback onto the integer grid with unit scale (the toy of 'Trick 2').

    w is one row (or rows x n); returns (q, pre) with the integers chosen and
    the value each weight had when it was rounded.
    """
    W = np.atleast_2d(np.asarray(w, dtype=np.float64))
    U = upper_cholesky_of_inverse(H)
    Q, pre = feedback_sweep(W, U, lambda k, Wt: np.floor(Wt[:, k] + 0.5))
    return Q.reshape(np.shape(w)), pre.reshape(np.shape(w))


def gptq_sweep(W, H, bits, group):
    """GPTQ codes and fp16 block scales for W (rows x n) given the damped H (n x n).

    ``bits`` is an int or a per-row array.  Returns a dict with
      codes  (rows x n, int64 in [0, L]),
      scales (rows x n/group, float64 holding fp16 values),
      t      (rows x n, the value of each weight in level units when rounded),
      U      (the factor used).
    """
    W = np.asarray(W, dtype=np.float64)
    rows, n = W.shape
    if n % group != 0:
        raise ValueError("n must be a multiple of the group size")
    nb = n // group
    L = np.broadcast_to(levels_count(bits), (rows,)).astype(np.float64)
    U = upper_cholesky_of_inverse(H)
    codes = np.zeros((rows, n), dtype=np.int64)
    scales = np.zeros((rows, nb), dtype=np.float64)
    tvals = np.zeros((rows, n), dtype=np.float64)

    def round_column(k, Wt):
        b = k // group
        if k % group == 0:
            scales[:, b] = fp16_rne(np.max(np.abs(Wt[:, k:k + group]), axis=1) / L)
        s = scales[:, b]
        t = np.divide(Wt[:, k], s, out=np.zeros(rows), where=s > 0)
        c = nearest_code(t, L)
        codes[:, k] = c
        tvals[:, k] = t
        return (2 * c - L) * s

    feedback_sweep(W, U, round_column)
    return {"codes": codes, "scales": scales, "t": tvals, "U": U}
