"""Random-sign Hadamard rotation (oracle, test infrastructure only).

Pingala-8 post, "Trick 1: rotate the weights first": for orthogonal R,
W x = (W R^T)(R x), so the stored weights become W R^T (each weight row w
becomes R w) and the inputs become R x; H0 = E[x x^T] becomes R H0 R^T.  The
post uses a Hadamard matrix with random signs and prints the natural-order 4x4
one scaled by 1/2.

Reading used here: R = blockdiag_k(H_m diag(d_k)) / sqrt(m), with H_m the
natural-order (Sylvester) Hadamard matrix of order m (a power of two), d_k the
+-1 signs of block k, and the stored dimension a multiple of m (zero-padded).
"""

import numpy as np


def sylvester(m):
    """Natural-order Hadamard matrix: H_1 = [1], H_2k = [[H_k, H_k], [H_k, -H_k]]."""
    if m < 1 or (m & (m - 1)) != 0:
        raise ValueError("Hadamard order must be a power of two")
    Hm = np.ones((1, 1), dtype=np.float64)
    while Hm.shape[0] < m:
        Hm = np.block([[Hm, Hm], [Hm, -Hm]])
    return Hm


def _check(n, m, signs):
    signs = np.asarray(signs, dtype=np.float64).reshape(-1)
    if n % m != 0:
        raise ValueError("stored dimension must be a multiple of the Hadamard block")
    if signs.shape[0] != n or not np.all(np.abs(signs) == 1.0):
        raise ValueError("signs must be +-1 of length n")
    return signs


def rotation_matrix(n, m, signs):
    """Dense R = blockdiag_k(H_m diag(d_k)) / sqrt(m) (only for small n)."""
    signs = _check(n, m, signs)
    Hm = sylvester(m)
    R = np.zeros((n, n), dtype=np.float64)
    for k in range(n // m):
        sl = slice(k * m, (k + 1) * m)
        R[sl, sl] = Hm * signs[sl][None, :] / np.sqrt(m)
    return R


def rotate_rows(M, m, signs):
    """Replace each row v of M (rows x n) by R v, i.e. return M R^T, block by block."""
    M = np.asarray(M, dtype=np.float64)
    n = M.shape[1]
    signs = _check(n, m, signs)
    Hm = sylvester(m) / np.sqrt(m)
    out = np.empty_like(M)
    for k in range(n // m):
        sl = slice(k * m, (k + 1) * m)
        # (H_m diag(d) v)^T = v^T diag(d) H_m^T
        out[:, sl] = (M[:, sl] * signs[sl][None, :]) @ Hm.T
    return out


def rotate_rows_inverse(M, m, signs):
    """Replace each row v of M by R^T v (undoes rotate_rows)."""
    M = np.asarray(M, dtype=np.float64)
    n = M.shape[1]
    signs = _check(n, m, signs)
    Hm = sylvester(m) / np.sqrt(m)
    out = np.empty_like(M)
    for k in range(n // m):
        sl = slice(k * m, (k + 1) * m)
        # (diag(d) H_m^T v)^T = v^T H_m diag(d)
        out[:, sl] = (M[:, sl] @ Hm) * signs[sl][None, :]
    return out


def rotate_sym(H, m, signs):
    """Two-sided rotation R H R^T of a square matrix (rows pass, then columns pass)."""
    Y = rotate_rows(H, m, signs)          # H R^T
    return rotate_rows(Y.T, m, signs).T   # R (H R^T)
