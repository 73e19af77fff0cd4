"""Calibration second moment and its Tikhonov damping (oracle, test infrastructure only).

H is the average of x x^T over calibration inputs: Pingala-8 post, "Trick 2:
round with error feedback" (the LDLQ paragraph).  The Wringer news article
(second paragraph) says the GPTQ solve is Tikhonov-regularised; the strength
used here, frac * mean(diag H), is the one the toy-layer workload states.
"""

import numpy as np


def second_moment(X):
    """H0 = (1/N) X^T X for calibration rows X (N x n): uncentred, so H0 = mean_i x_i x_i^T."""
    X = np.asarray(X, dtype=np.float64)
    if X.ndim != 2 or X.shape[0] == 0:
        raise ValueError("X must be a non-empty N x n matrix")
    return (X.T @ X) / X.shape[0]


def second_moment_chunks(chunks):
    """H0 = (1/N) sum over chunks of X_k^T X_k: the same average as second_moment, for calibration
    rows that arrive in chunks (N = total rows).  Each chunk is widened to float64."""
    S = None
    N = 0
    for X in chunks:
        Xd = np.asarray(X, dtype=np.float64)
        part = Xd.T @ Xd
        S = part if S is None else S + part
        N += Xd.shape[0]
    if S is None or N == 0:
        raise ValueError("no calibration rows")
    return S / N


def sum_of_products(X, pairs):
    """S[i, j] = sum over rows of x_i x_j for each (i, j) in pairs, one entry at a time (float64)."""
    X = np.asarray(X, dtype=np.float64)
    return np.array([float(np.dot(X[:, i], X[:, j])) for i, j in pairs])


def pad_square(H0, n_store):
    """Zero-pad an n x n matrix to n_store x n_store (the padded input dims carry no signal)."""
    n = H0.shape[0]
    if n_store < n:
        raise ValueError("n_store must be >= n")
    out = np.zeros((n_store, n_store), dtype=np.float64)
    out[:n, :n] = H0
    return out


def damp(H0, frac):
    """H = H0 + delta I with delta = frac * trace(H0) / n, n the stored (possibly padded) dimension.

    Returns (H, delta).  The trace is invariant under the orthogonal rotation,
    so damping before or after rotating gives the same H.
    """
    H0 = np.asarray(H0, dtype=np.float64)
    n = H0.shape[0]
    delta = float(frac) * float(np.trace(H0)) / n
    return H0 + delta * np.eye(n), delta
