"""Product of a packed module with input vectors (oracle, test infrastructure only).

Wringer model cards, "What is in this repo": the container holds packed codes and fp16 block
scales of the weights in the stored basis (rotated and zero-padded input dim); the pages name a
kernel that multiplies packed codes with the activations as the missing piece for decoding
from the container (the Agents-A1 card converts the same layout for a 4-bit kernel; the
Pingala-8 post decodes its codes inside the matrix-vector product).

For a module stored as W_s = W R^T (rows v -> R v, R = blockdiag(H_m diag(d)) / sqrt(m)) with
quantized rows W_q: y = W_q R x_pad, where x_pad is x zero-padded to n_store, so the input is
rotated once and multiplied with the dequantized stored weights.
"""

import numpy as np

from .grid import dequant
from .pack import unpack
from .rotation import rotate_rows


def packed_gemv(buf, rows, n_store, bits, group, had_block, signs, X):
    """Y (batch x rows) = X_pad R^T W_q^T for input rows X (batch x n_in, n_in <= n_store), fp64."""
    X = np.atleast_2d(np.asarray(X, dtype=np.float64))
    batch, n_in = X.shape
    Xp = np.zeros((batch, n_store))
    Xp[:, :n_in] = X
    if had_block:
        Xp = rotate_rows(Xp, had_block, signs)  # each row x -> R x
    codes, scales = unpack(buf, rows, n_store, bits, group)
    Wq = dequant(codes, scales, bits, group)
    return Xp @ Wq.T
