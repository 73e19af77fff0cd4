"""Materializing a packed module as bf16 weights (oracle, test infrastructure only).

Wringer model cards, "What is in this repo": a materializer turns the container
(packed codes plus fp16 block scales) and the bf16 source export into the
fake-quant bf16 checkpoint that inference loads; "Honest caveats": the weights
are materialized at ledger precision (fp16 scales).

Reading used here (the pages do not say where the one rounding to bf16 falls):
the dequantized weights (2c - L) s are exact, the inverse of the storage
rotation (each row v -> R^T v) is applied exactly, the zero-padded input
columns are dropped, and each weight is rounded to bf16 once, to nearest with
ties to even.

Since the rounding is taken once, the weights before it must carry no rounding
of their own where it could move a bf16 decision.  R^T v = diag(d) H_m v / sqrt(m)
(Pingala-8 post, "Trick 1: rotate the weights first"): the product H_m v of the unnormalised
Sylvester matrix with v is exact in fp64 here (each entry of v is an odd level
below 16 times an fp16 scale, so every partial sum is an integer multiple of the
smallest scale's ulp below 2^53 of it), and the one division by sqrt(m) rounds
once, so an output whose exact value is zero (the block's sum cancels) comes out
zero, not as the residue of a normalised product.
"""

import numpy as np

from .grid import dequant
from .pack import unpack
from .rotation import _check, sylvester


def bf16_rne_bits(x):
    """bf16 bit patterns of x (float64 array), rounded once to nearest, ties to even.

    A finite nonzero x = f 2^e with f in [0.5, 1); bf16 keeps 8 significant bits, so
    the representable neighbours are multiples of q = 2^(e - 8) and x / q is exact.
    (Normal range only: |x| in [2^-126, 2^128).)
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    q = np.ldexp(1.0, e - 8)
    r = np.where(x == 0.0, x, np.rint(x / q) * q)  # rint: ties to even; a zero keeps its sign
    r32 = r.astype(np.float32)  # exact: 8 significant bits
    return (r32.view(np.uint32) >> 16).astype(np.uint16)


def bf16_bits_to_f64(bits):
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def _inverse_rotation_exact(w, m, signs):
    """Each row v of w -> diag(d) (H_m v) / sqrt(m), block by block, H_m unnormalised."""
    n = w.shape[1]
    signs = _check(n, m, signs)
    Hm = sylvester(m)
    out = np.empty_like(w)
    for k in range(n // m):
        sl = slice(k * m, (k + 1) * m)
        out[:, sl] = (w[:, sl] @ Hm) / np.sqrt(m) * signs[sl][None, :]  # H_m is symmetric
    return out


def materialize_exact(buf, rows, n_store, bits, group, had_block, signs, n_out):
    """The fp64 weights before the bf16 rounding (rows x n_out)."""
    codes, scales = unpack(buf, rows, n_store, bits, group)
    w = dequant(codes, scales, bits, group)
    if had_block:
        w = _inverse_rotation_exact(w, had_block, signs)
    return w[:, :n_out]


def materialize(buf, rows, n_store, bits, group, had_block, signs, n_out):
    """bf16 bit patterns (rows x n_out, uint16) of the module's weights in the input basis."""
    return bf16_rne_bits(materialize_exact(buf, rows, n_store, bits, group, had_block, signs, n_out))
