"""The signed odd grid, nearest-point rounding and fp16 scale projection (oracle, test infrastructure only).

Wringer news article (second paragraph): a signed even grid.  Pingala-8 post,
"Why 2 bits is hard": the four 2-bit levels {-3, -1, 1, 3} times a group scale.
Reading used here: for b bits, L = 2^b - 1 and the levels are 2c - L for the
code c in [0, L] -- evenly spaced, symmetric, no zero level ({+-1, +-3} at 2
bits, {+-1, ..., +-7} at 3 bits).

Agents-A1-4B model card, "Honest caveats" (scale precision): block scales are
stored in fp16 and projected to fp16 when solved.  Reading: IEEE-754
round-to-nearest-even, sign kept, finite range clamped to +-65504.
"""

import numpy as np

FP16_MAX = 65504.0


def fp16_rne(x):
    """Round float64 values to the nearest fp16 value (ties to even), returned as float64."""
    x = np.clip(np.asarray(x, dtype=np.float64), -FP16_MAX, FP16_MAX)
    return x.astype(np.float16).astype(np.float64)


def levels_count(bits):
    """L = 2^b - 1 (the largest code); accepts a scalar or an array of per-row bit widths."""
    b = np.asarray(bits, dtype=np.int64)
    if np.any((b < 2) | (b > 4)):
        raise ValueError("bits must be 2, 3 or 4")
    return (1 << b) - 1


def nearest_code(t, L):
    """Nearest level index for t in level units: c = clamp(floor((t + L)/2 + 1/2), 0, L).

    Level 2c - L is the grid point nearest to t; an exact tie between two
    levels goes to the upper one.
    """
    t = np.asarray(t, dtype=np.float64)
    return np.clip(np.floor((t + L) / 2.0 + 0.5), 0, L).astype(np.int64)


def level_of(codes, L):
    """Signed odd level 2c - L of each code."""
    return 2 * np.asarray(codes, dtype=np.int64) - L


def dequant(codes, scales, bits, group):
    """W_hat[r, j] = (2 c[r, j] - L_r) * s[r, j // group], exact in float64."""
    codes = np.asarray(codes, dtype=np.int64)
    rows, n = codes.shape
    L = np.broadcast_to(levels_count(bits), (rows,)).reshape(rows, 1)
    s = np.repeat(np.asarray(scales, dtype=np.float64), group, axis=1)[:, :n]
    return level_of(codes, L).astype(np.float64) * s
