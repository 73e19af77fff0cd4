"""Comparison helpers for GPU-vs-oracle parity (test infrastructure)."""
import numpy as np

import oracle


def f16_bits(x):
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.int16).astype(np.int64)


def code_parity(gpu_codes, ref_codes, ref_t, L):
    """Fraction of differing codes and, per row with a difference, the oracle's distance of the
    first differing weight to its nearest decision threshold (in level units)."""
    gpu_codes = np.asarray(gpu_codes)
    ref_codes = np.asarray(ref_codes)
    mism = gpu_codes != ref_codes
    rows = np.nonzero(mism.any(axis=1))[0]
    Lr = np.broadcast_to(np.asarray(L), (gpu_codes.shape[0],))
    first = []
    for r in rows:
        k = int(np.argmax(mism[r]))
        first.append(float(oracle.threshold_distance(ref_t[r, k], Lr[r])))
    return {"frac": float(mism.mean()), "rows": rows, "first_dist": first,
            "worst_first": max(first) if first else 0.0, "identical_rows": ~mism.any(axis=1)}


def scale_ulps(gpu_scales, ref_scales):
    return np.abs(f16_bits(gpu_scales) - f16_bits(ref_scales))
