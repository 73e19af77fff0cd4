"""Measures used to compare results (oracle, test infrastructure only).

* proxy loss tr(dW H0 dW^T): the objective the error-feedback rounding works
  on -- the layer cares about its output (Pingala-8 post, "Trick 2"); it is
  evaluated with the undamped H0.
* ledger bits per weight = (code bits + 16 bits per block scale) / weights
  (Wringer model cards, "Recipe": "code 2.520 + scales 0.119 = 2.638 b/w").
* distance of a pre-rounding value to the nearest decision threshold of the
  odd grid (thresholds sit at the even integers strictly inside (-L, L)).
"""

import numpy as np


def proxy_loss(W_target, W_hat, H0):
    """sum_r (W_target - W_hat)_r H0 (W_target - W_hat)_r^T."""
    D = np.asarray(W_target, dtype=np.float64) - np.asarray(W_hat, dtype=np.float64)
    return float(np.sum((D @ np.asarray(H0, dtype=np.float64)) * D))


def ledger_bits_per_weight(weights, code_bits_total, n_scales, scale_bits=16):
    """(code bits + scale bits) / weights, and its two parts."""
    code = code_bits_total / weights
    scale = n_scales * scale_bits / weights
    return code + scale, code, scale


def threshold_distance(t, L):
    """|t - theta| for the decision threshold theta (even integer in (-L, L)) nearest to t."""
    t = np.asarray(t, dtype=np.float64)
    L = np.asarray(L, dtype=np.float64)
    theta = np.clip(2.0 * np.round(t / 2.0), -(L - 1), L - 1)
    return np.abs(t - theta)
