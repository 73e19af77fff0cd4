"""Measures used to compare results (oracle, test infrastructure only).

* proxy loss tr(dW H0 dW^T): the objective the error-feedback rounding works
  on -- the layer cares about its output (Pingala-8 post, "Trick 2"); it is
  evaluated with the undamped H0.
* ledger bits per weight = (code bits + 16 bits per block scale) / weights
  (Wringer model cards, "Recipe": "code 2.520 + scales 0.119 = 2.638 b/w").
* distance of a pre-rounding value to the nearest decision threshold of the
  odd grid (thresholds sit at the even integers strictly inside (-L, L)).
* the three measures the model cards report on their solves: the relative
  Frobenius distance of weights from their nearest representation on the
  joint-scale grid (Qwen3-4B card, "Why the solver changed": 0.46 for the parent
  weights, 0.07 for the filled ones), the share of codes on which the GPTQ and
  nearest-point solvers disagree (same section: 18 % at zero training, 1.7 %
  after the fill), and the share of bf16 weights that projecting the scales to
  fp16 at solve time moves by one ulp (Agents-A1 card, "Honest caveats": 2.95 %).

Readings: the "nearest representation on the joint-scale grid" of weights T is
the nearest-point codes of T on the current fp16 scales followed by the joint
scale solve against T (``grid_representation``), the wring's own finisher; the
one-ulp share compares the bf16 rounding of each stored-basis weight (2c - L) s
under the fp16 scale with that under the unprojected solution of the scale
solve.
"""

import numpy as np

from .grid import dequant, levels_count, nearest_code
from .joint import joint_scales
from .materialize import bf16_rne_bits


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


def grid_representation(T, scales, bits, group, H, lam):
    """Nearest-point codes of T (rows x n) on the fp16 scales, then joint scales against T with the
    prior centred on those scales.  Returns (codes, fp16 scales, unprojected scales)."""
    T = np.asarray(T, dtype=np.float64)
    rows, n = T.shape
    L = np.broadcast_to(levels_count(bits), (rows,)).reshape(rows, 1)
    s = np.repeat(np.asarray(scales, dtype=np.float64), group, axis=1)
    t = np.divide(T, s, out=np.zeros_like(T), where=s > 0)
    codes = nearest_code(t, L)
    s16, s_raw = joint_scales(codes, bits, group, H, T, scales, lam)
    return codes, s16, s_raw


def grid_distance(T, codes, scales, bits, group):
    """||T - dequant(codes, scales)||_F / ||T||_F."""
    T = np.asarray(T, dtype=np.float64)
    return float(np.linalg.norm(T - dequant(codes, scales, bits, group)) / np.linalg.norm(T))


def code_disagreement(codes_a, codes_b):
    """Share of positions where two code matrices differ."""
    return float(np.mean(np.asarray(codes_a) != np.asarray(codes_b)))


def projection_ulp_moves(codes, scales16, scales_raw, bits, group):
    """Share of weights whose bf16 rounding of (2c - L) s changes when the fp16 scale replaces the
    unprojected one (both products exact in fp64, rounded to bf16 once)."""
    codes = np.asarray(codes, dtype=np.int64)
    a = bf16_rne_bits(dequant(codes, scales16, bits, group))
    b = bf16_rne_bits(dequant(codes, scales_raw, bits, group))
    return float(np.mean(a != b))
