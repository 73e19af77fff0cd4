"""Plain fp64 CPU oracle for the per-linear-layer Wringer quantization solve.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP library (no kernels, headers, helpers, tables or pre/post-processing);
it takes numpy arrays and returns numpy arrays, everything widened to float64.

Sources (titles of the pages the method is described on):

* "Wringer Compresses Low-Rank Distillation Results Back into Low-Bit Weights,
  but So Far It Only Saves Storage Space" (news article on Wringer): GPTQ with
  a full second-order matrix, a signed even grid and Tikhonov regularisation;
  the wring re-solves codes and scales against the target ``Wq + BA/r``.
* Model card "Wringer — Qwen3-4B at 2.638 bits/weight", sections "Recipe" and
  "Why the solver changed": GPTQ codes, joint least-squares closed-form block
  scales with a prior (lambda = 0.01), wring = nearest-point codes on the same
  grid followed by the same joint scale solve against the watered weights.
* Model card "Wringer p3b_w2 — Agents-A1-4B at 2.655 bits/weight", sections
  "Recipe" and "Honest caveats" (scale precision): fp16 block scales, projected
  to fp16 at solve time.
* Post "How We Shrank an AI Model by 85% and Kept 90% of Its Smarts"
  (Pingala-8), sections "Trick 1: rotate the weights first" (Hadamard rotation
  and its 4x4 worked example) and "Trick 2: round with error feedback" (the
  [0.4, 0.4, 0.4] toy, LDLQ, H as the average of x x^T, diagonal H reduces to
  plain rounding).

Every function here is pinned by a CPU test in ``tests/test_oracle_*.py``
against worked examples, closed forms, invariants or brute force.
"""

from .hessian import second_moment, second_moment_chunks, sum_of_products, pad_square, damp
from .rotation import sylvester, rotation_matrix, rotate_rows, rotate_rows_inverse, rotate_sym
from .grid import fp16_rne, levels_count, nearest_code, level_of, dequant
from .gptq import upper_cholesky_of_inverse, feedback_sweep, gptq_sweep, integer_feedback_round
from .joint import joint_scales, row_gram
from .wring import wring_target, wring, wring_gptq, wring_scale_search, scale_search_block
from .pack import pack, unpack, packed_bytes, code_bytes_per_row
from .metrics import (proxy_loss, ledger_bits_per_weight, threshold_distance, grid_representation,
                      grid_distance, code_disagreement, projection_ulp_moves)
from .solve import solve_module, solve_rows
from .materialize import bf16_rne_bits, bf16_bits_to_f64, materialize, materialize_exact
from .trellis import viterbi as trellis_viterbi, greedy as trellis_greedy, decode as trellis_decode
from .gemv import packed_gemv

__all__ = [
    "second_moment", "second_moment_chunks", "sum_of_products", "pad_square", "damp",
    "sylvester", "rotation_matrix", "rotate_rows", "rotate_rows_inverse", "rotate_sym",
    "fp16_rne", "levels_count", "nearest_code", "level_of", "dequant",
    "upper_cholesky_of_inverse", "feedback_sweep", "gptq_sweep", "integer_feedback_round",
    "joint_scales", "row_gram",
    "wring_target", "wring", "wring_gptq", "wring_scale_search", "scale_search_block",
    "pack", "unpack", "packed_bytes", "code_bytes_per_row",
    "proxy_loss", "ledger_bits_per_weight", "threshold_distance", "grid_representation", "grid_distance",
    "code_disagreement", "projection_ulp_moves",
    "solve_module", "solve_rows",
    "bf16_rne_bits", "bf16_bits_to_f64", "materialize", "materialize_exact",
    "trellis_viterbi", "trellis_greedy", "trellis_decode",
    "packed_gemv",
]
