/*
 * wringer.h -- C ABI of the MI355X (gfx950) per-linear-layer quantization solve.
 *
 * The solve quantizes one linear layer W (rows x n, rows = output channels)
 * given calibration inputs X (N x n):
 *
 *   (a) H = X^T X / N + delta I          wr_hessian_accumulate, wr_hessian_finalize
 *   (b) optional random-sign Hadamard    wr_hadamard_rotate
 *   (c) GPTQ/LDLQ error-feedback sweep   wr_gptq_sweep
 *   (d) joint scales / the wring         wr_wring_solve
 *   (e) bit packing                      wr_pack, wr_unpack
 *
 * Conventions shared by every entry point:
 *   - Matrices are row-major with an explicit leading dimension (in elements).
 *   - Every data pointer is a DEVICE pointer owned by the caller; the library
 *     never frees or retains it past the call.  Inputs are const.
 *   - Work is enqueued on the context's HIP stream and the call returns
 *     without synchronising.  Argument errors are detected on the host before
 *     anything is launched and leave every output untouched.
 *   - The library allocates no device memory.  Entry points that need scratch
 *     space use the workspace registered with wr_set_workspace; its size comes
 *     from wr_workspace_bytes.  (The one exception, wr_hessian_accumulate_noalloc,
 *     uses a static device array that the HIP runtime places with the library's
 *     code on each GPU.)
 *   - Numerical failures are reported LAPACK-style through a device int32
 *     `dev_info` (read it after synchronising the stream): 0 = success;
 *     k > 0 = H is not numerically positive definite (the Cholesky
 *     factorisation of the reversed H, J H J, failed at pivot k, 1-based);
 *     -1 = a non-finite value in the weights/target.  On failure the kernels
 *     that would write codes or scales return without writing them.
 *   - Return value: WR_OK (0) or a positive WR_E* code; no exception crosses
 *     the ABI.  One context per stream; a context is not thread-safe.
 *
 * Grid: for b bits, L = 2^b - 1, codes c in [0, L] stand for the signed odd
 * levels 2c - L ({+-1, +-3} at 2 bits, {+-1..+-7} at 3 bits) times an fp16
 * block scale shared by `group` consecutive weights of a row.
 */
#ifndef WRINGER_H
#define WRINGER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum wr_status {
  WR_OK = 0,
  WR_EINVAL = 1,       /* invalid argument (null pointer, bad size, bad flag) */
  WR_EWORKSPACE = 2,   /* registered workspace missing or too small */
  WR_EHIP = 3,         /* a HIP runtime call failed */
  WR_EUNSUPPORTED = 4, /* valid request the library does not implement */
  WR_ESCRATCH = 5      /* request too large for the static scratch of an allocation-free entry point */
};

/* Device scratch, per GPU, of the allocation-free entry point (wr_hessian_accumulate_noalloc). */
#define WR_STATIC_SCRATCH_BYTES ((size_t)64 << 20)

enum wr_dtype { WR_F32 = 0, WR_BF16 = 1 };

enum wr_op {             /* operations that need workspace, for wr_workspace_bytes */
  WR_OP_HESSIAN = 0,     /* rows = calibration rows per call, n = input dim */
  WR_OP_GPTQ = 1,        /* rows = weight rows, n = stored dim, group, lazy_batch */
  WR_OP_WRING = 2,       /* rows = weight rows, n = stored dim, group, rank */
  WR_OP_ROTATE = 3,      /* none needed; returns 0 */
  WR_OP_FINALIZE = 4,    /* n = n_store; needed by wr_hessian_finalize with a rotation */
  WR_OP_WRING_GPTQ = 5,  /* rows, n, group, rank: wr_wring_solve with WR_RECODE_GPTQ */
  WR_OP_TRELLIS = 6,     /* rows, n, group = number of trellis states: wr_trellis_quantize */
  WR_OP_GEMV = 7,        /* rows = number of input vectors, n = n_store: wr_packed_gemv */
  WR_OP_STATS = 8        /* rows: wr_quant_stats */
};

enum wr_hessian_flags { WR_H_ZERO = 1 };               /* zero S before accumulating */
enum wr_rotate_mode { WR_ROT_ROWS = 0, WR_ROT_ROWS_INVERSE = 1, WR_ROT_SYM = 2 };
enum wr_wring_flags { WR_RECODE_NEAREST = 1, WR_RECODE_GPTQ = 2, WR_RECODE_SEARCH = 4 };

typedef struct wr_ctx wr_ctx;

/* Create a context bound to HIP device `device` and stream `hip_stream`
 * (a hipStream_t; NULL = the default stream).  *out receives the handle. */
int wr_create(wr_ctx** out, int device, void* hip_stream);
int wr_destroy(wr_ctx* ctx);

/* Device scratch bytes an operation needs for the given problem size. */
size_t wr_workspace_bytes(int op, int64_t rows, int64_t n, int32_t group, int32_t rank, int32_t lazy_batch);

/* Register caller-owned device scratch memory (256-byte aligned) for later calls. */
int wr_set_workspace(wr_ctx* ctx, void* dev_ptr, size_t bytes);

/*
 * (a) Calibration second moment.  H is the average of x x^T over the
 * calibration inputs (Pingala-8 post "How We Shrank an AI Model by 85% and
 * Kept 90% of Its Smarts", section "Trick 2: round with error feedback").
 *
 * S (n x n, fp64, ld n) += X^T X over the `rows` rows of X (rows x n, dtype
 * WR_BF16 or WR_F32, leading dimension ldx).  Only the lower triangle
 * (including the diagonal) of S is defined.  With WR_H_ZERO, S is zeroed
 * first.  Call once per chunk of calibration rows.  n % 8 == 0; for bf16 X,
 * ldx % 8 == 0 and X 16-byte aligned; ldx <= 2^24 (WR_EUNSUPPORTED above).
 * Products are exact: bf16 inputs directly, fp32 inputs as three bf16 parts
 * (x = x0 + x1 + x2, six cross terms).  The matrix cores sum at most 32768 rows
 * (512 for fp32 X) in fp32 before the sums are added into S in fp64, in a fixed
 * order: the result is deterministic with a relative error near 1e-7.
 * Workspace: WR_OP_HESSIAN with (rows, n).  rows may be 0 (no-op unless
 * WR_H_ZERO).
 */
int wr_hessian_accumulate(wr_ctx* ctx, const void* X, int x_dtype, int64_t rows, int64_t n, int64_t ldx,
                          double* S, int flags);

/*
 * Allocation-free variant of wr_hessian_accumulate, for callers that cannot allocate device
 * memory or register a workspace (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  Same arguments, operation and accuracy; the registered workspace is
 * not used.  Its scratch (the row splits' fp32 partial sums, and for fp32 X the three bf16 parts)
 * is a static device array of WR_STATIC_SCRATCH_BYTES per GPU, which the library holds from the
 * first wr_create on that GPU until the process ends.  bf16 X of any size: when the splits'
 * partials would not fit, fewer splits run at a time over row slices (each split still sums at
 * most 32768 rows in fp32); the result is bit-identical to wr_hessian_accumulate's when
 * wr_workspace_bytes(WR_OP_HESSIAN, rows, n, ...) <= WR_STATIC_SCRATCH_BYTES.  fp32 X: row
 * slices whose parts and partials fit; WR_ESCRATCH when not even 512 rows fit (n above 21845),
 * checked before any launch.  The call allocates nothing.  Every call on one GPU uses
 * that GPU's one array: calls that overlap on the same GPU (several streams, contexts or threads)
 * race and give wrong results; calls queued on one stream are safe.  Nothing in the array needs
 * to start at zero (every call writes what it reads).
 */
int wr_hessian_accumulate_noalloc(wr_ctx* ctx, const void* X, int x_dtype, int64_t rows, int64_t n, int64_t ldx,
                                  double* S, int flags);

/*
 * (a)+(b) Finalize, rotate and damp.  Writes the full symmetric H (n_store x
 * n_store, fp32, ld ldh):
 *   H = R pad(S / total_rows) R^T + delta I,
 *   delta = damp_frac * trace(S / total_rows) / n_store,
 * where pad() zero-fills rows/columns n..n_store-1 (the zero-padded input
 * dims) and R is the random-sign Hadamard rotation of wr_hadamard_rotate with
 * block had_block and signs (device int8, length n_store); had_block = 0 means
 * R = I.  The rotation runs in fp64 and H is rounded to fp32 once: rotating an
 * fp32 H would smear the rounding error of the large (outlier-channel)
 * entries over the small ones.  The damping is the Tikhonov regularisation
 * the Wringer news article names for the GPTQ solve (the trace is invariant
 * under R).  `delta_out` (device fp32, nullable) receives delta.
 * Workspace: 256 bytes, or WR_OP_FINALIZE (n = n_store) with a rotation.
 */
int wr_hessian_finalize(wr_ctx* ctx, const double* S, int64_t n, int64_t total_rows, float damp_frac,
                        int64_t n_store, float* H, int64_t ldh, float* delta_out, int32_t had_block,
                        const int8_t* signs);

/*
 * (b) Random-sign Hadamard rotation (Pingala-8 post, section "Trick 1:
 * rotate the weights first": W x = (W R^T)(R x)).
 * R = blockdiag_k(H_m diag(d_k)) / sqrt(m), H_m the natural-order (Sylvester)
 * Hadamard matrix of order m = had_block (a power of two, 2..4096),
 * d = signs (device int8, +-1, length n).  M is rows x n (fp32, ld), n a
 * multiple of m, transformed in place:
 *   WR_ROT_ROWS          each row v -> R v        (weights: W -> W R^T)
 *   WR_ROT_ROWS_INVERSE  each row v -> R^T v
 *   WR_ROT_SYM           M -> R M R^T             (requires rows == n; in fp32 --
 *                                                  wr_hessian_finalize rotates H in fp64)
 */
int wr_hadamard_rotate(wr_ctx* ctx, float* M, int64_t rows, int64_t n, int64_t ld, int32_t had_block,
                       const int8_t* signs, int mode);

/*
 * (c) GPTQ / LDLQ sweep (Pingala-8 post, "Trick 2"; Wringer model cards,
 * "Recipe": GPTQ codes on a fixed signed grid with fp16 block scales).
 * For every row of W (rows x n, WR_BF16 or WR_F32, ld ldw) independently and
 * the columns in natural order: at the start of each block of `group`
 * columns the scale is fp16_rne(max |w~| / L) of the block's current
 * feedback-updated values; each weight is rounded to the nearest level and
 * its error is pushed onto the later columns in the proportions set by the
 * damped H (n x n fp32, ld ldh, symmetric positive definite).
 * bits: device uint8 per row (2, 3 or 4).  n % group == 0, group % 8 == 0,
 * lazy_batch % group == 0; the library implements group in {32, 64, 128} and
 * lazy_batch = 128 (other valid values return WR_EUNSUPPORTED).
 * Outputs: codes (rows x n uint8, ld n), scales (rows x n/group fp16 bit
 * patterns).  dev_info as above.  Workspace: WR_OP_GPTQ.
 */
int wr_gptq_sweep(wr_ctx* ctx, const void* W, int w_dtype, int64_t rows, int64_t n, int64_t ldw,
                  const float* H, int64_t ldh, const uint8_t* bits, int32_t group, int32_t lazy_batch,
                  uint8_t* codes, uint16_t* scales, int32_t* dev_info);

/*
 * (d) Joint scales and the wring (Wringer model cards, "Recipe" and "Why the
 * solver changed"; Wringer news article, second paragraph; Agents-A1 card,
 * "Honest caveats": scales projected to fp16 at solve time).
 *
 * Target T (rows x n): `target` (WR_F32/WR_BF16, ld ldt) if non-null, else
 * dequant(codes, scales); plus (alpha / rank) * B A when B (rows x rank) and
 * A (rank x n) are both non-null (dtype ab_dtype, contiguous).
 * With WR_RECODE_NEAREST the codes are first replaced by the nearest level of
 * T / s on the current scales s (the v0.3 finisher of the Qwen3-4B card).  With
 * WR_RECODE_GPTQ (the v0.2 finisher: "GPTQ codes + joint scales", same card,
 * "Why the solver changed"; the Agents-A1 card's finisher) codes and scales
 * are first replaced by those of the GPTQ sweep of T with H (as wr_gptq_sweep,
 * lazy batch 128; n % 4 == 0), whose scales then serve as s0; a failure of the
 * sweep is reported in dev_info and leaves codes and scales as the sweep does.
 * With WR_RECODE_SEARCH (the finisher "nearest-point codes + block scale search" of
 * the same comparison) each block's scale is searched instead of solved: candidates
 * s_k = fp16((1 - k/64) max|t| / L), k = 0..31, each with the nearest codes of t / s_k;
 * the candidate with the least squared error of the block is kept (the smaller k on a
 * tie) and no joint solve follows (H and lambda are unused; H may be null).
 * At most one of the three flags.  Otherwise every row's scales are re-solved:
 *   s = argmin (t - Q s)^T H (t - Q s) + lambda mu ||s - s0||^2,
 *   mu = trace(Q^T H Q) / nb,  s0 = the scales passed in,
 * and projected to fp16 (round to nearest even).  codes and scales are
 * in/out.  H: damped, n x n fp32 (ld ldh).  Workspace: WR_OP_WRING, or
 * WR_OP_WRING_GPTQ with WR_RECODE_GPTQ.
 */
int wr_wring_solve(wr_ctx* ctx, const void* target, int t_dtype, int64_t ldt,
                   const void* B, const void* A, int32_t rank, float alpha, int ab_dtype,
                   const float* H, int64_t ldh, int64_t rows, int64_t n, const uint8_t* bits,
                   int32_t group, float lambda, int flags,
                   uint8_t* codes, uint16_t* scales, int32_t* dev_info);

/*
 * (e) Packing (Wringer model cards, "What is in this repo": packed codes plus
 * fp16 block scales).  Layout: per row, code j occupies bits [j b, (j+1) b)
 * of the row's bit stream, LSB first in little-endian bytes (a row is
 * n b / 8 bytes, so n * bits % 8 == 0); then the fp16 scales, little-endian,
 * row-major [rows][n / group].  out_bytes must equal
 * rows * n * bits / 8 + 2 * rows * (n / group).
 */
int wr_pack(wr_ctx* ctx, const uint8_t* codes, const uint16_t* scales, int64_t rows, int64_t n,
            int32_t bits, int32_t group, uint8_t* out, size_t out_bytes);

/* Inverse of wr_pack.  Each of codes, scales, dequant_bf16 (rows x n bf16 of
 * (2c - L) s, round to nearest even) may be null. */
int wr_unpack(wr_ctx* ctx, const uint8_t* in, size_t in_bytes, int64_t rows, int64_t n, int32_t bits,
              int32_t group, uint8_t* codes, uint16_t* scales, uint16_t* dequant_bf16);

/*
 * (f) Materialize (Wringer model cards, "What is in this repo": the materializer turns
 * the container into the fake-quant bf16 checkpoint that inference loads; "Honest
 * caveats": materializing at ledger precision).
 * For one packed module (wr_pack layout: rows x n_store codes of `bits` bits, fp16 scales
 * per `group`), writes out (rows x n_out bf16 bit patterns, leading dimension ldo):
 *   out[r][j] = bf16_RNE( (R^T v_r)_j ),  v_r = the dequantized row (2 c - L) s,  j < n_out,
 * where R is the rotation of wr_hadamard_rotate with had_block and signs (device int8, +-1,
 * length n_store); had_block 0 means R = I (signs may be null).  The dequantized values are
 * exact in fp32, R^T is applied in fp32 and each weight is rounded to bf16 once; the last
 * n_store - n_out columns (the zero padding of the input dim) are dropped.
 * n_out <= n_store, ldo >= n_out, n_store % 8 == 0; with a rotation had_block is a power of
 * two in 2..4096 dividing n_store.  in_bytes must equal the wr_pack size.  No workspace.
 */
int wr_materialize(wr_ctx* ctx, const uint8_t* in, size_t in_bytes, int64_t rows, int64_t n_store, int32_t bits,
                   int32_t group, int32_t had_block, const int8_t* signs, int64_t n_out, uint16_t* out, int64_t ldo);

/*
 * (f) Trellis-coded quantization with a Viterbi search (Pingala-8 post, "Trick 3: trellis
 * coding": a state carried from step to step selects the coset of values a step may use, the
 * bits written pick the value and the next state, and the Viterbi algorithm finds the
 * cheapest path).  One weight per step on a shift-register trellis of S = 2^log2_states
 * states (1 <= log2_states <= 4): branch bit u leads from state s to ((s << 1) | u) mod S
 * (the post's toy is S = 2, where the bit written becomes the next state); branch (s, u)
 * carries the coset values[(s * 2 + u) * coset_size + v], v < coset_size (1, 2 or 4),
 * fp32, device memory.  For each row of T (rows x n fp32, ld ldt, a multiple of 4, T
 * 16-byte aligned), starting in start_state, finds the path minimising the sum of squared
 * errors (per step the nearest value of the branch's coset); ties go to the smaller
 * predecessor state, the smaller end state, the smaller coset index.  Writes codes (rows x n
 * uint8, ld ldc: u | v << 1), optionally recon (rows x n fp32, ld ldr: the decoded values)
 * and cost (rows fp64: the path's sum of squared errors, summed in fp64).  The search runs in
 * fp32 with the costs renormalised every 16 steps; targets must be finite.
 * Workspace: WR_OP_TRELLIS (rows, n, group = S).
 */
int wr_trellis_quantize(wr_ctx* ctx, const float* T, int64_t ldt, int64_t rows, int64_t n, int32_t log2_states,
                        int32_t coset_size, const float* values, int32_t start_state, uint8_t* codes, int64_t ldc,
                        float* recon, int64_t ldr, double* cost);

/*
 * (f) Product of a packed module with input vectors (Wringer model cards, "What is in this
 * repo": the container of packed codes and fp16 block scales, stored in the rotated and
 * zero-padded basis; the cards name the multiplication of packed codes with the activations
 * as what decoding from the container needs).  For the module in `in` (wr_pack layout,
 * in_bytes its size; rows x n_store codes of `bits` bits, group a multiple of 32, n_store a
 * multiple of 32, `in` 16-byte aligned) and batch input vectors x (batch x n_in fp32, ld ldx,
 * n_in <= n_store, 1 <= batch <= 8):
 *   y[b][r] = sum_j (2 c_rj - L) s_r,j/group (R x_pad)_j
 * with x_pad the vector zero-padded to n_store and R the rotation of wr_hadamard_rotate
 * (had_block, signs: device int8 +-1 of length n_store; had_block 0: R = I), i.e. the
 * module's weights in the input basis times x.  x' = R x_pad is formed in fp32 in the
 * workspace, the products and sums run in fp32.  y: batch x rows fp32, ld ldy >= rows.
 * Workspace: WR_OP_GEMV (rows = batch, n = n_store).
 */
int wr_packed_gemv(wr_ctx* ctx, const uint8_t* in, size_t in_bytes, int64_t rows, int64_t n_store, int32_t bits,
                   int32_t group, int32_t had_block, const int8_t* signs, const float* x, int64_t n_in, int64_t ldx,
                   int32_t batch, float* y, int64_t ldy);

/*
 * Measures of a quantized module (Wringer Qwen3-4B model card, "Why the solver changed": the
 * relative Frobenius distance of weights to their nearest representation on the joint-scale grid,
 * and the share of codes on which the GPTQ and nearest-point solvers disagree; Agents-A1 model
 * card, "Honest caveats": the share of bf16 weights that projecting the scales to fp16 at solve
 * time moves by one ulp).  Off the solve's own path; three calls serve them:
 *
 * wr_set_scale_trace: when raw is non-null, every later joint scale solve on this context (the
 * joint solve of wr_wring_solve, with or without a recode; not WR_RECODE_SEARCH, which solves
 * none) also writes each row's solution before the fp16 projection, as fp32, to raw (rows x n/group
 * of that call, row-major); capacity (elements) smaller than a call's rows * n/group makes that
 * call return WR_EINVAL before launching anything.  raw = null stops it.
 */
int wr_set_scale_trace(wr_ctx* ctx, float* raw, int64_t capacity);

/*
 * wr_wring_target: the watered target alone, T_out (rows x n fp32, contiguous) = target (dtype
 * t_dtype, ld ldt) or, when target is null, dequant(codes, scales), plus (alpha / rank) B A when B and
 * A are non-null -- exactly the target wr_wring_solve forms.  codes and scales are read only.
 * dev_info: 0, or -1 for a non-finite value.  Workspace: WR_OP_WRING (rows, n, group, rank).
 */
int wr_wring_target(wr_ctx* ctx, const void* target, int t_dtype, int64_t ldt, const void* B, const void* A,
                    int32_t rank, float alpha, int ab_dtype, int64_t rows, int64_t n, const uint8_t* bits,
                    int32_t group, const uint8_t* codes, const uint16_t* scales, float* T_out, int32_t* dev_info);

/*
 * wr_quant_stats: sums over the module (rows x n codes of per-row `bits`, fp16 scales per `group`),
 * in fp64 and a fixed order (deterministic), written to out (device, 4 doubles):
 *   out[0] = sum (t - (2c - L) s)^2 and out[1] = sum t^2 over T (rows x n fp32, ld ldt), or 0 when
 *            T is null (the distance to the grid is sqrt(out[0] / out[1]));
 *   out[2] = the number of codes different from codes_ref (rows x n uint8), or 0 when null;
 *   out[3] = the number of weights whose bf16 rounding (nearest, ties to even) of (2c - L) s differs
 *            from that of (2c - L) s_raw, s_raw the unprojected fp32 scales (rows x n/group, as
 *            wr_set_scale_trace writes them), or 0 when null.
 * Workspace: WR_OP_STATS (rows).
 */
int wr_quant_stats(wr_ctx* ctx, const float* T, int64_t ldt, const uint8_t* codes, const uint16_t* scales,
                   const uint8_t* bits, int64_t rows, int64_t n, int32_t group, const uint8_t* codes_ref,
                   const float* scales_raw, double* out);

/* Static description of a status code. */
const char* wr_strerror(int status);

#ifdef __cplusplus
}
#endif
#endif /* WRINGER_H */
