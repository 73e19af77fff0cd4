// GPTQ / LDLQ error-feedback sweep (Pingala-8 post, "Trick 2: round with error
// feedback"; Wringer model cards, "Recipe": GPTQ codes on a fixed signed grid
// with fp16 block scales).
//
// Factorisation.  With J the reversal permutation, L = chol_lower(J H J) gives
// H = V V^T with V = J L J upper triangular, and H = M D M^T with the unit upper
// M = V diag(V)^-1.  The sweep needs only M: no triangular inverse.  The
// Cholesky runs in fp64, blocked by 32: per block column one single-wave kernel
// factors the diagonal block in registers, then one kernel solves the panel
// and updates the trailing lower matrix on the fp64 matrix cores; M is rounded
// to fp32 once.  (An fp32 factorisation moves GPTQ block scales by up to two fp16 ulps
// against an fp64 reference; fp64 keeps them within one.)
//
// Sweep (LDLQ pull form).  Every row is independent.  With delta_i = w_i - q_i,
// column k is rounded from v_k = w_k + sum_{i<k} M_ik delta_i.  The corrections
// C_k = sum_{i<k} M_ik delta_i are kept in a rows x n buffer: inside a lazy
// batch of columns they are updated one column at a time, and when a batch is
// done the remaining columns receive C += E M[batch, rest] as one GEMM.
// The block scale is fixed at the first column of a block from the values the
// GPTQ push form holds there, w_j + x_j with x = M_bb^-T C_b (M_bb the block's
// diagonal block of M): the optimal compensation of everything rounded so far.
// In exact arithmetic this gives the same codes and scales as the push form.
//
// Threads: P lanes share one row; lane p owns the batch columns p, p+P, ...
// The owner of column k rounds it and the error is broadcast within the
// P-lane group; every lane then updates its own columns from M's row k, which
// is staged in LDS in a lane-major order.
#include "common.hpp"

int wr_gemm_f32(hipStream_t st, int M, int N, int K, const float* A, int64_t lda, const float* B, int64_t ldb,
                bool b_kn, float* C, int64_t ldc, float alpha, bool accumulate, bool lower_tiles,
                const int32_t* dev_info);

namespace wr {

constexpr int CH_NB = 32;

// 1/sqrt(d) to fp64 precision: fp32 estimate and two Newton steps.
__device__ __forceinline__ double rsqrt_f64(double d) {
  double r = (double)rsqrtf((float)d);
  r = r * (1.5 - 0.5 * d * r * r);
  r = r * (1.5 - 0.5 * d * r * r);
  return r;
}

__device__ __forceinline__ double lane_bcast(double v, int lane) {
  const int64_t u = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane((int)(u & 0xffffffff), lane);
  const int hi = __builtin_amdgcn_readlane((int)(u >> 32), lane);
  return __longlong_as_double(((int64_t)hi << 32) | (uint32_t)lo);
}

// Triangular solve x L_kk^T = b for one panel row per lane (x overwrites b);
// Lt[j][i] = L_ij (staged in LDS), rinv[j] = 1 / L_jj.
template <int NB>
__device__ __forceinline__ void panel_solve(double (&b)[NB], const double (*Lt)[NB + 1], const double* rinv) {
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    b[j] *= rinv[j];
#pragma unroll
    for (int jj = j + 1; jj < NB; ++jj) b[jj] = fma(-b[j], Lt[j][jj], b[jj]);
  }
}


// A = J H J (lower triangle only), widened to fp64.
__global__ void reverse_copy_kernel(const float* __restrict__ H, int64_t ldh, int n, double* __restrict__ A) {
  const int i = blockIdx.x;
  for (int j = threadIdx.x; j <= i; j += blockDim.x)
    A[(int64_t)i * n + j] = (double)H[(int64_t)(n - 1 - i) * ldh + (n - 1 - j)];
}

typedef double f64x4 __attribute__((ext_vector_type(4)));

// Trailing update of one step, fused with the panel solve.  Tile (i, j) of the
// lower trailing matrix (rows/cols from kb + NB on, 64 x 64 per workgroup):
// waves 0-1 solve the 64 panel rows of block i against L_kk, waves 2-3 those
// of block j (the panel itself is read from A, which this step does not
// modify there); the diagonal tile's workgroup stores its solved rows into
// Lout.  Then A[i][j] -= P_i P_j^T on the fp64 matrix cores
// (v_mfma_f64_16x16x4f64: operand lane l holds row/column l % 16 at k = l / 16;
// accumulator v of lane l is row l / 16 + 4 v, column l % 16).
__global__ __launch_bounds__(256) void panel_update_kernel(double* __restrict__ A, double* __restrict__ Lout, int n,
                                                           int kb, const int32_t* __restrict__ dev_info) {
  if (*dev_info != 0) return;
  __shared__ double sp[2][CH_NB][64 + 1];  // solved panel blocks, k-major
  __shared__ double Lt[CH_NB][CH_NB + 1];  // L_kk transposed
  __shared__ double rinv[CH_NB];
  int ti, tj;
  {
    const int t = blockIdx.x;
    int i = (int)((sqrtf(8.0f * (float)t + 1.0f) - 1.0f) * 0.5f);
    while (i * (i + 1) / 2 > t) --i;
    while ((i + 1) * (i + 2) / 2 <= t) ++i;
    ti = i;
    tj = t - i * (i + 1) / 2;
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int base = kb + CH_NB;  // first trailing row/column
  for (int e = tid; e < CH_NB * CH_NB; e += 256) {
    const int i = e / CH_NB, j = e % CH_NB;
    const double v = Lout[(int64_t)(kb + i) * n + kb + j];
    Lt[j][i] = v;
    if (i == j) rinv[i] = 1.0 / v;
  }
  __syncthreads();
  {
    const int side = wave >> 1;  // 0: block i, 1: block j
    const int blk = side == 0 ? ti : tj;
    const int rloc = 32 * (wave & 1) + (lane & 31);
    const int64_t prow = (int64_t)base + blk * 64 + rloc;
    if (lane < 32 && (side == 0 || ti != tj)) {
      double b[CH_NB];
#pragma unroll
      for (int j = 0; j < CH_NB; ++j) b[j] = prow < n ? A[prow * n + kb + j] : 0.0;
      panel_solve<CH_NB>(b, Lt, rinv);
#pragma unroll
      for (int j = 0; j < CH_NB; ++j) sp[side][j][rloc] = b[j];
      if (side == 0 && ti == tj && prow < n) {
#pragma unroll
        for (int j = 0; j < CH_NB; ++j) Lout[prow * n + kb + j] = b[j];
      }
    }
  }
  __syncthreads();
  const int wi = wave >> 1, wj = wave & 1;
  const int sj = ti == tj ? 0 : 1;
  f64x4 acc[2][2];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y) acc[x][y] = f64x4{0.0, 0.0, 0.0, 0.0};
  const int li = lane & 15, lk = lane >> 4;
#pragma unroll
  for (int k0 = 0; k0 < CH_NB; k0 += 4) {
    double a[2], b[2];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      a[x] = sp[0][k0 + lk][32 * wi + 16 * x + li];
      b[x] = sp[sj][k0 + lk][32 * wj + 16 * x + li];
    }
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int y = 0; y < 2; ++y) acc[x][y] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[x], b[y], acc[x][y], 0, 0, 0);
  }
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int gi = base + ti * 64 + 32 * wi + 16 * x + (lane >> 4) + 4 * v;
        const int gj = base + tj * 64 + 32 * wj + 16 * y + (lane & 15);
        if (gi < n && gj < n && gj <= gi) A[(int64_t)gi * n + gj] -= acc[x][y][v];
      }
}


// Factor the NB x NB diagonal block at kb of the (updated) matrix A in fp64 and
// write L_kk into Lout; one wave, lane i holds row i in registers and column k
// is broadcast with readlane.
template <int NB>
__global__ __launch_bounds__(64) void chol_diag_kernel(const double* __restrict__ A, double* __restrict__ Lout, int n,
                                                       int kb, int32_t* __restrict__ dev_info) {
  if (*dev_info != 0) return;
  const int lane = threadIdx.x;
  const int r = lane < NB ? lane : NB - 1;
  const int row = kb + r;
  double a[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j)
    a[j] = (row < n && kb + j < n && j <= r) ? A[(int64_t)row * n + kb + j] : (j == r ? 1.0 : 0.0);
  int bad = -1;
#pragma unroll
  for (int k = 0; k < NB; ++k) {
    const double d = lane_bcast(a[k], k);
    if (!(d > 0.0) && bad < 0) bad = k;
    const double l = a[k] * rsqrt_f64(d);  // lane k: L_kk; lanes below: L_ik
    a[k] = l;
#pragma unroll
    for (int j = k + 1; j < NB; ++j) a[j] = fma(-l, lane_bcast(l, j), a[j]);
  }
  if (bad >= 0) {
    if (lane == 0) atomicCAS(dev_info, 0, kb + bad + 1);
    return;
  }
  if (lane < NB && row < n) {
#pragma unroll
    for (int j = 0; j < NB; ++j) Lout[(int64_t)row * n + kb + j] = j <= lane ? a[j] : 0.0;
  }
}

// M[i][j] = L[n-1-i][n-1-j] / L[n-1-j][n-1-j] for i < j; 0 on and below the diagonal
// (the unit diagonal is implicit and never used).
__global__ void build_m_kernel(const double* __restrict__ A, int n, float* __restrict__ M,
                               const int32_t* __restrict__ dev_info) {
  if (*dev_info != 0) return;
  const int i = blockIdx.x;
  const int64_t ri = n - 1 - i;
  for (int j = threadIdx.x; j < n; j += blockDim.x) {
    float v = 0.0f;
    if (j > i) {
      const int64_t rj = n - 1 - j;
      v = (float)(A[ri * n + rj] / A[rj * n + rj]);
    }
    M[(int64_t)i * n + j] = v;
  }
}

__global__ void check_finite_kernel(const void* __restrict__ W, int w_dtype, int64_t rows, int n, int64_t ldw,
                                    int32_t* __restrict__ dev_info) {
  const int64_t r = blockIdx.x;
  bool bad = false;
  for (int j = threadIdx.x; j < n; j += blockDim.x) {
    float v = w_dtype == WR_BF16 ? bf16_bits_to_f32(static_cast<const uint16_t*>(W)[r * ldw + j])
                                 : static_cast<const float*>(W)[r * ldw + j];
    bad |= !(fabsf(v) <= 3.0e38f);
  }
  if (__syncthreads_or(bad) && threadIdx.x == 0) atomicCAS(dev_info, 0, -1);
}

__global__ void sweep_set_int_kernel(int32_t* p, int32_t v) { *p = v; }

__global__ void zero_f32_kernel(float* __restrict__ p, int64_t count) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0.0f;
}

template <int P>
__device__ __forceinline__ float group_bcast(float v, int src) {
  return __shfl(v, src, P);
}

template <int P>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int o = P / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, P));
  return v;
}

// One lazy batch of BATCH columns starting at b0 (ncols <= BATCH valid columns).
template <int P, int BATCH, int G>
__global__ __launch_bounds__(256) void sweep_panel_kernel(const void* __restrict__ W, int w_dtype, int64_t rows,
                                                          int n, int64_t ldw, const float* __restrict__ M,
                                                          const uint8_t* __restrict__ bits, int b0, int ncols,
                                                          float* __restrict__ Cbuf, float* __restrict__ E,
                                                          uint8_t* __restrict__ codes, uint16_t* __restrict__ scales,
                                                          const int32_t* __restrict__ dev_info) {
  constexpr int S = BATCH / P;       // columns per lane
  constexpr int NBLK = BATCH / G;    // blocks per batch
  constexpr int SB = G / P;          // columns per lane per block
  __shared__ __attribute__((aligned(16))) float Ms[BATCH * BATCH];  // [k][p][slot]
  if (*dev_info != 0) return;
  const int tid = threadIdx.x;
  const int p = tid % P;
  const int64_t row = (int64_t)blockIdx.x * (256 / P) + tid / P;
  const bool active = row < rows;

  for (int e = tid; e < BATCH * BATCH; e += 256) {
    const int k = e / BATCH, j = e % BATCH;
    const float v = (k < ncols && j < ncols) ? M[(int64_t)(b0 + k) * n + b0 + j] : 0.0f;
    Ms[k * BATCH + (j % P) * S + j / P] = v;
  }

  float w[S], c[S], d[S];
  uint8_t code[S];
  float sc[NBLK];
  const int L = active ? (1 << bits[row]) - 1 : 3;
#pragma unroll
  for (int i = 0; i < S; ++i) {
    const int col = p + P * i;
    w[i] = 0.0f;
    c[i] = 0.0f;
    d[i] = 0.0f;
    code[i] = 0;
    if (active && col < ncols) {
      const int64_t gc = b0 + col;
      w[i] = w_dtype == WR_BF16 ? bf16_bits_to_f32(static_cast<const uint16_t*>(W)[row * ldw + gc])
                                : static_cast<const float*>(W)[row * ldw + gc];
      c[i] = Cbuf[row * n + gc];
    }
  }
  __syncthreads();

#pragma unroll
  for (int blk = 0; blk < NBLK; ++blk) {
    sc[blk] = 0.0f;
    if (blk * G >= ncols) continue;  // uniform
    // push-form values at the block start: x = M_bb^-T c_b
    float x[SB];
#pragma unroll
    for (int q = 0; q < SB; ++q) x[q] = c[blk * SB + q];
#pragma unroll
    for (int jj = 0; jj < G; ++jj) {
      const int j = blk * G + jj;
      const int owner = j % P, qo = jj / P;
      const float xj = group_bcast<P>(x[qo], owner);
      const float* mrow = &Ms[j * BATCH + p * S + blk * SB];
#pragma unroll
      for (int q = qo; q < SB; ++q) x[q] = fmaf(-mrow[q], xj, x[q]);
    }
    float m = 0.0f;
#pragma unroll
    for (int q = 0; q < SB; ++q) m = fmaxf(m, fabsf(w[blk * SB + q] + x[q]));
    m = group_max<P>(m);
    const float s = f16_bits_to_f32(f32_to_f16_bits_clamped(m / (float)L));
    sc[blk] = s;
    const float inv_s = s > 0.0f ? 1.0f / s : 0.0f;
    // round the block's columns one at a time, pushing each error to the later batch columns
#pragma unroll
    for (int jj = 0; jj < G; ++jj) {
      const int j = blk * G + jj;
      const int owner = j % P, io = j / P;
      const float v = w[io] + c[io];
      const int cd = nearest_code(v * inv_s, L);
      const float dl = w[io] - (float)(2 * cd - L) * s;
      if (p == owner) {
        code[io] = (uint8_t)cd;
        d[io] = dl;
      }
      const float dj = group_bcast<P>(dl, owner);
      const float* mrow = &Ms[j * BATCH + p * S];
#pragma unroll
      for (int i = io; i < S; ++i) c[i] = fmaf(mrow[i], dj, c[i]);
    }
  }

  if (!active) return;
#pragma unroll
  for (int i = 0; i < S; ++i) {
    const int col = p + P * i;
    if (col < ncols) {
      codes[row * n + b0 + col] = code[i];
      E[row * BATCH + col] = d[i];
    }
  }
  if (p == 0) {
#pragma unroll
    for (int blk = 0; blk < NBLK; ++blk)
      if (blk * G < ncols) scales[row * (n / G) + (b0 / G) + blk] = f32_to_f16_bits_clamped(sc[blk]);
  }
}

}  // namespace wr

using namespace wr;

static constexpr int kBatch = 128;

size_t wr_gptq_ws_bytes(int64_t rows, int64_t n) {
  size_t b = 0;
  b += (size_t)n * n * 8;          // A (J H J, reduced step by step), fp64
  b += (size_t)n * n * 8;          // L, fp64
  b += (size_t)n * n * 4;          // M
  b += (size_t)rows * n * 4;       // corrections C
  b += (size_t)rows * kBatch * 4;  // batch errors E
  return b + 1024;
}

// Blocked fp64 Cholesky of J H J: A holds the matrix being reduced, L collects
// the factor; then M rounded to fp32.
static int factor_m(wr_ctx* ctx, const float* H, int64_t ldh, int n, double* A, double* L, float* Mm,
                    int32_t* dev_info) {
  hipStream_t st = ctx->stream;
  hipLaunchKernelGGL(reverse_copy_kernel, dim3(n), dim3(256), 0, st, H, ldh, n, A);
  WR_CHECK_LAUNCH();
  for (int kb = 0; kb < n; kb += CH_NB) {
    hipLaunchKernelGGL(chol_diag_kernel<CH_NB>, dim3(1), dim3(64), 0, st, A, L, n, kb, dev_info);
    WR_CHECK_LAUNCH();
    const int rem = n - kb - CH_NB;
    if (rem <= 0) break;
    const int nt = (rem + 63) / 64;
    hipLaunchKernelGGL(panel_update_kernel, dim3((unsigned)(nt * (nt + 1) / 2)), dim3(256), 0, st, A, L, n, kb,
                       dev_info);
    WR_CHECK_LAUNCH();
  }
  hipLaunchKernelGGL(build_m_kernel, dim3(n), dim3(256), 0, st, L, n, Mm, dev_info);
  WR_CHECK_LAUNCH();
  return WR_OK;
}

template <int P, int G>
static void launch_panel(hipStream_t st, const void* W, int w_dtype, int64_t rows, int n, int64_t ldw, const float* Mm,
                         const uint8_t* bits, int b0, int ncols, float* Cb, float* E, uint8_t* codes, uint16_t* scales,
                         const int32_t* dev_info) {
  const unsigned grid = (unsigned)((rows + (256 / P) - 1) / (256 / P));
  hipLaunchKernelGGL((sweep_panel_kernel<P, kBatch, G>), dim3(grid), dim3(256), 0, st, W, w_dtype, rows, n, ldw, Mm,
                     bits, b0, ncols, Cb, E, codes, scales, dev_info);
}

template <int P>
static int launch_panel_g(hipStream_t st, int G, const void* W, int w_dtype, int64_t rows, int n, int64_t ldw,
                          const float* Mm, const uint8_t* bits, int b0, int ncols, float* Cb, float* E, uint8_t* codes,
                          uint16_t* scales, const int32_t* dev_info) {
  switch (G) {
    case 32: launch_panel<P, 32>(st, W, w_dtype, rows, n, ldw, Mm, bits, b0, ncols, Cb, E, codes, scales, dev_info); break;
    case 64: launch_panel<P, 64>(st, W, w_dtype, rows, n, ldw, Mm, bits, b0, ncols, Cb, E, codes, scales, dev_info); break;
    case 128: launch_panel<P, 128>(st, W, w_dtype, rows, n, ldw, Mm, bits, b0, ncols, Cb, E, codes, scales, dev_info); break;
    default: return WR_EUNSUPPORTED;
  }
  WR_CHECK_LAUNCH();
  return WR_OK;
}

int wr_gptq_sweep_impl(wr_ctx* ctx, const void* W, int w_dtype, int64_t rows, int64_t n64, int64_t ldw,
                       const float* H, int64_t ldh, const uint8_t* bits, int32_t group, int32_t lazy_batch,
                       uint8_t* codes, uint16_t* scales, int32_t* dev_info) {
  if (lazy_batch != kBatch || (group != 32 && group != 64 && group != 128)) return WR_EUNSUPPORTED;
  if (ctx->ws_bytes < wr_gptq_ws_bytes(rows, n64)) return WR_EWORKSPACE;
  const int n = (int)n64;
  hipStream_t st = ctx->stream;
  char* ws = static_cast<char*>(ctx->ws);
  double* A = reinterpret_cast<double*>(ws);
  double* Lf = A + (size_t)n * n;
  float* Mm = reinterpret_cast<float*>(Lf + (size_t)n * n);
  float* Cb = Mm + (size_t)n * n;
  float* E = Cb + (size_t)rows * n;

  hipLaunchKernelGGL(sweep_set_int_kernel, dim3(1), dim3(1), 0, st, dev_info, 0);
  WR_CHECK_LAUNCH();
  if (rows > 0) {
    hipLaunchKernelGGL(check_finite_kernel, dim3((unsigned)rows), dim3(256), 0, st, W, w_dtype, rows, n, ldw, dev_info);
    WR_CHECK_LAUNCH();
  }
  int rc = factor_m(ctx, H, ldh, n, A, Lf, Mm, dev_info);
  if (rc) return rc;
  if (rows == 0) return WR_OK;
  hipLaunchKernelGGL(zero_f32_kernel, dim3(1024), dim3(256), 0, st, Cb, (int64_t)rows * n);
  WR_CHECK_LAUNCH();
  for (int b0 = 0; b0 < n; b0 += kBatch) {
    const int ncols = std::min(kBatch, n - b0);
    rc = launch_panel_g<16>(st, group, W, w_dtype, rows, n, ldw, Mm, bits, b0, ncols, Cb, E, codes, scales, dev_info);
    if (rc) return rc;
    const int rest = n - b0 - ncols;
    if (rest > 0) {
      rc = wr_gemm_f32(st, (int)rows, rest, ncols, E, kBatch, Mm + (int64_t)b0 * n + b0 + ncols, n, true,
                       Cb + b0 + ncols, n, 1.0f, true, false, dev_info);
      if (rc) return rc;
    }
  }
  return WR_OK;
}
