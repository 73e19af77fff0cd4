// Measures of a quantized module (Wringer Qwen3-4B model card, "Why the solver changed": the
// relative Frobenius distance of weights to their nearest joint-scale grid representation, and
// the share of codes on which two solvers disagree; Agents-A1 model card, "Honest caveats": the
// share of materialized bf16 weights that the fp16 projection of the scales moves by one ulp).
//
// One workgroup per row sums, in fp64 and a fixed order:
//   [0] sum (t - (2c - L) s)^2   over the row (t the target, s the fp16 block scale),
//   [1] sum t^2,
//   [2] the number of codes that differ from a reference code matrix,
//   [3] the number of weights whose bf16 rounding of (2c - L) s differs between the fp16 scale and
//       the unprojected (fp32) solution of the scale solve;
// a second kernel adds the rows in index order.  Deterministic, no atomics.
#include "common.hpp"

namespace wr {

constexpr int QS_THREADS = 256;

__global__ __launch_bounds__(QS_THREADS) void quant_stats_rows_kernel(
    const float* __restrict__ T, int64_t ldt, const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales,
    const uint8_t* __restrict__ bits, int n, int group, const uint8_t* __restrict__ codes_ref,
    const float* __restrict__ raw, double* __restrict__ partial) {
  __shared__ double red[4][QS_THREADS];
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const int nb = n / group;
  const int L = (1 << bits[row]) - 1;
  double d2 = 0.0, t2 = 0.0, diff = 0.0, moved = 0.0;
  for (int j = tid; j < n; j += QS_THREADS) {
    const int c = codes[row * n + j];
    const double lev = (double)(2 * c - L);
    const double s = (double)f16_bits_to_f32(scales[row * nb + j / group]);
    const double q = lev * s;  // exact: an odd level below 16 times an 11-bit scale
    if (T) {
      const double t = (double)T[row * ldt + j];
      d2 += (t - q) * (t - q);
      t2 += t * t;
    }
    if (codes_ref && codes_ref[row * n + j] != c) diff += 1.0;
    if (raw && f64_to_bf16_bits(q) != f64_to_bf16_bits(lev * (double)raw[row * nb + j / group])) moved += 1.0;
  }
  red[0][tid] = d2;
  red[1][tid] = t2;
  red[2][tid] = diff;
  red[3][tid] = moved;
  __syncthreads();
  for (int w = QS_THREADS / 2; w > 0; w >>= 1) {
    if (tid < w)
#pragma unroll
      for (int k = 0; k < 4; ++k) red[k][tid] += red[k][tid + w];
    __syncthreads();
  }
  if (tid < 4) partial[row * 4 + tid] = red[tid][0];
}

__global__ __launch_bounds__(QS_THREADS) void quant_stats_sum_kernel(const double* __restrict__ partial, int64_t rows,
                                                                     double* __restrict__ out) {
  __shared__ double red[4][QS_THREADS];
  const int tid = threadIdx.x;
  double a[4] = {0.0, 0.0, 0.0, 0.0};
  for (int64_t r = tid; r < rows; r += QS_THREADS)
#pragma unroll
    for (int k = 0; k < 4; ++k) a[k] += partial[r * 4 + k];
#pragma unroll
  for (int k = 0; k < 4; ++k) red[k][tid] = a[k];
  __syncthreads();
  for (int w = QS_THREADS / 2; w > 0; w >>= 1) {
    if (tid < w)
#pragma unroll
      for (int k = 0; k < 4; ++k) red[k][tid] += red[k][tid + w];
    __syncthreads();
  }
  if (tid < 4) out[tid] = red[tid][0];
}

}  // namespace wr

using namespace wr;

size_t wr_stats_ws_bytes(int64_t rows) { return ((size_t)rows * 4 * sizeof(double) + 255) & ~(size_t)255; }

int wr_quant_stats_impl(wr_ctx* ctx, const float* T, int64_t ldt, const uint8_t* codes, const uint16_t* scales,
                        const uint8_t* bits, int64_t rows, int64_t n, int32_t group, const uint8_t* codes_ref,
                        const float* raw, double* out) {
  if (ctx->ws_bytes < wr_stats_ws_bytes(rows > 0 ? rows : 1)) return WR_EWORKSPACE;
  double* partial = static_cast<double*>(ctx->ws);
  if (rows > 0) {
    hipLaunchKernelGGL(quant_stats_rows_kernel, dim3((unsigned)rows), dim3(QS_THREADS), 0, ctx->stream, T, ldt, codes,
                       scales, bits, (int)n, group, codes_ref, raw, partial);
    WR_CHECK_LAUNCH();
  }
  hipLaunchKernelGGL(quant_stats_sum_kernel, dim3(1), dim3(QS_THREADS), 0, ctx->stream, partial, rows, out);
  WR_CHECK_LAUNCH();
  return WR_OK;
}
