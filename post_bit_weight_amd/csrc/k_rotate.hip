// Random-sign Hadamard rotation R = blockdiag_k(H_m diag(d_k)) / sqrt(m).
//
// For orthogonal R, W x = (W R^T)(R x): the weights are stored rotated and the
// inputs rotated the same way (Pingala-8 post, "Trick 1: rotate the weights
// first"); H_m is the natural-order Hadamard matrix printed there for m = 4.
// One workgroup transforms one length-m segment of one row in LDS with log2(m)
// butterfly stages (the in-place fast Walsh-Hadamard transform produces the
// natural ordering).  The two-sided form R H R^T runs the row pass, an in-place
// transpose and the row pass again.
#include "common.hpp"

namespace wr {

constexpr int ROT_THREADS = 256;

__global__ __launch_bounds__(ROT_THREADS) void fwht_rows_kernel(float* __restrict__ M, int64_t ld, int m, int log2m,
                                                                const int8_t* __restrict__ signs, int inverse,
                                                                float scale) {
  extern __shared__ float buf[];
  const int64_t row = blockIdx.y;
  const int64_t col0 = (int64_t)blockIdx.x * m;
  float* p = M + row * ld + col0;
  const int8_t* d = signs + col0;
  for (int i = threadIdx.x; i < m; i += ROT_THREADS) buf[i] = inverse ? p[i] : p[i] * (float)d[i];
  __syncthreads();
  for (int s = 0; s < log2m; ++s) {
    const int h = 1 << s;
    for (int q = threadIdx.x; q < (m >> 1); q += ROT_THREADS) {
      const int i = ((q >> s) << (s + 1)) | (q & (h - 1));
      const float a = buf[i], b = buf[i + h];
      buf[i] = a + b;
      buf[i + h] = a - b;
    }
    __syncthreads();
  }
  for (int i = threadIdx.x; i < m; i += ROT_THREADS) p[i] = inverse ? buf[i] * scale * (float)d[i] : buf[i] * scale;
}

// In-place transpose of a square n x n matrix: the workgroup for tile pair (I, J), I <= J, swaps them.
constexpr int TR_T = 32;
__global__ void transpose_inplace_kernel(float* __restrict__ M, int64_t n, int64_t ld, int ntile) {
  __shared__ float a[TR_T][TR_T + 1];
  __shared__ float b[TR_T][TR_T + 1];
  int t = blockIdx.x, I = 0;
  while (t >= ntile - I) {
    t -= ntile - I;
    ++I;
  }
  const int J = I + t;
  const int tx = threadIdx.x & (TR_T - 1), ty = threadIdx.x / TR_T;  // 256 threads: ty in [0, 8)
  for (int r = ty; r < TR_T; r += 8) {
    const int64_t i = (int64_t)I * TR_T + r, j = (int64_t)J * TR_T + tx;
    a[r][tx] = (i < n && j < n) ? M[i * ld + j] : 0.0f;
    const int64_t i2 = (int64_t)J * TR_T + r, j2 = (int64_t)I * TR_T + tx;
    b[r][tx] = (i2 < n && j2 < n) ? M[i2 * ld + j2] : 0.0f;
  }
  __syncthreads();
  for (int r = ty; r < TR_T; r += 8) {
    const int64_t i = (int64_t)I * TR_T + r, j = (int64_t)J * TR_T + tx;
    if (i < n && j < n) M[i * ld + j] = b[tx][r];
    const int64_t i2 = (int64_t)J * TR_T + r, j2 = (int64_t)I * TR_T + tx;
    if (i2 < n && j2 < n) M[i2 * ld + j2] = a[tx][r];
  }
}

}  // namespace wr

using namespace wr;

static int launch_rows(wr_ctx* ctx, float* M, int64_t rows, int64_t n, int64_t ld, int m, const int8_t* signs,
                       int inverse) {
  int log2m = 0;
  while ((1 << log2m) < m) ++log2m;
  const float scale = 1.0f / std::sqrt((float)m);
  dim3 grid((unsigned)(n / m), (unsigned)rows);
  hipLaunchKernelGGL(fwht_rows_kernel, grid, dim3(ROT_THREADS), (size_t)m * sizeof(float), ctx->stream, M, ld, m,
                     log2m, signs, inverse, scale);
  WR_CHECK_LAUNCH();
  return WR_OK;
}

int wr_hadamard_rotate_impl(wr_ctx* ctx, float* M, int64_t rows, int64_t n, int64_t ld, int32_t m,
                            const int8_t* signs, int mode) {
  if (mode == WR_ROT_ROWS || mode == WR_ROT_ROWS_INVERSE) return launch_rows(ctx, M, rows, n, ld, m, signs, mode);
  // R M R^T = rows( (rows(M))^T ) for symmetric M; for general square M the
  // column pass is the row pass of the transpose, transposed back.
  int rc = launch_rows(ctx, M, n, n, ld, m, signs, 0);  // M R^T
  if (rc) return rc;
  const int ntile = (int)((n + TR_T - 1) / TR_T);
  const unsigned pairs = (unsigned)(ntile * (ntile + 1) / 2);
  hipLaunchKernelGGL(transpose_inplace_kernel, dim3(pairs), dim3(256), 0, ctx->stream, M, n, ld, ntile);
  WR_CHECK_LAUNCH();
  rc = launch_rows(ctx, M, n, n, ld, m, signs, 0);       // (M R^T)^T R^T = R M^T R^T
  if (rc) return rc;
  hipLaunchKernelGGL(transpose_inplace_kernel, dim3(pairs), dim3(256), 0, ctx->stream, M, n, ld, ntile);
  WR_CHECK_LAUNCH();
  return WR_OK;                                          // (R M^T R^T)^T = R M R^T
}
