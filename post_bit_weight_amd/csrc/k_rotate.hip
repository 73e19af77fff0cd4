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

template <typename T>
__global__ __launch_bounds__(ROT_THREADS) void fwht_rows_kernel(T* __restrict__ M, int64_t ld, int m, int log2m,
                                                                const int8_t* __restrict__ signs, int inverse,
                                                                T scale) {
  extern __shared__ __attribute__((aligned(16))) unsigned char rot_smem[];
  T* buf = reinterpret_cast<T*>(rot_smem);
  const int64_t row = blockIdx.y;
  const int64_t col0 = (int64_t)blockIdx.x * m;
  T* p = M + row * ld + col0;
  const int8_t* d = signs + col0;
  for (int i = threadIdx.x; i < m; i += ROT_THREADS) buf[i] = inverse ? p[i] : p[i] * (T)d[i];
  __syncthreads();
  for (int s = 0; s < log2m; ++s) {
    const int h = 1 << s;
    for (int q = threadIdx.x; q < (m >> 1); q += ROT_THREADS) {
      const int i = ((q >> s) << (s + 1)) | (q & (h - 1));
      const T a = buf[i], b = buf[i + h];
      buf[i] = a + b;
      buf[i + h] = a - b;
    }
    __syncthreads();
  }
  for (int i = threadIdx.x; i < m; i += ROT_THREADS) p[i] = inverse ? buf[i] * scale * (T)d[i] : buf[i] * scale;
}

// The same row transform for fp32 with m = 64 V (V = 2^LOGV values per lane): one wave per
// (row, segment), lane l holding elements V l .. V l + V - 1.  Stages with h < V pair values inside
// the lane; the others pair lane l with lane l ^ (h / V), the lower element becoming a + b and the
// upper a - b, so every element takes the same additions, in the same stage order, as in the LDS
// form above (bit-identical).  Loads and stores are V consecutive floats per lane (16-byte pieces
// from V = 4 up: rows 16-byte aligned).  Four waves per workgroup on consecutive segments.
template <int LOGV>
__global__ __launch_bounds__(256) void fwht_rows_reg_kernel(float* __restrict__ M, int64_t ld, int64_t rows,
                                                            int nseg, const int8_t* __restrict__ signs, int inverse,
                                                            float scale) {
  constexpr int V = 1 << LOGV, m = 64 * V;
  const int lane = threadIdx.x & 63;
  const int64_t g = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (g >= rows * nseg) return;
  const int64_t row = g / nseg;
  const int64_t col = (g - row * nseg) * m + (int64_t)V * lane;
  float* p = M + row * ld + col;
  const int8_t* d = signs + col;
  float x[V];
  if constexpr (V >= 4) {
#pragma unroll
    for (int k = 0; k < V; k += 4) {
      const float4 v = *reinterpret_cast<const float4*>(p + k);
      x[k] = v.x;
      x[k + 1] = v.y;
      x[k + 2] = v.z;
      x[k + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int k = 0; k < V; ++k) x[k] = p[k];
  }
  if (!inverse) {
#pragma unroll
    for (int k = 0; k < V; ++k) x[k] = x[k] * (float)d[k];
  }
#pragma unroll
  for (int h = 1; h < V; h <<= 1)
#pragma unroll
    for (int k = 0; k < V; ++k)
      if (!(k & h)) {
        const float a = x[k], b = x[k + h];
        x[k] = a + b;
        x[k + h] = a - b;
      }
#pragma unroll
  for (int lh = 1; lh < 64; lh <<= 1) {
    const bool upper = (lane & lh) != 0;
#pragma unroll
    for (int k = 0; k < V; ++k) {
      const float y = __shfl_xor(x[k], lh);
      x[k] = upper ? y - x[k] : x[k] + y;
    }
  }
#pragma unroll
  for (int k = 0; k < V; ++k) x[k] = inverse ? x[k] * scale * (float)d[k] : x[k] * scale;
  if constexpr (V >= 4) {
#pragma unroll
    for (int k = 0; k < V; k += 4) *reinterpret_cast<float4*>(p + k) = float4{x[k], x[k + 1], x[k + 2], x[k + 3]};
  } else {
#pragma unroll
    for (int k = 0; k < V; ++k) p[k] = x[k];
  }
}

// In-place transpose of a square n x n matrix: the workgroup for tile pair (I, J), I <= J, swaps them.
constexpr int TR_T = 32;
template <typename T>
__global__ void transpose_inplace_kernel(T* __restrict__ M, int64_t n, int64_t ld, int ntile) {
  __shared__ T a[TR_T][TR_T + 1];
  __shared__ T b[TR_T][TR_T + 1];
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

template <int LOGV>
static void launch_rows_reg(wr_ctx* ctx, float* M, int64_t rows, int64_t n, int64_t ld, const int8_t* signs,
                            int inverse, float scale) {
  const int nseg = (int)(n >> (6 + LOGV));
  const int64_t blocks = (rows * nseg + 3) / 4;
  hipLaunchKernelGGL(fwht_rows_reg_kernel<LOGV>, dim3((unsigned)blocks), dim3(256), 0, ctx->stream, M, ld, rows, nseg,
                     signs, inverse, scale);
}

template <typename T>
static int launch_rows(wr_ctx* ctx, T* M, int64_t rows, int64_t n, int64_t ld, int m, const int8_t* signs,
                       int inverse) {
  int log2m = 0;
  while ((1 << log2m) < m) ++log2m;
  const T scale = (T)1 / std::sqrt((T)m);
  if constexpr (sizeof(T) == 4) {
    // fp32 with 64 <= m <= 2048: the register form (16-byte rows for m >= 256)
    const bool aligned16 = (reinterpret_cast<uintptr_t>(M) % 16 == 0) && ld % 4 == 0;
    if (m >= 64 && m <= 2048 && (m < 256 || aligned16) && rows * (n / m) <= ((int64_t)1 << 33)) {
      switch (log2m) {
        case 6: launch_rows_reg<0>(ctx, M, rows, n, ld, signs, inverse, scale); break;
        case 7: launch_rows_reg<1>(ctx, M, rows, n, ld, signs, inverse, scale); break;
        case 8: launch_rows_reg<2>(ctx, M, rows, n, ld, signs, inverse, scale); break;
        case 9: launch_rows_reg<3>(ctx, M, rows, n, ld, signs, inverse, scale); break;
        case 10: launch_rows_reg<4>(ctx, M, rows, n, ld, signs, inverse, scale); break;
        default: launch_rows_reg<5>(ctx, M, rows, n, ld, signs, inverse, scale); break;
      }
      WR_CHECK_LAUNCH();
      return WR_OK;
    }
  }
  dim3 grid((unsigned)(n / m), (unsigned)rows);
  hipLaunchKernelGGL(fwht_rows_kernel<T>, grid, dim3(ROT_THREADS), (size_t)m * sizeof(T), ctx->stream, M, ld, m, log2m,
                     signs, inverse, scale);
  WR_CHECK_LAUNCH();
  return WR_OK;
}

// R M R^T for a square M: rows pass (M R^T), transpose, rows pass, transpose.
template <typename T>
static int rotate_sym(wr_ctx* ctx, T* M, int64_t n, int64_t ld, int m, const int8_t* signs) {
  const int ntile = (int)((n + TR_T - 1) / TR_T);
  const unsigned pairs = (unsigned)(ntile * (ntile + 1) / 2);
  for (int pass = 0; pass < 2; ++pass) {
    int rc = launch_rows<T>(ctx, M, n, n, ld, m, signs, 0);
    if (rc) return rc;
    hipLaunchKernelGGL(transpose_inplace_kernel<T>, dim3(pairs), dim3(256), 0, ctx->stream, M, n, ld, ntile);
    WR_CHECK_LAUNCH();
  }
  return WR_OK;
}

int wr_rotate_sym_f64(wr_ctx* ctx, double* M, int64_t n, int64_t ld, int32_t m, const int8_t* signs) {
  return rotate_sym<double>(ctx, M, n, ld, m, signs);
}

int wr_hadamard_rotate_impl(wr_ctx* ctx, float* M, int64_t rows, int64_t n, int64_t ld, int32_t m,
                            const int8_t* signs, int mode) {
  if (mode == WR_ROT_ROWS || mode == WR_ROT_ROWS_INVERSE) return launch_rows<float>(ctx, M, rows, n, ld, m, signs, mode);
  return rotate_sym<float>(ctx, M, n, ld, m, signs);
}
