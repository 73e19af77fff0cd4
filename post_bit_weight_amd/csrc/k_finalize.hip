// H = S/N + delta I from the lower triangle of S, optionally rotated two-sided:
// H = R pad(S/N) R^T + delta I.
//
// H is the average of x x^T over calibration inputs (Pingala-8 post, "Trick 2: round with error
// feedback"), rotated with the weights (same post, "Trick 1"); delta is the Tikhonov damping of the
// GPTQ solve (Wringer news article, second paragraph), delta = damp * trace(S/N) / n_store (the
// rotation is orthogonal, so the trace is taken before it).  The rotation runs in fp64 and H is
// rounded to fp32 once.
#include "common.hpp"

namespace wr {

// delta = damp * trace(S / N) / n_store, summed in a fixed order by one workgroup.
__global__ __launch_bounds__(1024) void trace_kernel(const double* __restrict__ S, int n, double inv_rows,
                                                     double damp_over_nstore, double* __restrict__ delta64,
                                                     float* __restrict__ delta_out) {
  __shared__ double red[1024];
  double acc = 0.0;
  for (int i = threadIdx.x; i < n; i += 1024) acc += S[(size_t)i * n + i];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double d = damp_over_nstore * red[0] * inv_rows;
    *delta64 = d;
    if (delta_out) *delta_out = (float)d;
  }
}

// Hd (n_store x n_store fp64, full) = pad(S / N), for a rotation in fp64 before rounding to fp32.
__global__ void expand_kernel(const double* __restrict__ S, int n, int64_t n_store, double inv_rows,
                              double* __restrict__ Hd) {
  const int64_t i = blockIdx.y;
  for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n_store; j += (int64_t)gridDim.x * blockDim.x) {
    double v = 0.0;
    if (i < n && j < n) v = (i >= j ? S[i * n + j] : S[j * n + i]) * inv_rows;
    Hd[i * n_store + j] = v;
  }
}

__global__ void damp_round_kernel(const double* __restrict__ Hd, int64_t n_store, const double* __restrict__ delta64,
                                  float* __restrict__ H, int64_t ldh) {
  const int64_t i = blockIdx.y;
  const double delta = *delta64;
  for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n_store; j += (int64_t)gridDim.x * blockDim.x)
    H[i * ldh + j] = (float)(Hd[i * n_store + j] + (i == j ? delta : 0.0));
}

// H = S/N + delta I (S's lower triangle mirrored, zero padding to n_store, delta on the whole
// diagonal), rounded to fp32.  One workgroup per lower 64 x 64 tile (I, J) of the padded matrix:
// the tile of S is read once, coalesced, into LDS and written to H at (I, J) and transposed at
// (J, I); a diagonal tile takes its upper half from its own lower half.
constexpr int FZ_T = 64;
__global__ __launch_bounds__(256) void finalize_kernel(const double* __restrict__ S, int n, int64_t n_store,
                                                       double inv_rows, const double* __restrict__ delta64,
                                                       float* __restrict__ H, int64_t ldh) {
  __shared__ double t[FZ_T][FZ_T + 1];
  int I, J;
  tri_tile(blockIdx.x, I, J);
  const double delta = *delta64;
  const int c = threadIdx.x & (FZ_T - 1);
  const int64_t i0 = (int64_t)FZ_T * I, j0 = (int64_t)FZ_T * J;
  for (int r = threadIdx.x / FZ_T; r < FZ_T; r += 256 / FZ_T) {
    const int64_t i = i0 + r, j = j0 + c;
    t[r][c] = (i < n && j < n && i >= j) ? S[i * n + j] : 0.0;
  }
  __syncthreads();
  // element (i, j) of H from the tile: S[i][j] for i >= j, else S[j][i]
  for (int r = threadIdx.x / FZ_T; r < FZ_T; r += 256 / FZ_T) {
    const int64_t i = i0 + r, j = j0 + c;
    if (i < n_store && j < n_store) {
      double v = (I != J || r >= c ? t[r][c] : t[c][r]) * inv_rows;
      if (i == j) v += delta;
      H[i * ldh + j] = (float)v;
    }
  }
  if (I == J) return;
  for (int r = threadIdx.x / FZ_T; r < FZ_T; r += 256 / FZ_T) {  // H[j0 + r][i0 + c] = S[i0 + c][j0 + r]
    const int64_t i = j0 + r, j = i0 + c;
    if (i < n_store && j < n_store) H[i * ldh + j] = (float)(t[c][r] * inv_rows);
  }
}


// The rotated form H = R pad(S/N) R^T + delta I with R = blockdiag_k(H_m diag(d_k)) / sqrt(m)
// (64 <= m <= 1024) in two passes over fp64 memory instead of six.  A workgroup holds 4096
// values in LDS: 4096 / m vectors of length m, each stored in chunks of 32 values at a pitch of 33
// (element i of vector v at v (m / 32) 33 + 33 (i / 32) + i % 32).  The transform of a vector is
// done by m / 32 threads in two register passes: each thread takes one chunk (32 consecutive
// values) through the stages 0..4 of the butterfly (pairs i, i + 2^s), then, after one exchange
// through LDS, 32 / (m / 32) columns of the chunk grid through the stages 5..log2(m) - 1.  The
// stages run in the natural order, so every value takes the same additions as in the one-stage-
// at-a-time transform.
constexpr int RT_THREADS = 128;             // one chunk of 32 values per thread
constexpr int RT_VALS = 32 * RT_THREADS;    // values per workgroup
constexpr int RT_LDS = RT_THREADS * 33;     // doubles: the chunks at a pitch of 33 (34 KB)
constexpr int RT_LOG2VALS = 12;

__device__ __forceinline__ int rt_pos(int v, int i, int m) { return v * (m >> 5) * 33 + (i >> 5) * 33 + (i & 31); }

// In-place transform of the 4096 / m vectors in buf (layout above); 128 threads; m >= 64.
__device__ __forceinline__ void rt_fwht(double* buf, int m, int log2m, int tid) {
  const int g = m >> 5;                                   // chunks per vector = threads per vector
  const int v = tid >> (log2m - 5), q = tid & (g - 1);    // this thread's vector and chunk
  double x[32];
  double* base = buf + v * g * 33;
#pragma unroll
  for (int k = 0; k < 32; ++k) x[k] = base[q * 33 + k];
#pragma unroll
  for (int h = 1; h < 32; h <<= 1)
#pragma unroll
    for (int k = 0; k < 32; ++k)
      if (!(k & h)) {
        const double a = x[k], b = x[k + h];
        x[k] = a + b;
        x[k + h] = a - b;
      }
#pragma unroll
  for (int k = 0; k < 32; ++k) base[q * 33 + k] = x[k];
  __syncthreads();
  // stages 5..: thread q takes columns l = q (32 / g) + u (u < 32 / g) of the g x 32 chunk grid;
  // x[u g + c] = element 32 c + l
  const int per = 32 >> (log2m - 5), l0 = q * per;
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    const int u = k >> (log2m - 5), c = k & (g - 1);
    x[k] = base[c * 33 + l0 + u];
  }
#pragma unroll
  for (int h = 1; h < 32; h <<= 1) {
    if (h < g) {  // uniform
#pragma unroll
      for (int k = 0; k < 32; ++k)
        if (!(k & h)) {
          const double a = x[k], b = x[k + h];
          x[k] = a + b;
          x[k + h] = a - b;
        }
    }
  }
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    const int u = k >> (log2m - 5), c = k & (g - 1);
    base[c * 33 + l0 + u] = x[k];
  }
  __syncthreads();
}

// Rows pass, T = pad(S/N) R^T: one workgroup per (block of 4096 / m rows, segment of m columns);
// the rows' segment of the mirrored S (scaled by 1/N, times the signs of its columns) is read into
// LDS -- from S's rows below the diagonal, from S's columns above it (then read as rows of S, 4096/m
// consecutive values each), element by element where the segment crosses the diagonal -- and its
// transform, times 1/sqrt(m), written to T.
__global__ __launch_bounds__(RT_THREADS) void rot_rows_sym_kernel(const double* __restrict__ S, int n, int64_t ns,
                                                           double inv_rows, const int8_t* __restrict__ signs, int m,
                                                           int log2m, double scale, double* __restrict__ T) {
  __shared__ double buf[RT_LDS];
  const int rb = RT_VALS / m, log2rb = RT_LOG2VALS - log2m;  // m, rb powers of two: shifts, no division
  const int64_t i0 = (int64_t)blockIdx.y * rb, j0 = (int64_t)blockIdx.x * m;
  const int tid = threadIdx.x;
  // every load of the thread is issued before the first LDS store (32 in flight per thread)
  constexpr int PER = RT_VALS / RT_THREADS;
  double v[PER];
  if (j0 + m - 1 <= i0) {  // wholly below the diagonal: rows of S
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int e = tid + RT_THREADS * k, r = e >> log2m, c = e & (m - 1);
      const int64_t i = i0 + r, j = j0 + c;
      v[k] = i < n && j < n ? S[i * n + j] : 0.0;
    }
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int e = tid + RT_THREADS * k, r = e >> log2m, c = e & (m - 1);
      buf[rt_pos(r, c, m)] = v[k] * inv_rows * (double)signs[j0 + c];
    }
  } else if (j0 > i0 + rb - 1) {  // wholly above: S[j][i] for the rows i of the block
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int e = tid + RT_THREADS * k, c = e >> log2rb, r = e & (rb - 1);
      const int64_t i = i0 + r, j = j0 + c;
      v[k] = i < n && j < n ? S[j * n + i] : 0.0;
    }
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int e = tid + RT_THREADS * k, c = e >> log2rb, r = e & (rb - 1);
      buf[rt_pos(r, c, m)] = v[k] * inv_rows * (double)signs[j0 + c];
    }
  } else {
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int e = tid + RT_THREADS * k, r = e >> log2m, c = e & (m - 1);
      const int64_t i = i0 + r, j = j0 + c;
      v[k] = i < n && j < n ? (i >= j ? S[i * n + j] : S[j * n + i]) : 0.0;
    }
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int e = tid + RT_THREADS * k, r = e >> log2m, c = e & (m - 1);
      buf[rt_pos(r, c, m)] = v[k] * inv_rows * (double)signs[j0 + c];
    }
  }
  __syncthreads();
  rt_fwht(buf, m, log2m, tid);
  for (int e = tid; e < RT_VALS; e += RT_THREADS) {
    const int r = e >> log2m, c = e & (m - 1);
    if (i0 + r < ns) T[(i0 + r) * ns + j0 + c] = buf[rt_pos(r, c, m)] * scale;
  }
}

// Columns pass, H = R T + delta I rounded to fp32: one workgroup per (segment of m rows, strip of
// 4096 / m columns); the strip of T times the signs of its rows goes to LDS as 4096 / m column
// vectors, each takes the transform, times 1/sqrt(m), delta on the diagonal, rounded once.
__global__ __launch_bounds__(RT_THREADS) void rot_cols_damp_kernel(const double* __restrict__ T, int64_t ns,
                                                            const int8_t* __restrict__ signs, int m, int log2m,
                                                            double scale, const double* __restrict__ delta64,
                                                            float* __restrict__ H, int64_t ldh) {
  __shared__ double buf[RT_LDS];
  const int cw = RT_VALS / m, log2cw = RT_LOG2VALS - log2m;
  const int64_t i0 = (int64_t)blockIdx.y * m, j0 = (int64_t)blockIdx.x * cw;
  const int tid = threadIdx.x;
  constexpr int PER = RT_VALS / RT_THREADS;
  double v[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) {  // every load issued before the first LDS store
    const int e = tid + RT_THREADS * k, r = e >> log2cw, c = e & (cw - 1);
    const int64_t j = j0 + c;
    v[k] = j < ns ? T[(i0 + r) * ns + j] : 0.0;
  }
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int e = tid + RT_THREADS * k, r = e >> log2cw, c = e & (cw - 1);
    buf[rt_pos(c, r, m)] = j0 + c < ns ? v[k] * (double)signs[i0 + r] : 0.0;
  }
  __syncthreads();
  rt_fwht(buf, m, log2m, tid);
  const double delta = *delta64;
  for (int e = tid; e < RT_VALS; e += RT_THREADS) {
    const int r = e >> log2cw, c = e & (cw - 1);
    const int64_t i = i0 + r, j = j0 + c;
    if (j < ns) {
      double val = buf[rt_pos(c, r, m)] * scale;
      if (i == j) val += delta;
      H[i * ldh + j] = (float)val;
    }
  }
}

}  // namespace wr

using namespace wr;

int wr_rotate_sym_f64(wr_ctx* ctx, double* M, int64_t n, int64_t ld, int32_t m, const int8_t* signs);

size_t wr_finalize_ws_bytes(int64_t n_store) { return 256 + (size_t)n_store * n_store * sizeof(double); }

int wr_hessian_finalize_impl(wr_ctx* ctx, const double* S, int64_t n, int64_t total_rows, float damp_frac,
                             int64_t n_store, float* H, int64_t ldh, float* delta_out, int32_t had_block,
                             const int8_t* signs) {
  const size_t need = had_block ? wr_finalize_ws_bytes(n_store) : 256;
  if (ctx->ws_bytes < need) return WR_EWORKSPACE;
  double* delta64 = static_cast<double*>(ctx->ws);
  const double inv_rows = 1.0 / (double)total_rows;
  hipLaunchKernelGGL(trace_kernel, dim3(1), dim3(1024), 0, ctx->stream, S, (int)n, inv_rows,
                     (double)damp_frac / (double)n_store, delta64, delta_out);
  WR_CHECK_LAUNCH();
  const unsigned gx = (unsigned)std::min<int64_t>((n_store + 255) / 256, 64);
  if (!had_block) {
    const int64_t nt = (n_store + FZ_T - 1) / FZ_T;
    hipLaunchKernelGGL(finalize_kernel, dim3((unsigned)(nt * (nt + 1) / 2)), dim3(256), 0, ctx->stream, S, (int)n,
                       n_store, inv_rows, delta64, H, ldh);
    WR_CHECK_LAUNCH();
    return WR_OK;
  }
  // H = R pad(S/N) R^T + delta I, rotated in fp64 and rounded to fp32 once
  double* Hd = reinterpret_cast<double*>(static_cast<char*>(ctx->ws) + 256);
  if (had_block >= 64 && had_block <= 1024) {
    int log2m = 0;
    while ((1 << log2m) < had_block) ++log2m;
    const double scale = 1.0 / std::sqrt((double)had_block);
    const int rb = RT_VALS / had_block;
    hipLaunchKernelGGL(rot_rows_sym_kernel, dim3((unsigned)(n_store / had_block), (unsigned)((n_store + rb - 1) / rb)),
                       dim3(RT_THREADS), 0, ctx->stream, S, (int)n, n_store, inv_rows, signs, had_block, log2m, scale,
                       Hd);
    WR_CHECK_LAUNCH();
    hipLaunchKernelGGL(rot_cols_damp_kernel, dim3((unsigned)((n_store + rb - 1) / rb), (unsigned)(n_store / had_block)),
                       dim3(RT_THREADS), 0, ctx->stream, Hd, n_store, signs, had_block, log2m, scale, delta64, H, ldh);
    WR_CHECK_LAUNCH();
    return WR_OK;
  }
  hipLaunchKernelGGL(expand_kernel, dim3(gx, (unsigned)n_store), dim3(256), 0, ctx->stream, S, (int)n, n_store,
                     inv_rows, Hd);
  WR_CHECK_LAUNCH();
  const int rc = wr_rotate_sym_f64(ctx, Hd, n_store, n_store, had_block, signs);
  if (rc) return rc;
  hipLaunchKernelGGL(damp_round_kernel, dim3(gx, (unsigned)n_store), dim3(256), 0, ctx->stream, Hd, n_store, delta64,
                     H, ldh);
  WR_CHECK_LAUNCH();
  return WR_OK;
}
