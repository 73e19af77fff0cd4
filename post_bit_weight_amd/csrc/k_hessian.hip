// Calibration second moment S += X^T X (lower triangle) and H = S/N + delta I.
//
// H is the average of x x^T over calibration inputs (Pingala-8 post, "Trick 2:
// round with error feedback"); delta is the Tikhonov damping of the GPTQ solve
// (Wringer news article, second paragraph).
//
// bf16 path: a SYRK on the bf16 matrix cores.  Each workgroup owns one 128x128
// lower tile of S and a range of calibration rows.  X rows are row-major with
// the feature index contiguous, while an MFMA operand wants 8 consecutive rows
// per lane, so each thread loads an 8x8 bf16 block, transposes it in registers
// and stores it to LDS with one 16-byte write.  bf16 x bf16 products are exact
// in fp32; the fp32 accumulators are flushed into fp64 every 512 rows, which
// keeps the relative error of S near 1e-8.  Tiles with a range of rows shorter
// than the whole call write fp32 partials that a second kernel adds into S in
// a fixed order (deterministic, no atomics).
#include "common.hpp"

namespace wr {

constexpr int SY_TILE = 128;
constexpr int SY_KT = 64;                // calibration rows per LDS stage
constexpr int SY_PITCH = SY_KT + 8;      // bf16 per LDS row (+16 B: conflict-free 16-byte reads)
constexpr int SY_SEG_STAGES = 8;         // 8 x 64 = 512 rows per fp32 segment
constexpr int F32_TILE = 64;

__device__ __forceinline__ void tile_from_linear(int t, int& ti, int& tj) {
  int i = (int)((sqrtf(8.0f * (float)t + 1.0f) - 1.0f) * 0.5f);
  while (i * (i + 1) / 2 > t) --i;
  while ((i + 1) * (i + 2) / 2 <= t) ++i;
  ti = i;
  tj = t - i * (i + 1) / 2;
}

// Writes one tile element's contribution: directly into S (single range of rows)
// or into the fp32 partial buffer of this split.
__device__ __forceinline__ void emit(double v, int gi, int gj, int ii, int jj, int n, int tile, int tiles,
                                     int split, int tdim, double* S, float* partial) {
  if (partial) {
    partial[(((size_t)split * tiles + tile) * tdim + ii) * tdim + jj] = (float)v;
  } else if (gi < n && gj < n && gi >= gj) {
    S[(size_t)gi * n + gj] += v;
  }
}

__global__ __launch_bounds__(256, 1) void syrk_bf16_kernel(const uint16_t* __restrict__ X, int64_t rows, int n,
                                                           int64_t ldx, int64_t rows_per_split, int tiles,
                                                           double* __restrict__ S, float* __restrict__ partial) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][SY_TILE * SY_PITCH];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][SY_TILE * SY_PITCH];

  const int tile = blockIdx.x, split = blockIdx.y;
  int ti, tj;
  tile_from_linear(tile, ti, tj);
  const int64_t r0 = (int64_t)split * rows_per_split;
  const int64_t r1 = r0 + rows_per_split < rows ? r0 + rows_per_split : rows;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wi = wave >> 1, wj = wave & 1;

  // loader coordinates: operand 0 = i-side columns, 1 = j-side columns
  const int op = tid >> 7, b = tid & 127, kg = b >> 4, ig = b & 15;
  const int colbase = (op == 0 ? ti : tj) * SY_TILE + 8 * ig;
  const bool col_ok = colbase < n;
  uint16_t* sdst = op == 0 ? &sA[0][0] : &sB[0][0];

  u32x4 ld[8];
  auto load_stage = [&](int64_t k0) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      int64_t row = k0 + 8 * kg + r;
      if (col_ok && row < r1) {
        ld[r] = *reinterpret_cast<const u32x4*>(X + row * ldx + colbase);
      } else {
        ld[r] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto store_stage = [&](int buf) {
    uint16_t* base = sdst + buf * (SY_TILE * SY_PITCH);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int d = c >> 1;
      u32x4 o;
      uint32_t w[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) w[r] = ld[r][d];
      if ((c & 1) == 0) {
        o[0] = (w[0] & 0xffffu) | (w[1] << 16);
        o[1] = (w[2] & 0xffffu) | (w[3] << 16);
        o[2] = (w[4] & 0xffffu) | (w[5] << 16);
        o[3] = (w[6] & 0xffffu) | (w[7] << 16);
      } else {
        o[0] = (w[0] >> 16) | (w[1] & 0xffff0000u);
        o[1] = (w[2] >> 16) | (w[3] & 0xffff0000u);
        o[2] = (w[4] >> 16) | (w[5] & 0xffff0000u);
        o[3] = (w[6] >> 16) | (w[7] & 0xffff0000u);
      }
      *reinterpret_cast<u32x4*>(base + (8 * ig + c) * SY_PITCH + 8 * kg) = o;
    }
  };

  f32x16 acc[2][2];
  double tot[2][2][16];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y) {
      acc[x][y] = f32x16{};
#pragma unroll
      for (int v = 0; v < 16; ++v) tot[x][y][v] = 0.0;
    }

  const int64_t nstages = r1 > r0 ? (r1 - r0 + SY_KT - 1) / SY_KT : 0;
  if (nstages > 0) {
    load_stage(r0);
    store_stage(0);
  }
  __syncthreads();
  const int arow = 64 * wi + (lane & 31), brow = 64 * wj + (lane & 31), koff = 8 * (lane >> 5);
  for (int64_t s = 0; s < nstages; ++s) {
    const int buf = (int)(s & 1);
    if (s + 1 < nstages) load_stage(r0 + (s + 1) * SY_KT);
    const uint16_t* pa = &sA[buf][0];
    const uint16_t* pb = &sB[buf][0];
#pragma unroll
    for (int ks = 0; ks < SY_KT / 16; ++ks) {
      bf16x8 a0 = as_bf16x8(*reinterpret_cast<const u32x4*>(pa + arow * SY_PITCH + 16 * ks + koff));
      bf16x8 a1 = as_bf16x8(*reinterpret_cast<const u32x4*>(pa + (arow + 32) * SY_PITCH + 16 * ks + koff));
      bf16x8 b0 = as_bf16x8(*reinterpret_cast<const u32x4*>(pb + brow * SY_PITCH + 16 * ks + koff));
      bf16x8 b1 = as_bf16x8(*reinterpret_cast<const u32x4*>(pb + (brow + 32) * SY_PITCH + 16 * ks + koff));
      acc[0][0] = mfma32x32x16_bf16(a0, b0, acc[0][0]);
      acc[0][1] = mfma32x32x16_bf16(a0, b1, acc[0][1]);
      acc[1][0] = mfma32x32x16_bf16(a1, b0, acc[1][0]);
      acc[1][1] = mfma32x32x16_bf16(a1, b1, acc[1][1]);
    }
    if (s + 1 < nstages) store_stage(buf ^ 1);
    if ((s + 1) % SY_SEG_STAGES == 0 || s + 1 == nstages) {
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y) {
#pragma unroll
          for (int v = 0; v < 16; ++v) tot[x][y][v] += (double)acc[x][y][v];
          acc[x][y] = f32x16{};
        }
    }
    __syncthreads();
  }

#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int ii = 64 * wi + 32 * x + acc_row(v, lane);
        const int jj = 64 * wj + 32 * y + (lane & 31);
        emit(tot[x][y][v], ti * SY_TILE + ii, tj * SY_TILE + jj, ii, jj, n, tile, tiles, split, SY_TILE, S, partial);
      }
}

// fp32 inputs (products rounded to fp32): plain FMA tiles, 64x64 per workgroup,
// fp32 accumulation flushed into fp64 every 512 rows.
__global__ __launch_bounds__(256) void syrk_f32_kernel(const float* __restrict__ X, int64_t rows, int n, int64_t ldx,
                                                       int64_t rows_per_split, int tiles, double* __restrict__ S,
                                                       float* __restrict__ partial) {
  __shared__ float sA[16][F32_TILE + 4];
  __shared__ float sB[16][F32_TILE + 4];
  const int tile = blockIdx.x, split = blockIdx.y;
  int ti, tj;
  tile_from_linear(tile, ti, tj);
  const int64_t r0 = (int64_t)split * rows_per_split;
  const int64_t r1 = r0 + rows_per_split < rows ? r0 + rows_per_split : rows;
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  float acc[4][4] = {};
  double tot[4][4] = {};
  const int lrow = tid >> 4, lcol = (tid & 15) * 4;
  int seg = 0;
  for (int64_t k0 = r0; k0 < r1; k0 += 16) {
    const int64_t row = k0 + lrow;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      int ci = ti * F32_TILE + lcol + c, cj = tj * F32_TILE + lcol + c;
      sA[lrow][lcol + c] = (row < r1 && ci < n) ? X[row * ldx + ci] : 0.0f;
      sB[lrow][lcol + c] = (row < r1 && cj < n) ? X[row * ldx + cj] : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      float a[4], bb[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        a[q] = sA[k][4 * ty + q];
        bb[q] = sB[k][4 * tx + q];
      }
#pragma unroll
      for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[p][q] = fmaf(a[p], bb[q], acc[p][q]);
    }
    __syncthreads();
    if (++seg == 32 || k0 + 16 >= r1) {
      seg = 0;
#pragma unroll
      for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          tot[p][q] += (double)acc[p][q];
          acc[p][q] = 0.0f;
        }
    }
  }
#pragma unroll
  for (int p = 0; p < 4; ++p)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int ii = 4 * ty + p, jj = 4 * tx + q;
      emit(tot[p][q], ti * F32_TILE + ii, tj * F32_TILE + jj, ii, jj, n, tile, tiles, split, F32_TILE, S, partial);
    }
}

// S[lower] += sum over splits of the fp32 partials, splits added in index order.
__global__ void syrk_reduce_kernel(const float* __restrict__ partial, int ksplit, int tiles, int tdim, int n,
                                   double* __restrict__ S) {
  const int tile = blockIdx.x;
  int ti, tj;
  tile_from_linear(tile, ti, tj);
  for (int e = threadIdx.x; e < tdim * tdim; e += blockDim.x) {
    const int ii = e / tdim, jj = e % tdim;
    const int gi = ti * tdim + ii, gj = tj * tdim + jj;
    if (gi >= n || gj >= n || gi < gj) continue;
    double acc = 0.0;
    for (int s = 0; s < ksplit; ++s) acc += (double)partial[(((size_t)s * tiles + tile) * tdim + ii) * tdim + jj];
    S[(size_t)gi * n + gj] += acc;
  }
}

__global__ void zero_lower_kernel(double* S, int n) {
  const int i = blockIdx.x;
  for (int j = threadIdx.x; j <= i; j += blockDim.x) S[(size_t)i * n + j] = 0.0;
}

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

__global__ void finalize_kernel(const double* __restrict__ S, int n, int64_t n_store, double inv_rows,
                                const double* __restrict__ delta64, float* __restrict__ H, int64_t ldh) {
  const int64_t i = blockIdx.y;
  const double delta = *delta64;
  for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n_store; j += (int64_t)gridDim.x * blockDim.x) {
    double v = 0.0;
    if (i < n && j < n) v = (i >= j ? S[i * n + j] : S[j * n + i]) * inv_rows;
    if (i == j) v += delta;
    H[i * ldh + j] = (float)v;
  }
}

}  // namespace wr

using namespace wr;

// Row splits are chosen for a 256-CU part so the workspace size does not depend on the device.
static constexpr int kSplitCUs = 256;

static int syrk_tiles(int64_t n, int tdim) {
  const int nt = (int)((n + tdim - 1) / tdim);
  return nt * (nt + 1) / 2;
}

// Number of row splits: enough workgroups to fill the chip in near-whole waves.
static int syrk_ksplit(int64_t rows, int64_t n, int tdim, int num_cu) {
  if (rows <= 0) return 1;
  const int tiles = syrk_tiles(n, tdim);
  const int64_t max_split = (rows + 511) / 512;
  int best = 1;
  double best_eff = 0.0;
  for (int k = 1; k <= 32 && k <= max_split; ++k) {
    const double wgs = (double)tiles * k;
    const double waves = std::ceil(wgs / num_cu);
    const double eff = wgs / (waves * num_cu);
    if (eff > best_eff + 0.05) {
      best_eff = eff;
      best = k;
    }
    if (eff >= 0.9) break;
  }
  return best;
}

size_t wr_hessian_ws_bytes(int64_t rows, int64_t n, int x_dtype, int num_cu) {
  const int tdim = x_dtype == WR_F32 ? F32_TILE : SY_TILE;
  const int ks = syrk_ksplit(rows, n, tdim, num_cu);
  size_t bytes = 256;  // finalize scalars
  if (ks > 1) bytes += (size_t)ks * syrk_tiles(n, tdim) * tdim * tdim * sizeof(float);
  return bytes;
}

int wr_hessian_accumulate_impl(wr_ctx* ctx, const void* X, int x_dtype, int64_t rows, int64_t n, int64_t ldx,
                               double* S, int flags) {
  hipStream_t st = ctx->stream;
  if (flags & WR_H_ZERO) {
    hipLaunchKernelGGL(zero_lower_kernel, dim3((unsigned)n), dim3(256), 0, st, S, (int)n);
    WR_CHECK_LAUNCH();
  }
  if (rows == 0) return WR_OK;
  const int tdim = x_dtype == WR_F32 ? F32_TILE : SY_TILE;
  const int tiles = syrk_tiles(n, tdim);
  const int ks = syrk_ksplit(rows, n, tdim, kSplitCUs);
  const int64_t rps = (rows + ks - 1) / ks;
  float* partial = nullptr;
  if (ks > 1) {
    if (ctx->ws_bytes < wr_hessian_ws_bytes(rows, n, x_dtype, kSplitCUs)) return WR_EWORKSPACE;
    partial = reinterpret_cast<float*>(static_cast<char*>(ctx->ws) + 256);
  }
  dim3 grid((unsigned)tiles, (unsigned)ks);
  if (x_dtype == WR_BF16) {
    hipLaunchKernelGGL(syrk_bf16_kernel, grid, dim3(256), 0, st, static_cast<const uint16_t*>(X), rows, (int)n, ldx,
                       rps, tiles, S, partial);
  } else {
    hipLaunchKernelGGL(syrk_f32_kernel, grid, dim3(256), 0, st, static_cast<const float*>(X), rows, (int)n, ldx, rps,
                       tiles, S, partial);
  }
  WR_CHECK_LAUNCH();
  if (ks > 1) {
    hipLaunchKernelGGL(syrk_reduce_kernel, dim3((unsigned)tiles), dim3(256), 0, st, partial, ks, tiles, tdim, (int)n, S);
    WR_CHECK_LAUNCH();
  }
  return WR_OK;
}

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
    hipLaunchKernelGGL(finalize_kernel, dim3(gx, (unsigned)n_store), dim3(256), 0, ctx->stream, S, (int)n, n_store,
                       inv_rows, delta64, H, ldh);
    WR_CHECK_LAUNCH();
    return WR_OK;
  }
  // H = R pad(S/N) R^T + delta I, rotated in fp64 and rounded to fp32 once
  double* Hd = reinterpret_cast<double*>(static_cast<char*>(ctx->ws) + 256);
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
