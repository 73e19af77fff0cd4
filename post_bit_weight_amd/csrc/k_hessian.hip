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
constexpr int SY_KT = 64;                // calibration rows per LDS stage (8 chunks of 16 bytes per LDS row)
constexpr int SY_SEG_STAGES = 8;         // 8 x 64 = 512 rows per fp32 segment
constexpr int SY_XCD = 8;                // workgroups are dispatched round-robin over 8 XCDs

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

// LDS row r of an operand tile holds 64 calibration rows (k) of feature r as eight
// 16-byte chunks; chunk q is stored at position q ^ swz(r).  The transposed
// stores (8 lanes: rows 8g + c, g = 0..7, one chunk) and the MFMA fragment reads
// (8 lanes: 8 consecutive rows, one chunk) then both touch 8 distinct bank groups.
__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

// S_lower += XA^T XB over the rows (XA supplies the tile's row features, XB its
// column features; both rows x n bf16 with leading dimension ldx).
__global__ __launch_bounds__(256, 1) void syrk_bf16_kernel(const uint16_t* __restrict__ XA, const uint16_t* __restrict__ XB,
                                                           int64_t rows, int n, int64_t ldx, int64_t rows_per_split,
                                                           int tiles, int ksplit, double* __restrict__ S,
                                                           float* __restrict__ partial) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][SY_TILE * SY_KT];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][SY_TILE * SY_KT];

  // XCD-aware order: all workgroups of one row split land on the same XCD, so the
  // X rows they share are fetched into that XCD's L2 once.
  int tile, split;
  {
    const int bid = blockIdx.x;
    if (ksplit % SY_XCD == 0) {
      const int per = SY_XCD * tiles;
      split = (bid % SY_XCD) + SY_XCD * (bid / per);
      tile = (bid / SY_XCD) % tiles;
    } else {
      split = bid / tiles;
      tile = bid % tiles;
    }
  }
  int ti, tj;
  tile_from_linear(tile, ti, tj);
  const int64_t r0 = (int64_t)split * rows_per_split;
  const int64_t r1 = r0 + rows_per_split < rows ? r0 + rows_per_split : rows;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wi = wave >> 1, wj = wave & 1;

  // loader: operand 0 = i-side columns, 1 = j-side columns; an 8x8 block per thread
  const int op = tid >> 7, b = tid & 127, kg = b >> 4, ig = b & 15;
  const int colbase = (op == 0 ? ti : tj) * SY_TILE + 8 * ig;
  const bool col_ok = colbase < n;
  uint16_t* sdst = op == 0 ? &sA[0][0] : &sB[0][0];
  const uint16_t* X = op == 0 ? XA : XB;

  u32x4 ld[8];
  auto load_stage = [&](int64_t k0) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int64_t row = k0 + 8 * kg + r;
      if (col_ok && row < r1) {
        ld[r] = *reinterpret_cast<const u32x4*>(X + row * ldx + colbase);
      } else {
        ld[r] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto store_stage = [&](int buf) {
    uint16_t* base = sdst + buf * (SY_TILE * SY_KT);
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
      const int rr = 8 * ig + c;
      *reinterpret_cast<u32x4*>(base + rr * SY_KT + 8 * (kg ^ swz(rr))) = o;
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
  const int arow0 = 64 * wi + (lane & 31), brow0 = 64 * wj + (lane & 31), khalf = lane >> 5;
  const int sa0 = swz(arow0), sa1 = swz(arow0 + 32), sb0 = swz(brow0), sb1 = swz(brow0 + 32);
  for (int64_t s = 0; s < nstages; ++s) {
    const int buf = (int)(s & 1);
    if (s + 1 < nstages) load_stage(r0 + (s + 1) * SY_KT);
    const uint16_t* pa = &sA[buf][0];
    const uint16_t* pb = &sB[buf][0];
#pragma unroll
    for (int ks = 0; ks < SY_KT / 16; ++ks) {
      const int q = 2 * ks + khalf;
      bf16x8 a0 = as_bf16x8(*reinterpret_cast<const u32x4*>(pa + arow0 * SY_KT + 8 * (q ^ sa0)));
      bf16x8 a1 = as_bf16x8(*reinterpret_cast<const u32x4*>(pa + (arow0 + 32) * SY_KT + 8 * (q ^ sa1)));
      bf16x8 b0 = as_bf16x8(*reinterpret_cast<const u32x4*>(pb + brow0 * SY_KT + 8 * (q ^ sb0)));
      bf16x8 b1 = as_bf16x8(*reinterpret_cast<const u32x4*>(pb + (brow0 + 32) * SY_KT + 8 * (q ^ sb1)));
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

// fp32 inputs: x = x0 + x1 + x2 with bf16 parts (exact for normal-range values),
// so X^T X = sum_{a+b<=2} Xa^T Xb to about 2^-24 with every product exact.
__global__ void split3_kernel(const float* __restrict__ X, int64_t rows, int n, int64_t ldx, uint16_t* __restrict__ P0,
                              uint16_t* __restrict__ P1, uint16_t* __restrict__ P2) {
  const int64_t r = blockIdx.y;
  for (int j = blockIdx.x * blockDim.x + threadIdx.x; j < n; j += gridDim.x * blockDim.x) {
    const float x = X[r * ldx + j];
    const uint32_t a = f32_to_bf16_bits(x);
    const float r1 = x - bf16_bits_to_f32(a);
    const uint32_t b = f32_to_bf16_bits(r1);
    const float r2 = r1 - bf16_bits_to_f32(b);
    P0[r * n + j] = (uint16_t)a;
    P1[r * n + j] = (uint16_t)b;
    P2[r * n + j] = (uint16_t)f32_to_bf16_bits(r2);
  }
}

// S[lower] += sum over splits of the fp32 partials, splits added in index order.
// One thread per tile element; grid.y = tile.
__global__ void syrk_reduce_kernel(const float* __restrict__ partial, int ksplit, int tiles, int tdim, int n,
                                   double* __restrict__ S) {
  const int tile = blockIdx.y;
  int ti, tj;
  tile_from_linear(tile, ti, tj);
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= tdim * tdim) return;
  const int ii = e / tdim, jj = e - ii * tdim;
  const int gi = ti * tdim + ii, gj = tj * tdim + jj;
  if (gi >= n || gj >= n || gi < gj) return;
  const size_t stride = (size_t)tiles * tdim * tdim;
  const float* p = partial + (size_t)tile * tdim * tdim + e;
  double acc = 0.0;
  for (int s = 0; s < ksplit; ++s) acc += (double)p[s * stride];
  S[(size_t)gi * n + gj] += acc;
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

// Number of row splits: a multiple of the XCD count (each XCD works through its
// own rows), enough workgroups for near-whole waves on the chip, and at least
// 512 rows per split.
static int syrk_ksplit(int64_t rows, int64_t n, int num_cu) {
  if (rows <= 0) return 1;
  const int tiles = syrk_tiles(n, SY_TILE);
  const int64_t max_split = std::max<int64_t>(1, rows / 512);
  int best = 1;
  double best_eff = 0.0;
  for (int k = SY_XCD; k <= 64 && k <= max_split; k += SY_XCD) {
    const double wgs = (double)tiles * k;
    const double eff = wgs / (std::ceil(wgs / num_cu) * num_cu);
    if (eff > best_eff + 0.03) {
      best_eff = eff;
      best = k;
    }
    if (eff >= 0.9) break;
  }
  return best;
}

static size_t partial_bytes(int64_t rows, int64_t n) {
  const int ks = syrk_ksplit(rows, n, kSplitCUs);
  return ks > 1 ? (size_t)ks * syrk_tiles(n, SY_TILE) * SY_TILE * SY_TILE * sizeof(float) : 0;
}

size_t wr_hessian_ws_bytes(int64_t rows, int64_t n, int x_dtype, int num_cu) {
  (void)num_cu;
  size_t bytes = 256 + ((partial_bytes(rows, n) + 255) & ~(size_t)255);
  if (x_dtype == WR_F32) bytes += 3 * (((size_t)rows * n * 2 + 255) & ~(size_t)255);
  return bytes;
}

// One SYRK pass S_lower += XA^T XB (bf16 sources, ld ldx), with its split-K reduction.
static int syrk_pass(wr_ctx* ctx, const uint16_t* XA, const uint16_t* XB, int64_t rows, int64_t n, int64_t ldx,
                     double* S, float* partial) {
  hipStream_t st = ctx->stream;
  const int tiles = syrk_tiles(n, SY_TILE);
  const int ks = syrk_ksplit(rows, n, kSplitCUs);
  const int64_t rps = (rows + ks - 1) / ks;
  hipLaunchKernelGGL(syrk_bf16_kernel, dim3((unsigned)(tiles * ks)), dim3(256), 0, st, XA, XB, rows, (int)n, ldx, rps,
                     tiles, ks, S, ks > 1 ? partial : nullptr);
  WR_CHECK_LAUNCH();
  if (ks > 1) {
    dim3 rgrid((unsigned)((SY_TILE * SY_TILE + 255) / 256), (unsigned)tiles);
    hipLaunchKernelGGL(syrk_reduce_kernel, rgrid, dim3(256), 0, st, partial, ks, tiles, SY_TILE, (int)n, S);
    WR_CHECK_LAUNCH();
  }
  return WR_OK;
}

int wr_hessian_accumulate_impl(wr_ctx* ctx, const void* X, int x_dtype, int64_t rows, int64_t n, int64_t ldx,
                               double* S, int flags) {
  hipStream_t st = ctx->stream;
  if (flags & WR_H_ZERO) {
    hipLaunchKernelGGL(zero_lower_kernel, dim3((unsigned)n), dim3(256), 0, st, S, (int)n);
    WR_CHECK_LAUNCH();
  }
  if (rows == 0) return WR_OK;
  if (ctx->ws_bytes < wr_hessian_ws_bytes(rows, n, x_dtype, kSplitCUs)) return WR_EWORKSPACE;
  char* ws = static_cast<char*>(ctx->ws);
  float* partial = reinterpret_cast<float*>(ws + 256);
  if (x_dtype == WR_BF16) {
    const uint16_t* Xb = static_cast<const uint16_t*>(X);
    return syrk_pass(ctx, Xb, Xb, rows, n, ldx, S, partial);
  }
  const size_t plane = ((size_t)rows * n * 2 + 255) & ~(size_t)255;
  uint16_t* P[3];
  for (int k = 0; k < 3; ++k)
    P[k] = reinterpret_cast<uint16_t*>(ws + 256 + ((partial_bytes(rows, n) + 255) & ~(size_t)255) + k * plane);
  const unsigned gx = (unsigned)std::min<int64_t>((n + 255) / 256, 16);
  hipLaunchKernelGGL(split3_kernel, dim3(gx, (unsigned)rows), dim3(256), 0, st, static_cast<const float*>(X), rows,
                     (int)n, ldx, P[0], P[1], P[2]);
  WR_CHECK_LAUNCH();
  static const int terms[6][2] = {{2, 0}, {1, 1}, {0, 2}, {1, 0}, {0, 1}, {0, 0}};  // small terms first
  for (const auto& t : terms) {
    const int rc = syrk_pass(ctx, P[t[0]], P[t[1]], rows, n, n, S, partial);
    if (rc) return rc;
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
