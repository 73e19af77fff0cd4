// GPTQ / LDLQ error-feedback sweep (Pingala-8 post, "Trick 2: round with error
// feedback"; Wringer model cards, "Recipe": GPTQ codes on a fixed signed grid
// with fp16 block scales).
//
// The unit upper factor M of H = M D M^T comes from the fp64 blocked Cholesky
// of the reversed H (k_chol.hip), rounded to fp32 once.  (An fp32 factorisation
// moves GPTQ block scales by up to two fp16 ulps against an fp64 reference; fp64
// keeps them within one.)
//
// Sweep (LDLQ pull form).  Every row is independent.  With delta_i = w_i - q_i,
// column k is rounded from v_k = w_k + sum_{i<k} M_ik delta_i.  The corrections
// C_k = sum_{i<k} M_ik delta_i are kept in a rows x n buffer: inside a lazy
// batch of columns they are updated one column at a time, and when a batch is
// done the remaining columns receive C += E M[batch, rest] as one product on
// the bf16 matrix cores: E and M split into three bf16 parts each (24
// significant bits, as fp32), the six part products with i + j <= 2 summed in
// fp32, smallest first.
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

size_t wr_factor_ws_bytes(int64_t n);
int wr_factor_m(hipStream_t st, const float* H, int64_t ldh, int n, void* ws, float* M, int32_t* dev_info);

namespace wr {

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

// Value of lane N of each 16-lane row (DPP row broadcast: one VALU op, no LDS round trip).
template <int N>
__device__ __forceinline__ float row_bcast(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x150 + N, 0xf, 0xf, false));
}

// Value of lane SRC of each P-lane group.
template <int P, int SRC>
__device__ __forceinline__ float group_bcast(float v) {
  if constexpr (P == 16) {
    return row_bcast<SRC>(v);
  } else {
    return __shfl(v, SRC, P);
  }
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
                                                          float* __restrict__ Cbuf, uint16_t* __restrict__ E0,
                                                          uint16_t* __restrict__ E1, uint16_t* __restrict__ E2,
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

  {
    // M's diagonal batch block: every thread's 16 four-wide loads are in flight before the LDS stores
    static_assert(BATCH * BATCH == 256 * 64, "16 loads of four floats per thread");
    f32x4 mv[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int e = 4 * (tid + 256 * q), k = e / BATCH, j = e % BATCH;
      mv[q] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (k < ncols && j < ncols) mv[q] = *reinterpret_cast<const f32x4*>(M + (int64_t)(b0 + k) * n + b0 + j);
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int e = 4 * (tid + 256 * q), k = e / BATCH, j = e % BATCH;
#pragma unroll
      for (int u = 0; u < 4; ++u) Ms[k * BATCH + ((j + u) % P) * S + (j + u) / P] = mv[q][u];
    }
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

  static_for<0, NBLK>([&](auto BLK) {
    constexpr int blk = BLK;
    sc[blk] = 0.0f;
    if (blk * G >= ncols) return;  // uniform
    // push-form values at the block start: x = M_bb^-T c_b
    float x[SB];
#pragma unroll
    for (int q = 0; q < SB; ++q) x[q] = c[blk * SB + q];
    // M's rows are read one step ahead so that their LDS latency stays off the serial chain
    float mx[SB];
#pragma unroll
    for (int q = 0; q < SB; ++q) mx[q] = Ms[(blk * G) * BATCH + p * S + blk * SB + q];
    static_for<0, G>([&](auto JJ) {
      constexpr int jj = JJ;
      constexpr int j = blk * G + jj;
      constexpr int owner = j % P, qo = jj / P;
      float mn[SB];
      if constexpr (jj + 1 < G) {
#pragma unroll
        for (int q = 0; q < SB; ++q) mn[q] = Ms[(j + 1) * BATCH + p * S + blk * SB + q];
      }
      const float xj = group_bcast<P, owner>(x[qo]);
#pragma unroll
      for (int q = qo; q < SB; ++q) x[q] = fmaf(-mx[q], xj, x[q]);
      if constexpr (jj + 1 < G) {
#pragma unroll
        for (int q = 0; q < SB; ++q) mx[q] = mn[q];
      }
    });
    float m = 0.0f;
#pragma unroll
    for (int q = 0; q < SB; ++q) m = fmaxf(m, fabsf(w[blk * SB + q] + x[q]));
    m = group_max<P>(m);
    const float s = f16_bits_to_f32(f32_to_f16_bits_clamped(m / (float)L));
    sc[blk] = s;
    const float inv_s = s > 0.0f ? 1.0f / s : 0.0f;
    // round the block's columns one at a time, pushing each error to the later batch columns
    float mc[S];
#pragma unroll
    for (int i = 0; i < S; ++i) mc[i] = Ms[(blk * G) * BATCH + p * S + i];
    static_for<0, G>([&](auto JJ) {
      constexpr int jj = JJ;
      constexpr int j = blk * G + jj;
      constexpr int owner = j % P, io = j / P;
      float mn[S];
      if constexpr (jj + 1 < G) {
#pragma unroll
        for (int i = 0; i < S; ++i) mn[i] = Ms[(j + 1) * BATCH + p * S + i];
      }
      const float v = w[io] + c[io];
      const int cd = nearest_code(v * inv_s, L);
      const float dl = w[io] - (float)(2 * cd - L) * s;
      if (p == owner) {
        code[io] = (uint8_t)cd;
        d[io] = dl;
      }
      const float dj = group_bcast<P, owner>(dl);
#pragma unroll
      for (int i = io; i < S; ++i) c[i] = fmaf(mc[i], dj, c[i]);
      if constexpr (jj + 1 < G) {
#pragma unroll
        for (int i = 0; i < S; ++i) mc[i] = mn[i];
      }
    });
  });

  if (!active) return;
#pragma unroll
  for (int i = 0; i < S; ++i) {
    const int col = p + P * i;
    if (col < ncols) {
      codes[row * n + b0 + col] = code[i];
      const int64_t e = row * BATCH + col;
      split3(d[i], E0[e], E1[e], E2[e]);
    }
  }
  if (p == 0) {
#pragma unroll
    for (int blk = 0; blk < NBLK; ++blk)
      if (blk * G < ncols) scales[row * (n / G) + (b0 / G) + blk] = f32_to_f16_bits_clamped(sc[blk]);
  }
}

// Mt_i[c][k] = part i of M[k][c] (three bf16 planes of M transposed), for the
// trailing update.  64 x 64 tiles through LDS; tiles below the diagonal (M = 0 there)
// are skipped.
__global__ __launch_bounds__(256) void split_mt_kernel(const float* __restrict__ M, int n, uint16_t* __restrict__ Mt0,
                                                       uint16_t* __restrict__ Mt1, uint16_t* __restrict__ Mt2,
                                                       const int32_t* __restrict__ dev_info) {
  __shared__ float t[64][65];
  if (*dev_info != 0) return;
  const int k0 = 64 * blockIdx.y, c0 = 64 * blockIdx.x;
  if (k0 > c0 + 63) return;
  const int tid = threadIdx.x;
  for (int e = tid; e < 64 * 64; e += 256) {
    const int i = e >> 6, j = e & 63;
    t[i][j] = k0 + i < n && c0 + j < n ? M[(int64_t)(k0 + i) * n + c0 + j] : 0.0f;
  }
  __syncthreads();
  for (int e = tid; e < 64 * 64; e += 256) {
    const int j = e >> 6, i = e & 63;  // output row c0 + j, column k0 + i
    if (c0 + j < n && k0 + i < n) {
      const int64_t o = (int64_t)(c0 + j) * n + k0 + i;
      split3(t[i][j], Mt0[o], Mt1[o], Mt2[o]);
    }
  }
}

// C[r][c0 + c] += sum_k E[r][k] M[b0 + k][c0 + c] for r < rows, c < N, k < 128, with E
// and M given as three bf16 planes each (E_i: rows x 128; Mt_i: n x n, transposed).
// 64 x 64 output tile per workgroup.  Wave w takes k in [32 w, 32 w + 32) for the whole
// tile (2 x 2 blocks of 32 x 32, v_mfma_f32_32x32x16_bf16: operand lane l supplies row
// or column l % 32 at k = 8 (l / 32) .. +7 of a 16-wide step), so each wave issues all
// of its operand loads at once (16 contiguous bytes per lane, straight from global
// memory) together with the C tile; the four partial tiles are summed through LDS in
// wave order and added to C.
__global__ __launch_bounds__(256, 2) void trail_s6_kernel(int64_t rows, int N, int n, int b0, int c0,
                                                          const uint16_t* __restrict__ E0,
                                                          const uint16_t* __restrict__ E1,
                                                          const uint16_t* __restrict__ E2,
                                                          const uint16_t* __restrict__ Mt0,
                                                          const uint16_t* __restrict__ Mt1,
                                                          const uint16_t* __restrict__ Mt2, float* __restrict__ C,
                                                          const int32_t* __restrict__ dev_info) {
  __shared__ float red[4][64][65];
  if (*dev_info != 0) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t R0 = (int64_t)blockIdx.y * 64;
  const int C0 = blockIdx.x * 64;
  // the C tile: thread tid holds elements tid + 256 q (row e / 64, column e % 64)
  float cv[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int e = tid + 256 * q, r = e >> 6, c = e & 63;
    cv[q] = R0 + r < rows && C0 + c < N ? C[(R0 + r) * n + c0 + C0 + c] : 0.0f;
  }
  const int kofs = 32 * wave + 8 * (lane >> 5);
  bf16x8 a[3][2][2], b[3][2][2];  // [part][block][step]
  auto ld = [](const uint16_t* p) { return as_bf16x8(*reinterpret_cast<const u32x4*>(p)); };
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int64_t r = std::min<int64_t>(R0 + 32 * t + (lane & 31), rows - 1);
    const int c = std::min(C0 + 32 * t + (lane & 31), N - 1);
    const int64_t ao = r * 128 + kofs;
    const int64_t bo = (int64_t)(c0 + c) * n + b0 + kofs;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      a[0][t][kk] = ld(E0 + ao + 16 * kk);
      a[1][t][kk] = ld(E1 + ao + 16 * kk);
      a[2][t][kk] = ld(E2 + ao + 16 * kk);
      b[0][t][kk] = ld(Mt0 + bo + 16 * kk);
      b[1][t][kk] = ld(Mt1 + bo + 16 * kk);
      b[2][t][kk] = ld(Mt2 + bo + 16 * kk);
    }
  }
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y) {
      f32x16 v = {};
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        v = mfma32x32x16_bf16(a[2][x][kk], b[0][y][kk], v);  // smallest terms first
        v = mfma32x32x16_bf16(a[1][x][kk], b[1][y][kk], v);
        v = mfma32x32x16_bf16(a[0][x][kk], b[2][y][kk], v);
        v = mfma32x32x16_bf16(a[1][x][kk], b[0][y][kk], v);
        v = mfma32x32x16_bf16(a[0][x][kk], b[1][y][kk], v);
        v = mfma32x32x16_bf16(a[0][x][kk], b[0][y][kk], v);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) red[wave][32 * x + acc_row(i, lane)][32 * y + (lane & 31)] = v[i];
    }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int e = tid + 256 * q, r = e >> 6, c = e & 63;
    if (R0 + r < rows && C0 + c < N)
      C[(R0 + r) * n + c0 + C0 + c] = cv[q] + (((red[0][r][c] + red[1][r][c]) + red[2][r][c]) + red[3][r][c]);
  }
}

}  // namespace wr

using namespace wr;

static constexpr int kBatch = 128;

static size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

struct GptqLayout {
  size_t M, C, E[3], Mt[3], total;
};

static GptqLayout gptq_layout(int64_t rows, int64_t n) {
  GptqLayout l{};
  size_t off = align256(wr_factor_ws_bytes(n));  // factorisation scratch (fp64) at the start
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align256(bytes);
    return o;
  };
  l.M = take((size_t)n * n * 4);                                       // M, fp32
  l.C = take((size_t)rows * n * 4);                                    // corrections C
  for (int i = 0; i < 3; ++i) l.E[i] = take((size_t)rows * kBatch * 2);  // batch errors, bf16 parts
  for (int i = 0; i < 3; ++i) l.Mt[i] = take((size_t)n * n * 2);          // M transposed, bf16 parts
  l.total = off;
  return l;
}

size_t wr_gptq_ws_bytes(int64_t rows, int64_t n) { return gptq_layout(rows, n).total; }

template <int P, int G>
static void launch_panel(hipStream_t st, const void* W, int w_dtype, int64_t rows, int n, int64_t ldw, const float* Mm,
                         const uint8_t* bits, int b0, int ncols, float* Cb, uint16_t* const* E, uint8_t* codes,
                         uint16_t* scales, const int32_t* dev_info) {
  const unsigned grid = (unsigned)((rows + (256 / P) - 1) / (256 / P));
  hipLaunchKernelGGL((sweep_panel_kernel<P, kBatch, G>), dim3(grid), dim3(256), 0, st, W, w_dtype, rows, n, ldw, Mm,
                     bits, b0, ncols, Cb, E[0], E[1], E[2], codes, scales, dev_info);
}

template <int P>
static int launch_panel_g(hipStream_t st, int G, const void* W, int w_dtype, int64_t rows, int n, int64_t ldw,
                          const float* Mm, const uint8_t* bits, int b0, int ncols, float* Cb, uint16_t* const* E,
                          uint8_t* codes, uint16_t* scales, const int32_t* dev_info) {
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
  const GptqLayout lay = gptq_layout(rows, n64);
  if (ctx->ws_bytes < lay.total) return WR_EWORKSPACE;
  const int n = (int)n64;
  hipStream_t st = ctx->stream;
  char* ws = static_cast<char*>(ctx->ws);
  void* fws = ws;
  float* Mm = reinterpret_cast<float*>(ws + lay.M);
  float* Cb = reinterpret_cast<float*>(ws + lay.C);
  uint16_t* E[3];
  uint16_t* Mt[3];
  for (int i = 0; i < 3; ++i) {
    E[i] = reinterpret_cast<uint16_t*>(ws + lay.E[i]);
    Mt[i] = reinterpret_cast<uint16_t*>(ws + lay.Mt[i]);
  }

  hipLaunchKernelGGL(sweep_set_int_kernel, dim3(1), dim3(1), 0, st, dev_info, 0);
  WR_CHECK_LAUNCH();
  if (rows > 0) {
    hipLaunchKernelGGL(check_finite_kernel, dim3((unsigned)rows), dim3(256), 0, st, W, w_dtype, rows, n, ldw, dev_info);
    WR_CHECK_LAUNCH();
  }
  int rc = wr_factor_m(st, H, ldh, n, fws, Mm, dev_info);
  if (rc) return rc;
  if (rows == 0) return WR_OK;
  hipLaunchKernelGGL(zero_f32_kernel, dim3(1024), dim3(256), 0, st, Cb, (int64_t)rows * n);
  WR_CHECK_LAUNCH();
  if (n > kBatch) {
    const unsigned nt = (unsigned)((n + 63) / 64);
    hipLaunchKernelGGL(split_mt_kernel, dim3(nt, nt), dim3(256), 0, st, Mm, n, Mt[0], Mt[1], Mt[2], dev_info);
    WR_CHECK_LAUNCH();
  }
  for (int b0 = 0; b0 < n; b0 += kBatch) {
    const int ncols = std::min(kBatch, n - b0);
    rc = launch_panel_g<16>(st, group, W, w_dtype, rows, n, ldw, Mm, bits, b0, ncols, Cb, E, codes, scales, dev_info);
    if (rc) return rc;
    const int rest = n - b0 - ncols;
    if (rest > 0) {  // ncols == kBatch here: only the last batch can be short
      const dim3 grid((unsigned)((rest + 63) / 64), (unsigned)((rows + 63) / 64));
      hipLaunchKernelGGL(trail_s6_kernel, grid, dim3(256), 0, st, rows, rest, n, b0, b0 + ncols, E[0], E[1], E[2],
                         Mt[0], Mt[1], Mt[2], Cb, dev_info);
      WR_CHECK_LAUNCH();
    }
  }
  return WR_OK;
}
