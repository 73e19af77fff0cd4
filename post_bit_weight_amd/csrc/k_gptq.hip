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

// The same test on 16-byte vectors (8 bf16 or 4 fp32 values) over the whole matrix, for rows
// of a multiple of 16 bytes at 16-byte aligned starts.
__global__ __launch_bounds__(256) void check_finite_vec_kernel(const void* __restrict__ W, int w_dtype, int64_t rows,
                                                               int n, int64_t ldw, int32_t* __restrict__ dev_info) {
  const int per = w_dtype == WR_BF16 ? 8 : 4;  // values per vector
  const int64_t nv = n / per, total = rows * nv;
  const int64_t ldv = ldw / per;  // row stride in vectors
  const u32x4* V = static_cast<const u32x4*>(W);
  bool bad = false;
  for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < total; k += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = k / nv;
    const u32x4 v = V[r * ldv + (k - r * nv)];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (w_dtype == WR_BF16) {
        bad |= !(fabsf(__uint_as_float(v[q] << 16)) <= 3.0e38f);
        bad |= !(fabsf(__uint_as_float(v[q] & 0xFFFF0000u)) <= 3.0e38f);
      } else {
        bad |= !(fabsf(__uint_as_float(v[q])) <= 3.0e38f);
      }
    }
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

// Block-start substitution of the sweep panel, x = M_bb^-T c_b (the corrections a block's columns will
// receive from the block's own earlier columns, for the block's scale), as a product with the
// precomputed Y_b = (I + U_b^T)^-1 (U_b the strictly upper part of M's diagonal G x G block b; Y_b is
// unit lower triangular) instead of a serial chain of G dependent steps.  Y_b's strictly lower part
// is stored by columns, column k holding Y[k + 1 .. G - 1][k] from offset sub_col(k), and each block
// at a stride of sub_stride(G) floats (groups of up to 64 columns).
__host__ __device__ constexpr int sub_col(int k, int G) { return k * (2 * G - k - 1) / 2; }
__host__ __device__ constexpr int sub_stride(int G) { return G == 32 ? 512 : 2048; }

template <int G>
__global__ __launch_bounds__(G) void sub_inverse_kernel(const float* __restrict__ M, int n, float* __restrict__ Y,
                                                        const int32_t* __restrict__ dev_info) {
  __shared__ float sU[G][G + 1];   // sU[i][j] = M[b0 + j][b0 + i] for j < i, else 0 (M is fp32)
  __shared__ double sY[G][G + 1];  // column k of Y_b in sY[.][k]
  if (*dev_info != 0) return;
  const int b0 = blockIdx.x * G, k = threadIdx.x;
  for (int e = k; e < G * G; e += G) {
    const int r = e / G, c = e % G;
    sU[c][r] = r < c ? M[(int64_t)(b0 + r) * n + b0 + c] : 0.0f;
  }
  __syncthreads();
  // column k: y_i = 0 (i < k), 1 (i = k), -sum_{j < i} U^T[i][j] y_j (i > k), in fp64
  for (int i = 0; i < G; ++i) {
    double acc = 0.0;
    for (int j = 0; j < i; ++j) acc = fma((double)sU[i][j], sY[j][k], acc);
    sY[i][k] = i < k ? 0.0 : (i == k ? 1.0 : -acc);
  }
  __syncthreads();
  float* dst = Y + (size_t)blockIdx.x * sub_stride(G);
  for (int e = k; e < G * G; e += G) {
    const int i = e / G, kk = e % G;
    if (kk < i) dst[sub_col(kk, G) + i - kk - 1] = (float)sY[i][kk];
  }
}

// Lazy batches of BATCH columns: without GROUP the one batch at b0first (gcols <= BATCH valid
// columns), with GROUP the batches of gcols columns from b0first one after the other.  For a
// batch at b0 with kprev columns of its group before it, the errors of those columns (E0g..E2g:
// three bf16 parts, leading dimension lde, slot kprev) are first applied to the batch's
// corrections, C_b += E M[b0 - kprev.., b0..] with M's transposed bf16 parts Mt0..Mt2, on the
// bf16 matrix cores; Cbuf holds the corrections from the groups before.  The batch's errors go
// to its slot.  kprev0: the group's columns before the launch's first batch.
template <int P, int BATCH, int G, bool GROUP>
__global__ __launch_bounds__(256) void sweep_panel_kernel(const void* __restrict__ W, int w_dtype, int64_t rows,
                                                          int n, int64_t ldw, const float* __restrict__ M,
                                                          const uint8_t* __restrict__ bits, int b0first,
                                                          int gcols, float* __restrict__ Cbuf, int lde, int kprev0,
                                                          uint16_t* __restrict__ E0g,
                                                          uint16_t* __restrict__ E1g, uint16_t* __restrict__ E2g,
                                                          const uint16_t* __restrict__ Mt0,
                                                          const uint16_t* __restrict__ Mt1,
                                                          const uint16_t* __restrict__ Mt2,
                                                          uint8_t* __restrict__ codes, uint16_t* __restrict__ scales,
                                                          const float* __restrict__ Ysub, int use_inv,
                                                          const int32_t* __restrict__ dev_info) {
  constexpr int S = BATCH / P;       // columns per lane
  constexpr int NBLK = BATCH / G;    // blocks per batch
  constexpr int SB = G / P;          // columns per lane per block
  constexpr int R = 256 / P;         // rows per workgroup
  __shared__ __attribute__((aligned(16))) float Ms[BATCH * BATCH];  // [k][p][slot]
  __shared__ __attribute__((aligned(16))) float La[R * BATCH];      // earlier errors of the group, [row][col]
  if (*dev_info != 0) return;
  // With GROUP the launch takes the batches of its group one after the other (a batch reads back
  // only the errors this workgroup's own rows wrote in the earlier batches, behind the barrier that
  // starts the batch); otherwise it takes the one batch at b0first.  kprev0: the columns of the
  // group before the launch's first batch.
  const int nbat = GROUP ? (gcols + BATCH - 1) / BATCH : 1;
#pragma unroll 1
  for (int ib = 0; ib < nbat; ++ib) {
  const int bb = BATCH * ib;
  // with GROUP the thread index passes through an empty asm each batch, so that nothing computed
  // from it (row addresses) is hoisted out of the loop and held in registers across the batches
  int tidv = (int)threadIdx.x;
  if constexpr (GROUP) asm volatile("" : "+v"(tidv));
  const int tid = tidv;
  const int p = tid % P;
  const int64_t row = (int64_t)blockIdx.x * R + tid / P;
  const bool active = row < rows;
  const int b0 = b0first + bb, ncols = min(BATCH, gcols - bb), kprev = kprev0 + bb;
  uint16_t* const E0 = E0g + kprev;
  uint16_t* const E1 = E1g + kprev;
  uint16_t* const E2 = E2g + kprev;
  if (ib > 0) __syncthreads();  // every lane is done with Ms and La, and the errors are written
  // groups of up to 64 columns, with use_inv (many rows: the serial chain would dominate): the batch's
  // Y blocks, fetched now and staged in LDS before each block (the first in La's space once La is
  // read, later ones in the rows of Ms the previous block used)
  constexpr bool kInv = G <= 64;
  constexpr int YPT = kInv ? sub_stride(G) / 256 : 1;  // floats per thread and block
  float yreg[NBLK][YPT];
  if (kInv && use_inv) {
#pragma unroll
    for (int blk = 0; blk < NBLK; ++blk)
#pragma unroll
      for (int u = 0; u < YPT; ++u)
        yreg[blk][u] = blk * G < ncols ? Ysub[(size_t)(b0 / G + blk) * sub_stride(G) + tid * YPT + u] : 0.0f;
  }

  if (kprev > 0) {
    // wave w: columns 32 w .. 32 w + 31 as two 16 x 16 blocks on v_mfma_f32_16x16x32_bf16
    // (operand lane l supplies row/column l % 16 at k = 8 (l / 16) .. +7; result v of lane l
    // is row 4 (l / 16) + v), the errors and M as three bf16 parts each, the six part
    // products with i + j <= 2 summed smallest first.
    static_assert(R == 16 && BATCH == 128, "16 rows x 128 columns: two 16 x 16 blocks per wave");
    const int lane = tid & 63, wave = tid >> 6, li = lane & 15, lk = lane >> 4;
    const int64_t er = std::min<int64_t>((int64_t)blockIdx.x * R + li, rows - 1);
    const int64_t eo = er * lde - kprev + 8 * lk;  // relative to this batch's slot
    int64_t mo[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int col = std::min(32 * wave + 16 * t + li, ncols - 1);
      mo[t] = (int64_t)(b0 + col) * n + (b0 - kprev) + 8 * lk;
    }
    auto ld = [](const uint16_t* q) { return as_bf16x8(*reinterpret_cast<const u32x4*>(q)); };
    f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    // one batch (128 k, four 32-wide steps) at a time: all of its loads are issued before
    // its MFMAs, so each batch costs one memory round trip
    for (int kb = 0; kb < kprev; kb += 128) {
      bf16x8 ea[4][3], mb[4][3][2];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int k0 = kb + 32 * u;
        ea[u][0] = ld(E0 + eo + k0);
        ea[u][1] = ld(E1 + eo + k0);
        ea[u][2] = ld(E2 + eo + k0);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          mb[u][0][t] = ld(Mt0 + mo[t] + k0);
          mb[u][1][t] = ld(Mt1 + mo[t] + k0);
          mb[u][2][t] = ld(Mt2 + mo[t] + k0);
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          f32x4 v = acc[t];
          v = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ea[u][2], mb[u][0][t], v, 0, 0, 0);
          v = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ea[u][1], mb[u][1][t], v, 0, 0, 0);
          v = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ea[u][0], mb[u][2][t], v, 0, 0, 0);
          v = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ea[u][1], mb[u][0][t], v, 0, 0, 0);
          v = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ea[u][0], mb[u][1][t], v, 0, 0, 0);
          v = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ea[u][0], mb[u][0][t], v, 0, 0, 0);
          acc[t] = v;
        }
    }
    const bool c0ok = 32 * wave + li < ncols, c1ok = 32 * wave + 16 + li < ncols;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      La[(4 * lk + v) * BATCH + 32 * wave + li] = c0ok ? acc[0][v] : 0.0f;
      La[(4 * lk + v) * BATCH + 32 * wave + 16 + li] = c1ok ? acc[1][v] : 0.0f;
    }
  }
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
  if (kprev > 0) {
#pragma unroll
    for (int i = 0; i < S; ++i) c[i] += La[(tid / P) * BATCH + p + P * i];
  }
  if (kInv && use_inv) {
    __syncthreads();  // La has been read
#pragma unroll
    for (int u = 0; u < YPT; ++u) La[tid * YPT + u] = yreg[0][u];
    __syncthreads();
  }

  static_for<0, NBLK>([&](auto BLK) {
    constexpr int blk = BLK;
    sc[blk] = 0.0f;
    if (blk * G >= ncols) return;  // uniform
    // push-form values at the block start: x = M_bb^-T c_b
    float x[SB];
#pragma unroll
    for (int q = 0; q < SB; ++q) x[q] = c[blk * SB + q];
    if (kInv && use_inv) {
      // x_i = c_i + sum_{k < i} Y[i][k] c_k, k in order; lane p's columns i = p + P q
      const float* Yl = blk == 0 ? La : Ms + (blk - 1) * G * BATCH;
      static_for<0, G>([&](auto KK) {
        constexpr int k = KK;
        const float ck = group_bcast<P, k % P>(c[blk * SB + k / P]);
#pragma unroll
        for (int q = k / P; q < SB; ++q) {
          const int i = p + P * q;
          if (i > k) x[q] = fmaf(Yl[sub_col(k, G) + i - k - 1], ck, x[q]);
        }
      });
    } else {
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
    }
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
    if constexpr (kInv && blk + 1 < NBLK) {
      if (use_inv && (blk + 1) * G < ncols) {  // uniform
        __syncthreads();  // every lane is done with Ms's rows of this block
#pragma unroll
        for (int u = 0; u < YPT; ++u) Ms[blk * G * BATCH + tid * YPT + u] = yreg[blk + 1][u];
        __syncthreads();
      }
    }
  });

  if (active) {
#pragma unroll
    for (int i = 0; i < S; ++i) {
      const int col = p + P * i;
      if (col < ncols) {
        codes[row * n + b0 + col] = code[i];
        const int64_t e = row * lde + col;
        split3(d[i], E0[e], E1[e], E2[e]);
      }
    }
    if (p == 0) {
#pragma unroll
      for (int blk = 0; blk < NBLK; ++blk)
        if (blk * G < ncols) scales[row * (n / G) + (b0 / G) + blk] = f32_to_f16_bits_clamped(sc[blk]);
    }
  }
  }  // batches
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
  if (n % 8 == 0) {  // eight consecutive output columns per thread: one 16-byte store per plane
    for (int e = tid; e < 64 * 8; e += 256) {
      const int j = e >> 3, i0 = 8 * (e & 7);  // output row c0 + j, columns k0 + i0 .. + 7
      if (c0 + j < n && k0 + i0 < n) {
        uint16_t p[3][8];
#pragma unroll
        for (int q = 0; q < 8; ++q) split3(t[i0 + q][j], p[0][q], p[1][q], p[2][q]);
        const int64_t o = (int64_t)(c0 + j) * n + k0 + i0;
        uint16_t* dst[3] = {Mt0, Mt1, Mt2};
#pragma unroll
        for (int q = 0; q < 3; ++q) {
          u32x4 w;
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) w[e2] = (uint32_t)p[q][2 * e2] | ((uint32_t)p[q][2 * e2 + 1] << 16);
          *reinterpret_cast<u32x4*>(dst[q] + o) = w;
        }
      }
    }
    return;
  }
  for (int e = tid; e < 64 * 64; e += 256) {
    const int j = e >> 6, i = e & 63;  // output row c0 + j, column k0 + i
    if (c0 + j < n && k0 + i < n) {
      const int64_t o = (int64_t)(c0 + j) * n + k0 + i;
      split3(t[i][j], Mt0[o], Mt1[o], Mt2[o]);
    }
  }
}

typedef __attribute__((address_space(3))) char tw_lds_char;

// Wave-wide LDS DMA: lane l copies 16 bytes from sbase + voff to LDS byte m0 + 16 l (inline
// assembly so that the compiler does not wait for it before unrelated LDS reads; completion
// is awaited with tw_vm_wait).  The M0 write needs one wait state.
__device__ __forceinline__ void tw_dma16(const void* sbase, uint32_t voff, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %2" ::"v"(voff), "s"(m0), "s"(sbase)
               : "memory", "m0");
}
template <int N>
__device__ __forceinline__ void tw_vm_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void tw_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

constexpr int TW_R = 256;                    // output tile rows (weight rows)
constexpr int TW_C = 128;                    // output tile columns
constexpr int TW_KC = 32;                    // k per stage
constexpr int TW_EPLANE = TW_R * TW_KC * 2;  // one bf16 part of the E tile: 16 KB
constexpr int TW_MPLANE = TW_C * TW_KC * 2;  // one bf16 part of the M tile: 8 KB
constexpr int TW_STAGE = 3 * TW_EPLANE + 3 * TW_MPLANE;  // E0..2 then Mt0..2: 72 KB, two stages
constexpr int TW_DMA = TW_STAGE / 1024 / 8;  // 1 KB DMAs per wave per stage: 9
constexpr int TW_XCD = 8;                    // workgroups are dispatched round-robin over 8 XCDs

// 16-byte unit (row r, k-octet q) of a tile of 32 bf16 columns: sixteen consecutive rows at one
// octet fall on sixteen distinct 16-byte bank groups of a 256-byte line.
__device__ __forceinline__ int tw_unit(int r, int q) { return r * 4 + (q ^ ((r >> 2) & 3)); }

static unsigned trail_wide_grid(int64_t rows, int N) {
  const int64_t tiles = (rows + TW_R - 1) / TW_R * ((N + TW_C - 1) / TW_C);
  return (unsigned)((tiles + TW_XCD - 1) / TW_XCD * TW_XCD);
}

// The wide trailing update C[r][c0 + c] += sum_{k < K} E[r][k] M[b0 + k][c0 + c] (K a multiple
// of 32; E and M as three bf16 planes each, E_i rows x K with leading dimension lde, Mt_i n x n
// transposed; the six part products with i + j <= 2, smallest first).  256 x 128 tile per
// workgroup of eight waves (two per SIMD); wave w owns rows 64 (w / 2).., columns 64 (w % 2).. as
// 2 x 2 blocks of 32 x 32.  The operand tiles of a 32-wide k stage go to LDS by DMA into one of two
// stages while the other is multiplied.  Tiles are numbered with the column tiles of one row tile
// consecutive, and each XCD takes a contiguous range of them, so the workgroups it runs at once
// share E rows and M columns.
__global__ __launch_bounds__(512) void trail_wide_kernel(int64_t rows, int N, int n, int K, int b0, int c0,
                                                         const uint16_t* __restrict__ E0,
                                                         const uint16_t* __restrict__ E1,
                                                         const uint16_t* __restrict__ E2, int lde,
                                                         const uint16_t* __restrict__ Mt0,
                                                         const uint16_t* __restrict__ Mt1,
                                                         const uint16_t* __restrict__ Mt2, float* __restrict__ C,
                                                         const int32_t* __restrict__ dev_info) {
  extern __shared__ __attribute__((aligned(1024))) char tw_lds[];
  if (*dev_info != 0) return;
  int64_t R0;
  int C0;
  {
    const int gx = (N + TW_C - 1) / TW_C;
    const int tiles = (int)((rows + TW_R - 1) / TW_R) * gx, bid = blockIdx.x;
    const int q = tiles / TW_XCD, rem = tiles % TW_XCD, x = bid % TW_XCD, slot = bid / TW_XCD;
    if (slot >= q + (x < rem ? 1 : 0)) return;  // the grid is rounded up to a multiple of 8
    const int t = x * q + min(x, rem) + slot;
    R0 = (int64_t)(t / gx) * TW_R;
    C0 = (t % gx) * TW_C;
  }
  const tw_lds_char* lds = (const tw_lds_char*)tw_lds;
  const uint32_t lds_base = (uint32_t)(uintptr_t)lds;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rmax = (int)std::min<int64_t>(rows - 1 - R0, TW_R - 1);
  const int cmax = std::min(N - 1 - C0, TW_C - 1);
  // DMA q (0..71 per stage) fills LDS bytes [1024 q, +1024): q < 48 the E plane q / 16 (its 1 KB
  // part q % 16), else the M plane (q - 48) / 8 (part (q - 48) % 8).  Wave w issues q = w + 8 i.
  uint32_t voff[TW_DMA];
#pragma unroll
  for (int i = 0; i < TW_DMA; ++i) {
    const int q = wave + 8 * i;
    const int u = (q < 48 ? (q & 15) : ((q - 48) & 7)) * 64 + lane, r = u >> 2;
    const int oct = (u & 3) ^ ((r >> 2) & 3);
    voff[i] = q < 48 ? (uint32_t)((std::min(r, rmax) * (int64_t)lde + 8 * oct) * 2)
                     : (uint32_t)(((int64_t)std::min(r, cmax) * n + 8 * oct) * 2);
  }
  auto issue = [&](int k0, int slot) {
    const uint32_t base = lds_base + slot * TW_STAGE;
    const int64_t eo = R0 * lde + k0;
    const int64_t mo = (int64_t)(c0 + C0) * n + b0 + k0;
#pragma unroll
    for (int i = 0; i < TW_DMA; ++i) {
      const int q = wave + 8 * i;
      const uint16_t* src = q < 16 ? E0 + eo : q < 32 ? E1 + eo : q < 48 ? E2 + eo
                          : q < 56 ? Mt0 + mo : q < 64 ? Mt1 + mo : Mt2 + mo;
      tw_dma16(src, voff[i], base + q * 1024);
    }
  };
  const int wr0 = 64 * (wave >> 1), wc0 = 64 * (wave & 1);
  f32x16 acc[2][2];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y) acc[x][y] = f32x16{};
  auto fragE = [&](const tw_lds_char* st, int plane, int r, int q) {
    const u32x4 v = *(const __attribute__((address_space(3))) u32x4*)(st + plane * TW_EPLANE + tw_unit(r, q) * 16);
    return as_bf16x8(v);
  };
  auto fragM = [&](const tw_lds_char* st, int plane, int r, int q) {
    const u32x4 v = *(const __attribute__((address_space(3))) u32x4*)(st + 3 * TW_EPLANE + plane * TW_MPLANE +
                                                                       tw_unit(r, q) * 16);
    return as_bf16x8(v);
  };
  const int nst = K / TW_KC;
  issue(0, 0);
  for (int stg = 0; stg < nst; ++stg) {
    tw_vm_wait<0>();
    tw_barrier();  // stage stg is in LDS for every wave, and every wave is done with stage stg - 1
    if (stg + 1 < nst) issue(TW_KC * (stg + 1), (stg + 1) & 1);  // into the other stage
    const tw_lds_char* st = lds + (stg & 1) * TW_STAGE;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int q = 2 * ks + (lane >> 5);
      bf16x8 a[3][2], b[3][2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int p = 0; p < 3; ++p) {
          a[p][t] = fragE(st, p, wr0 + 32 * t + (lane & 31), q);
          b[p][t] = fragM(st, p, wc0 + 32 * t + (lane & 31), q);
        }
      }
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y) {
          f32x16 v = acc[x][y];
          v = mfma32x32x16_bf16(a[2][x], b[0][y], v);  // smallest terms first
          v = mfma32x32x16_bf16(a[1][x], b[1][y], v);
          v = mfma32x32x16_bf16(a[0][x], b[2][y], v);
          v = mfma32x32x16_bf16(a[1][x], b[0][y], v);
          v = mfma32x32x16_bf16(a[0][x], b[1][y], v);
          v = mfma32x32x16_bf16(a[0][x], b[0][y], v);
          acc[x][y] = v;
        }
    }
  }
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y) {
      const int c = C0 + wc0 + 32 * y + (lane & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t r = R0 + wr0 + 32 * x + acc_row(v, lane);
        if (r < rows && c < N) C[r * n + c0 + c] += acc[x][y][v];
      }
    }
}

}  // namespace wr

using namespace wr;

static constexpr int kBatch = 128;
static constexpr int kSuper = 4 * kBatch;  // columns whose errors one wide trailing update applies
static constexpr int64_t kInvRows = 4096;  // rows from which the panels use the precomputed inverses
static constexpr int64_t kGroupRows = 4096;  // rows below which one panel launch takes a group of batches

static size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

struct GptqLayout {
  size_t M, C, E[3], Mt[3], Y, total;
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
  for (int i = 0; i < 3; ++i) l.E[i] = take((size_t)rows * kSuper * 2);  // errors of 4 batches, bf16 parts
  for (int i = 0; i < 3; ++i) l.Mt[i] = take((size_t)n * n * 2);          // M transposed, bf16 parts
  l.Y = take((size_t)n * 32 * 4);  // the blocks' Y_b (n / 64 x 2048 or n / 32 x 512 floats)
  l.total = off;
  return l;
}

size_t wr_gptq_ws_bytes(int64_t rows, int64_t n) { return gptq_layout(rows, n).total; }

// Panels of the group of up to four batches at s0 (a multiple of kSuper), gcols columns.  With
// few rows (fewer workgroups than CUs, so occupancy does not matter) one launch takes the whole
// group: a quarter of the launches on the serial chain, each of which waits for free CUs when other
// streams share the chip.  With many rows one launch per batch keeps the kernel at two waves per
// SIMD (the loop over batches needs more registers).
template <int P, int G>
static void launch_panel(hipStream_t st, const void* W, int w_dtype, int64_t rows, int n, int64_t ldw, const float* Mm,
                         const uint8_t* bits, int s0, int gcols, float* Cb, uint16_t* const* E, uint16_t* const* Mt,
                         uint8_t* codes, uint16_t* scales, const float* Ysub, const int32_t* dev_info) {
  const unsigned grid = (unsigned)((rows + (256 / P) - 1) / (256 / P));
  const int use_inv = Ysub != nullptr ? 1 : 0;
  if (rows < kGroupRows) {
    hipLaunchKernelGGL((sweep_panel_kernel<P, kBatch, G, true>), dim3(grid), dim3(256), 0, st, W, w_dtype, rows, n, ldw,
                       Mm, bits, s0, gcols, Cb, kSuper, 0, E[0], E[1], E[2], Mt[0], Mt[1], Mt[2], codes, scales, Ysub,
                       use_inv, dev_info);
    return;
  }
  for (int bb = 0; bb < gcols; bb += kBatch)
    hipLaunchKernelGGL((sweep_panel_kernel<P, kBatch, G, false>), dim3(grid), dim3(256), 0, st, W, w_dtype, rows, n,
                       ldw, Mm, bits, s0 + bb, std::min(kBatch, gcols - bb), Cb, kSuper, bb, E[0], E[1], E[2], Mt[0],
                       Mt[1], Mt[2], codes, scales, Ysub, use_inv, dev_info);
}

template <int P>
static int launch_panel_g(hipStream_t st, int G, const void* W, int w_dtype, int64_t rows, int n, int64_t ldw,
                          const float* Mm, const uint8_t* bits, int s0, int gcols, float* Cb, uint16_t* const* E,
                          uint16_t* const* Mt, uint8_t* codes, uint16_t* scales, const float* Ysub,
                          const int32_t* dev_info) {
  switch (G) {
    case 32: launch_panel<P, 32>(st, W, w_dtype, rows, n, ldw, Mm, bits, s0, gcols, Cb, E, Mt, codes, scales, Ysub, dev_info); break;
    case 64: launch_panel<P, 64>(st, W, w_dtype, rows, n, ldw, Mm, bits, s0, gcols, Cb, E, Mt, codes, scales, Ysub, dev_info); break;
    case 128: launch_panel<P, 128>(st, W, w_dtype, rows, n, ldw, Mm, bits, s0, gcols, Cb, E, Mt, codes, scales, Ysub, dev_info); break;
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
  float* Ysub = reinterpret_cast<float*>(ws + lay.Y);

  hipLaunchKernelGGL(sweep_set_int_kernel, dim3(1), dim3(1), 0, st, dev_info, 0);
  WR_CHECK_LAUNCH();
  if (rows > 0) {
    const int esz = w_dtype == WR_BF16 ? 2 : 4;
    if ((n * esz) % 16 == 0 && (ldw * esz) % 16 == 0 && (reinterpret_cast<uintptr_t>(W) & 15) == 0)
      hipLaunchKernelGGL(check_finite_vec_kernel, dim3(1024), dim3(256), 0, st, W, w_dtype, rows, n, ldw, dev_info);
    else
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
  // The block-start substitution as a product with precomputed inverses pays where many rows keep
  // the chip busy (4096 rows and more: 148 -> 131 us per panel at 25600 rows); with few rows the
  // panel is latency-bound and the serial chain is shorter (23 us against 28 us at 2560 rows).
  if (rows < kInvRows || group > 64) {
    Ysub = nullptr;
  } else {
    if (group == 64)
      hipLaunchKernelGGL(sub_inverse_kernel<64>, dim3((unsigned)(n / 64)), dim3(64), 0, st, Mm, n, Ysub, dev_info);
    else
      hipLaunchKernelGGL(sub_inverse_kernel<32>, dim3((unsigned)(n / 32)), dim3(32), 0, st, Mm, n, Ysub, dev_info);
    WR_CHECK_LAUNCH();
  }
  // Batches go in groups of four (kSuper columns), one panel launch per group.  A batch
  // applies the errors of the earlier batches of its group to its own columns; after the
  // group its errors reach every column after it at once (K = 512), so the corrections C of
  // the far columns are read and written once per group, not per batch.
  for (int s0 = 0; s0 < n; s0 += kSuper) {
    const int s1 = std::min(s0 + kSuper, n);
    rc = launch_panel_g<16>(st, group, W, w_dtype, rows, n, ldw, Mm, bits, s0, s1 - s0, Cb, E, Mt, codes, scales, Ysub,
                            dev_info);
    if (rc) return rc;
    if (s1 < n) {  // a group followed by more columns is full (s1 - s0 == kSuper)
      if (!lds_limit(reinterpret_cast<const void*>(trail_wide_kernel), 2 * TW_STAGE)) return WR_EHIP;
      hipLaunchKernelGGL(trail_wide_kernel, dim3(trail_wide_grid(rows, n - s1)), dim3(512), 2 * TW_STAGE, st, rows,
                         n - s1, n, kSuper, s0, s1, E[0], E[1], E[2], kSuper, Mt[0], Mt[1], Mt[2], Cb, dev_info);
      WR_CHECK_LAUNCH();
    }
  }
  return WR_OK;
}
