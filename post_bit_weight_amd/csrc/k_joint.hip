// Joint least-squares block scales with a prior, and the wring.
//
// Wringer model cards, "Recipe" / "Why the solver changed": scales by a joint
// least-squares closed form with a prior (lambda = 0.01); the wring rounds the
// watered weights W' = W_hat + (alpha/r) B A to the nearest point of the same
// grid and re-solves the scales against W'.  Agents-A1 card, "Honest
// caveats": scales projected to fp16 at solve time.
//
// Per row, with levels l_j = 2 c_j - L, Q[j, block(j)] = l_j, G = Q^T H Q,
// h = Q^T H t and mu = trace(G)/nb, the minimiser of
//   (t - Q s)^T H (t - Q s) + lambda mu ||s - s0||^2
// is s = (G + lambda mu I)^-1 (h + lambda mu s0).  G and h are formed on the
// bf16 matrix cores from exact bf16 levels and three-way bf16 splits
// x = x_0 + x_1 + x_2 (24 significant bits, as fp32):
//   G[r][b][c] = sum_{j in b} l_j (H_{b,c} l_c)_j    three passes (H_0, H_1, H_2)
//   h[r][b]    = sum_{j in b} l_j (H t_r)_j          six passes: H_i t_j for i + j <= 2
// with fp32 accumulation.  Both need the full split: a two-way split (16
// bits) is an H perturbed by ~1e-5, and after a Hadamard rotation that moves
// some fp16 scales by two ulps.  The MFMA computes
// D[j][r] = sum_l H[j][l] X[r][l] with j down the accumulator rows, so the
// level-weighted sum over a block's j stays mostly inside a lane.  Each row's
// nb x nb system is then factored and solved in fp64.  (Solving for the step
// s - s0 instead would shrink the error only when the scales move little; the
// joint solve routinely moves them by their own size.)
#include "chol16.hpp"

int wr_gemm_f32(hipStream_t st, int M, int N, int K, const float* A, int64_t lda, const float* B, int64_t ldb,
                bool b_kn, float* C, int64_t ldc, float alpha, bool accumulate, bool lower_tiles,
                const int32_t* dev_info);

namespace wr {

__global__ void set_int_kernel(int32_t* p, int32_t v) { *p = v; }

__global__ void to_f32_kernel(const void* __restrict__ src, int dtype, int64_t count, float* __restrict__ dst) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += (int64_t)gridDim.x * blockDim.x)
    dst[i] = dtype == WR_BF16 ? bf16_bits_to_f32(static_cast<const uint16_t*>(src)[i]) : static_cast<const float*>(src)[i];
}

// T = target, or dequant(codes, scales) when target is null.
__global__ void target_kernel(const void* __restrict__ target, int t_dtype, int64_t ldt, const uint8_t* __restrict__ codes,
                              const uint16_t* __restrict__ scales, const uint8_t* __restrict__ bits, int64_t rows, int n,
                              int group, float* __restrict__ T) {
  const int64_t r = blockIdx.y;
  const int nb = n / group;
  const int L = (1 << bits[r]) - 1;
  for (int j = blockIdx.x * blockDim.x + threadIdx.x; j < n; j += gridDim.x * blockDim.x) {
    float v;
    if (target) {
      v = t_dtype == WR_BF16 ? bf16_bits_to_f32(static_cast<const uint16_t*>(target)[r * ldt + j])
                             : static_cast<const float*>(target)[r * ldt + j];
    } else {
      v = (float)(2 * (int)codes[r * n + j] - L) * f16_bits_to_f32(scales[r * nb + j / group]);
    }
    T[r * n + j] = v;
  }
}

// Optional nearest-point recode on the incoming scales, then exact bf16 levels and the bf16-split target.
__global__ void recode_residual_kernel(const float* __restrict__ T, uint8_t* __restrict__ codes,
                                       const uint16_t* __restrict__ scales, const uint8_t* __restrict__ bits,
                                       int64_t rows, int n, int group, int recode, uint16_t* __restrict__ Lev,
                                       uint16_t* __restrict__ T0, uint16_t* __restrict__ T1, uint16_t* __restrict__ T2,
                                       int32_t* __restrict__ dev_info) {
  const int64_t r = blockIdx.y;
  const int nb = n / group;
  const int L = (1 << bits[r]) - 1;
  bool bad = false;
  for (int j = blockIdx.x * blockDim.x + threadIdx.x; j < n; j += gridDim.x * blockDim.x) {
    const int64_t e = r * n + j;
    const float t = T[e];
    bad |= !(fabsf(t) <= 3.0e38f);
    const float s = f16_bits_to_f32(scales[r * nb + j / group]);
    int c;
    if (recode) {
      c = nearest_code(s > 0.0f ? t / s : 0.0f, L);
      codes[e] = (uint8_t)c;
    } else {
      c = codes[e];
    }
    Lev[e] = (uint16_t)f32_to_bf16_bits((float)(2 * c - L));
    if (T0) split3(t, T0[e], T1[e], T2[e]);
  }
  if (bad) atomicCAS(dev_info, 0, -1);
}

// At[c][k] = A[k][c] (the rank x n adapter factor transposed, bf16 bits).
__global__ void transpose_ab_kernel(const uint16_t* __restrict__ A, int rank, int n, uint16_t* __restrict__ At) {
  const int k = blockIdx.y;
  for (int c = blockIdx.x * blockDim.x + threadIdx.x; c < n; c += gridDim.x * blockDim.x)
    At[(int64_t)c * rank + k] = A[(int64_t)k * n + c];
}

// The target, recode and levels in one pass, for a 64 x 64 tile per workgroup (group 64):
//   t = target (or dequant(codes, scales) when target is null) + scale_ab (B A)[r][c],
// with B A (rank a multiple of 16, bf16 B and At = A^T) on the bf16 matrix cores (exact
// products, fp32 sums); with recode, c = nearest code of t / s on the current scales;
// writes T = t, the level 2 c - L (bf16, exact) and the codes.  A non-finite t sets
// dev_info = -1.  Wave w owns the 32 x 32 block (w / 2, w % 2) of the product, which goes
// through LDS; then thread i handles 16 consecutive columns of tile row i / 4.
__global__ __launch_bounds__(256) void wring_prep_kernel(const void* __restrict__ target, int t_dtype, int64_t ldt,
                                                         const uint16_t* __restrict__ B,
                                                         const uint16_t* __restrict__ At, int rank, float scale_ab,
                                                         const uint8_t* __restrict__ bits, int64_t rows, int n,
                                                         int recode, uint8_t* __restrict__ codes,
                                                         const uint16_t* __restrict__ scales, float* __restrict__ T,
                                                         uint16_t* __restrict__ Lev, int32_t* __restrict__ dev_info) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t R0 = (int64_t)blockIdx.y * 64 + 32 * (wave >> 1);
  const int C0 = blockIdx.x * 64 + 32 * (wave & 1);
  f32x16 acc = {};
  if (rank > 0) {
    const int64_t ra = std::min<int64_t>(R0 + (lane & 31), rows - 1);
    const int ca = std::min(C0 + (lane & 31), n - 1);
    const uint16_t* pa = B + ra * rank + 8 * (lane >> 5);
    const uint16_t* pb = At + (int64_t)ca * rank + 8 * (lane >> 5);
    for (int k0 = 0; k0 < rank; k0 += 64) {
      bf16x8 a[4], b[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bool ok = k0 + 16 * u < rank;
        a[u] = as_bf16x8(ok ? *reinterpret_cast<const u32x4*>(pa + k0 + 16 * u) : u32x4{0u, 0u, 0u, 0u});
        b[u] = as_bf16x8(ok ? *reinterpret_cast<const u32x4*>(pb + k0 + 16 * u) : u32x4{0u, 0u, 0u, 0u});
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) acc = mfma32x32x16_bf16(a[u], b[u], acc);
    }
  }
  // the tile's B A through LDS, so that each thread then works on 16 consecutive columns
  __shared__ float ab[64][65];
  if (rank > 0) {
#pragma unroll
    for (int v = 0; v < 16; ++v) ab[32 * (wave >> 1) + acc_row(v, lane)][32 * (wave & 1) + (lane & 31)] = acc[v];
  }
  __syncthreads();
  const int nb = n / 64;
  const int lr = tid >> 2, lc = 16 * (tid & 3);
  const int64_t r = (int64_t)blockIdx.y * 64 + lr;
  const int c0 = blockIdx.x * 64 + lc;  // 16 columns inside one group of 64 (n % 64 == 0)
  bool bad = false;
  if (r < rows) {
    const int L = (1 << bits[r]) - 1;
    const int64_t e0 = r * n + c0;
    const float s = f16_bits_to_f32(scales[r * nb + (c0 >> 6)]);
    uint8_t cin[16];
    *reinterpret_cast<u32x4*>(cin) = *reinterpret_cast<const u32x4*>(codes + e0);
    float t[16];
    if (target) {
      if (t_dtype == WR_BF16) {
        const uint16_t* tp = static_cast<const uint16_t*>(target) + r * ldt + c0;
#pragma unroll
        for (int i = 0; i < 16; ++i) t[i] = bf16_bits_to_f32(tp[i]);
      } else {
        const float* tp = static_cast<const float*>(target) + r * ldt + c0;
#pragma unroll
        for (int i = 0; i < 16; ++i) t[i] = tp[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) t[i] = (float)(2 * (int)cin[i] - L) * s;
    }
    uint8_t cout[16];
    uint32_t lev[8];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float x = t[i];
      if (rank > 0) x = x + scale_ab * ab[lr][lc + i];
      bad |= !(fabsf(x) <= 3.0e38f);
      const int cd = recode ? nearest_code(s > 0.0f ? x / s : 0.0f, L) : (int)cin[i];
      t[i] = x;
      cout[i] = (uint8_t)cd;
      const uint32_t lb = __float_as_uint((float)(2 * cd - L)) >> 16;  // small odd integer: exact in bf16
      lev[i >> 1] = (i & 1) ? (lev[i >> 1] | (lb << 16)) : lb;
    }
#pragma unroll
    for (int q = 0; q < 16; q += 4) *reinterpret_cast<f32x4*>(T + e0 + q) = f32x4{t[q], t[q + 1], t[q + 2], t[q + 3]};
    *reinterpret_cast<u32x4*>(Lev + e0) = u32x4{lev[0], lev[1], lev[2], lev[3]};
    *reinterpret_cast<u32x4*>(Lev + e0 + 8) = u32x4{lev[4], lev[5], lev[6], lev[7]};
    if (recode) *reinterpret_cast<u32x4*>(codes + e0) = *reinterpret_cast<const u32x4*>(cout);
  }
  if (bad) atomicCAS(dev_info, 0, -1);
}

__global__ void split_h_kernel(const float* __restrict__ H, int64_t ldh, int n, uint16_t* __restrict__ H0,
                               uint16_t* __restrict__ H1, uint16_t* __restrict__ H2) {
  const int64_t i = blockIdx.y;
  for (int j = blockIdx.x * blockDim.x + threadIdx.x; j < n; j += gridDim.x * blockDim.x)
    split3(H[i * ldh + j], H0[i * n + j], H1[i * n + j], H2[i * n + j]);
}

// The same split 8 values per thread: two 16-byte reads, one 16-byte write per plane (n % 8 == 0,
// ldh % 4 == 0, H 16-byte aligned).
__global__ __launch_bounds__(256) void split_h_vec_kernel(const float* __restrict__ H, int64_t ldh, int n,
                                                          uint16_t* __restrict__ H0, uint16_t* __restrict__ H1,
                                                          uint16_t* __restrict__ H2) {
  const int64_t nv = n / 8, total = (int64_t)n * nv;
  for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < total; k += (int64_t)gridDim.x * blockDim.x) {
    const int64_t i = k / nv, j = 8 * (k - i * nv);
    const f32x4 a = *reinterpret_cast<const f32x4*>(H + i * ldh + j);
    const f32x4 b = *reinterpret_cast<const f32x4*>(H + i * ldh + j + 4);
    uint16_t p[3][8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      split3(a[e], p[0][e], p[1][e], p[2][e]);
      split3(b[e], p[0][e + 4], p[1][e + 4], p[2][e + 4]);
    }
    uint16_t* dst[3] = {H0, H1, H2};
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = (uint32_t)p[q][2 * e] | ((uint32_t)p[q][2 * e + 1] << 16);
      *reinterpret_cast<u32x4*>(dst[q] + i * n + j) = w;
    }
  }
}

// One workgroup: 128 rows (four waves of 32) x one block b.  Loops over all column blocks c.
template <int G>
__global__ __launch_bounds__(256) void gram_kernel(const uint16_t* __restrict__ Lev, const uint16_t* __restrict__ T0,
                                                   const uint16_t* __restrict__ T1, const uint16_t* __restrict__ T2,
                                                   int64_t rows, int n, const uint16_t* __restrict__ H0,
                                                   const uint16_t* __restrict__ H1, const uint16_t* __restrict__ H2,
                                                   float* __restrict__ Gm, float* __restrict__ rhs,
                                                   const int32_t* __restrict__ dev_info) {
  constexpr int IB = G / 32;
  constexpr int PITCH = G + 8;
  __shared__ __attribute__((aligned(16))) uint16_t sH[3][G * PITCH];
  if (*dev_info != 0) return;
  const int nb = n / G;
  const int b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t r = (int64_t)blockIdx.x * 128 + wave * 32 + (lane & 31);
  const bool rok = r < rows;
  const int64_t rr = rok ? r : 0;

  float levj[IB][16];
#pragma unroll
  for (int ib = 0; ib < IB; ++ib)
#pragma unroll
    for (int v = 0; v < 16; ++v)
      levj[ib][v] = rok ? bf16_bits_to_f32(Lev[rr * n + b * G + ib * 32 + acc_row(v, lane)]) : 0.0f;

  float rtot[IB][16];
#pragma unroll
  for (int ib = 0; ib < IB; ++ib)
#pragma unroll
    for (int v = 0; v < 16; ++v) rtot[ib][v] = 0.0f;

  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  for (int c = 0; c < nb; ++c) {
    __syncthreads();
    for (int e = tid; e < G * G / 8; e += 256) {
      const int j = e / (G / 8), l8 = (e % (G / 8)) * 8;
      const int64_t src = (int64_t)(b * G + j) * n + c * G + l8;
      *reinterpret_cast<u32x4*>(&sH[0][j * PITCH + l8]) = *reinterpret_cast<const u32x4*>(H0 + src);
      *reinterpret_cast<u32x4*>(&sH[1][j * PITCH + l8]) = *reinterpret_cast<const u32x4*>(H1 + src);
      *reinterpret_cast<u32x4*>(&sH[2][j * PITCH + l8]) = *reinterpret_cast<const u32x4*>(H2 + src);
    }
    __syncthreads();
    const bool doG = c >= b;
    f32x16 accG[IB], accR[IB];
#pragma unroll
    for (int ib = 0; ib < IB; ++ib) {
      accG[ib] = f32x16{};
      accR[ib] = f32x16{};
    }
#pragma unroll
    for (int ks = 0; ks < G / 16; ++ks) {
      const int lk = ks * 16 + 8 * (lane >> 5);
      const int64_t src = rr * n + c * G + lk;
      const bf16x8 t0 = as_bf16x8(rok ? *reinterpret_cast<const u32x4*>(T0 + src) : zero4);
      const bf16x8 t1 = as_bf16x8(rok ? *reinterpret_cast<const u32x4*>(T1 + src) : zero4);
      const bf16x8 t2 = as_bf16x8(rok ? *reinterpret_cast<const u32x4*>(T2 + src) : zero4);
      bf16x8 fL = as_bf16x8(zero4);
      if (doG) fL = as_bf16x8(rok ? *reinterpret_cast<const u32x4*>(Lev + src) : zero4);
#pragma unroll
      for (int ib = 0; ib < IB; ++ib) {
        const int ja = (ib * 32 + (lane & 31)) * PITCH + lk;
        const bf16x8 h0 = as_bf16x8(*reinterpret_cast<const u32x4*>(&sH[0][ja]));
        const bf16x8 h1 = as_bf16x8(*reinterpret_cast<const u32x4*>(&sH[1][ja]));
        const bf16x8 h2 = as_bf16x8(*reinterpret_cast<const u32x4*>(&sH[2][ja]));
        // smallest terms first
        accR[ib] = mfma32x32x16_bf16(h2, t0, accR[ib]);
        accR[ib] = mfma32x32x16_bf16(h1, t1, accR[ib]);
        accR[ib] = mfma32x32x16_bf16(h0, t2, accR[ib]);
        accR[ib] = mfma32x32x16_bf16(h1, t0, accR[ib]);
        accR[ib] = mfma32x32x16_bf16(h0, t1, accR[ib]);
        accR[ib] = mfma32x32x16_bf16(h0, t0, accR[ib]);
        if (doG) {
          accG[ib] = mfma32x32x16_bf16(h2, fL, accG[ib]);
          accG[ib] = mfma32x32x16_bf16(h1, fL, accG[ib]);
          accG[ib] = mfma32x32x16_bf16(h0, fL, accG[ib]);
        }
      }
    }
#pragma unroll
    for (int ib = 0; ib < IB; ++ib)
#pragma unroll
      for (int v = 0; v < 16; ++v) rtot[ib][v] += accR[ib][v];
    if (doG) {
      float part = 0.0f;
#pragma unroll
      for (int ib = 0; ib < IB; ++ib)
#pragma unroll
        for (int v = 0; v < 16; ++v) part = fmaf(levj[ib][v], accG[ib][v], part);
      part += __shfl_xor(part, 32);
      if (lane < 32 && rok) {
        Gm[((size_t)r * nb + b) * nb + c] = part;
        Gm[((size_t)r * nb + c) * nb + b] = part;
      }
    }
  }
  float part = 0.0f;
#pragma unroll
  for (int ib = 0; ib < IB; ++ib)
#pragma unroll
    for (int v = 0; v < 16; ++v) part = fmaf(levj[ib][v], rtot[ib][v], part);
  part += __shfl_xor(part, 32);
  if (lane < 32 && rok) rhs[(size_t)r * nb + b] = part;
}

// ------------------------------------------------------------------ group 64
// With Z = H Q (column c of Z is H restricted to the columns of block c, times the
// levels there), G = Q^T Z and h = Q^T H t = Z^T t.  So one product per block pair,
//   D^(b,c)_j = sum_{k in c} H_jk l_k      (j in block b),
// gives both G[b][c] = sum_{j in b} l_j D_j and block b's share of h_c,
// sum_{j in b} t_j D_j: three bf16 passes (H_0, H_1, H_2 against the exact levels)
// over all block pairs instead of six passes for H t plus three for G.  The shares
// of h_c from the nb blocks b are summed afterwards in a fixed order.

typedef __attribute__((address_space(3))) char lds_char;

// Wave-wide LDS DMA: lane l copies 16 bytes from sbase + voff to LDS byte m0 + 16 l.
// Inline assembly so that the compiler does not wait for it before unrelated LDS
// reads; completion is awaited with vm_wait.  The M0 write needs one wait state.
__device__ __forceinline__ void lh_dma16(const void* sbase, uint32_t voff, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %2" ::"v"(voff), "s"(m0), "s"(sbase)
               : "memory", "m0");
}
template <int N>
__device__ __forceinline__ void lh_vm_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// Barrier the compiler cannot move LDS accesses across; the wave's own LDS reads are
// complete before it.
__device__ __forceinline__ void lh_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

constexpr int LH_ROWS = 256;                     // weight rows per workgroup (64 per wave)
constexpr int LH_PLANE = 64 * 64 * 2;            // one H split tile, 64 x 64 bf16: 8 KB
constexpr int LH_LEV = LH_ROWS * 64 * 2;         // the rows' level tile, 256 x 64 bf16: 32 KB
constexpr int LH_STAGE = 6 * LH_PLANE + LH_LEV;  // two blocks b: 80 KB, two stages fill the LDS
constexpr int LH_DMA = LH_STAGE / 1024 / 8;      // 1 KB DMAs per wave per stage
constexpr int LH_XCD = 8;                        // workgroups are dispatched round-robin over 8 XCDs

// Position of the 16-byte unit (row j, octet q of 64 bf16 columns) in a tile of 128-byte rows:
// eight consecutive rows at one octet fall on eight distinct units of a 128-byte line, and
// sixteen consecutive rows on sixteen of a 256-byte line.
__device__ __forceinline__ int lh_unit(int j, int q) { return 8 * j + (q ^ (j & 7) ^ ((j >> 3) & 1)); }

__device__ __forceinline__ bf16x8 lh_frag(const lds_char* p) {
  const u32x4 v = *(const __attribute__((address_space(3))) u32x4*)p;
  return as_bf16x8(v);
}

// Workgroups of the Gram launch: one per (row tile, pair of blocks b), rounded up to a multiple
// of the XCD count.
static unsigned gram_lh_grid(int64_t rows, int nb) {
  const int64_t tiles = (rows + LH_ROWS - 1) / LH_ROWS * ((nb + 1) / 2);
  return (unsigned)((tiles + LH_XCD - 1) / LH_XCD * LH_XCD);
}

// One workgroup: 256 weight rows x the blocks b = 2 bp, 2 bp + 1, looping over the column blocks
// c.  Per c the three H split tiles H_i[b, c] of both blocks and the rows' levels on c are DMAed
// into one of two LDS stages while the other is multiplied; waves 4 h .. 4 h + 3 take block
// 2 bp + h, wave w multiplying into D (64 j x its 64 rows, four 32 x 32 MFMA blocks) and reducing
// D with the rows' levels and targets on its block (kept in registers).  The level tile serves
// both blocks: per weight row and block pair the levels are read once, per block pair and 256
// rows the H stripes once.  Tiles are numbered with the row tiles of one pair consecutive, and
// each XCD takes a contiguous range of them, so the workgroups it runs at once share the H
// stripes.  Outputs: G[r][b][c] = G[r][c][b] for b <= c; hp[b][c][r] = block b's share of h_c.
// With nb odd the second block of the last pair repeats the first and writes nothing.
__global__ __launch_bounds__(512) void gram_lh_kernel(const uint16_t* __restrict__ Lev, const float* __restrict__ T,
                                                      int64_t rows, int n, const uint16_t* __restrict__ H0,
                                                      const uint16_t* __restrict__ H1, const uint16_t* __restrict__ H2,
                                                      float* __restrict__ Gm, float* __restrict__ hp,
                                                      const int32_t* __restrict__ dev_info) {
  extern __shared__ __attribute__((aligned(1024))) char lh_lds[];
  if (*dev_info != 0) return;
  const int nb = n / 64, np = (nb + 1) / 2;
  const int gx = (int)((rows + LH_ROWS - 1) / LH_ROWS);
  int bp, xt;
  {
    const int tiles = gx * np, bid = blockIdx.x;
    const int q = tiles / LH_XCD, rem = tiles % LH_XCD, x = bid % LH_XCD, slot = bid / LH_XCD;
    if (slot >= q + (x < rem ? 1 : 0)) return;  // the grid is rounded up to a multiple of 8
    const int t = x * q + min(x, rem) + slot;
    bp = t / gx;
    xt = t % gx;
  }
  const lds_char* lds = (const lds_char*)lh_lds;
  const uint32_t lds_base = (uint32_t)(uintptr_t)lds;
  const int64_t r0 = (int64_t)xt * LH_ROWS;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = wave >> 2, wr = wave & 3;
  const bool bok = 2 * bp + half < nb;          // this wave's block exists
  const int b = std::min(2 * bp + half, nb - 1);
  const int bdma1 = std::min(2 * bp + 1, nb - 1);  // the second block's H stripe (the first's if none)
  const int rmax = (int)std::min<int64_t>(rows - 1 - r0, LH_ROWS - 1);

  // DMA q (0..79 per stage) fills LDS bytes [1024 q, 1024 q + 1024) of the stage: q < 48 the H
  // split tile (q % 24) / 8 of block 2 bp + q / 24, else the level tile.  Wave w issues q = w + 8 i.
  uint32_t voff[LH_DMA];
#pragma unroll
  for (int i = 0; i < LH_DMA; ++i) {
    const int q = wave + 8 * i;
    const int u = (q < 48 ? (q & 7) : q - 48) * 64 + lane, j = u >> 3;
    const int oct = (u & 7) ^ (j & 7) ^ ((j >> 3) & 1);
    voff[i] = (uint32_t)(((q < 48 ? j : std::min(j, rmax)) * n + oct * 8) * 2);
  }
  auto issue = [&](int s) {
    const uint32_t base = lds_base + (s & 1) * LH_STAGE;
    const int64_t col = (int64_t)64 * s;  // stage s: block c = s
    const int64_t hoff0 = (int64_t)64 * (2 * bp) * n + col;
    const int64_t hoff1 = (int64_t)64 * bdma1 * n + col;
    const int64_t loff = r0 * n + col;
#pragma unroll
    for (int i = 0; i < LH_DMA; ++i) {
      const int q = wave + 8 * i;
      const int pl = (q % 24) >> 3;
      const int64_t hoff = q < 24 ? hoff0 : hoff1;
      const uint16_t* src = q >= 48 ? Lev + loff : pl == 0 ? H0 + hoff : pl == 1 ? H1 + hoff : H2 + hoff;
      lh_dma16(src, voff[i], base + q * 1024);
    }
  };

  // levels (bf16 pairs) and targets of this lane's rows on block b at the accumulator positions:
  // four consecutive j per group of accumulator registers, read as one vector (rows past the end
  // read the last row and are zeroed), all issued before the first use
  uint32_t lvp[2][2][8];
  float tv[2][2][16];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int64_t r = r0 + 64 * wr + 32 * rt + (lane & 31);
    const bool rok = r < rows;
    const int64_t rc = rok ? r : rows - 1;
#pragma unroll
    for (int jt = 0; jt < 2; ++jt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t e = rc * n + 64 * b + 32 * jt + 8 * g + 4 * (lane >> 5);
        const float4 t4 = *reinterpret_cast<const float4*>(T + e);
        const uint2 l2 = *reinterpret_cast<const uint2*>(Lev + e);
        tv[jt][rt][4 * g + 0] = rok ? t4.x : 0.0f;
        tv[jt][rt][4 * g + 1] = rok ? t4.y : 0.0f;
        tv[jt][rt][4 * g + 2] = rok ? t4.z : 0.0f;
        tv[jt][rt][4 * g + 3] = rok ? t4.w : 0.0f;
        lvp[jt][rt][2 * g] = rok ? l2.x : 0u;
        lvp[jt][rt][2 * g + 1] = rok ? l2.y : 0u;
      }
  }

  issue(0);
  f32x16 acc[2][2];
  const int hsel = half * 3 * LH_PLANE;
  for (int s = 0; s < nb; ++s) {
    lh_vm_wait<0>();
    lh_barrier();  // stage s is in LDS for every wave, and every wave is done with stage s - 1
    if (s + 1 < nb) issue(s + 1);  // into the other buffer
    const lds_char* st = lds + (s & 1) * LH_STAGE;
#pragma unroll
    for (int jt = 0; jt < 2; ++jt)
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) acc[jt][rt] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int oct = 2 * ks + (lane >> 5);
      bf16x8 fb[2];
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
        fb[rt] = lh_frag(st + 6 * LH_PLANE + lh_unit(64 * wr + 32 * rt + (lane & 31), oct) * 16);
#pragma unroll
      for (int jt = 0; jt < 2; ++jt) {
        const int ua = hsel + lh_unit(32 * jt + (lane & 31), oct) * 16;
        const bf16x8 a2 = lh_frag(st + 2 * LH_PLANE + ua);
        const bf16x8 a1 = lh_frag(st + LH_PLANE + ua);
        const bf16x8 a0 = lh_frag(st + ua);
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
          acc[jt][rt] = mfma32x32x16_bf16(a2, fb[rt], acc[jt][rt]);  // smallest terms first
          acc[jt][rt] = mfma32x32x16_bf16(a1, fb[rt], acc[jt][rt]);
          acc[jt][rt] = mfma32x32x16_bf16(a0, fb[rt], acc[jt][rt]);
        }
      }
    }
    const int c = s;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const int64_t r = r0 + 64 * wr + 32 * rt + (lane & 31);
      float hpart = 0.0f, gpart = 0.0f;
#pragma unroll
      for (int jt = 0; jt < 2; ++jt)
#pragma unroll
        for (int v = 0; v < 16; ++v) hpart = fmaf(tv[jt][rt][v], acc[jt][rt][v], hpart);
      hpart += __shfl_xor(hpart, 32);
      if (b <= c) {
#pragma unroll
        for (int jt = 0; jt < 2; ++jt)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const uint32_t w2 = lvp[jt][rt][v >> 1];
            const float l = __uint_as_float((v & 1) ? (w2 & 0xffff0000u) : (w2 << 16));
            gpart = fmaf(l, acc[jt][rt][v], gpart);
          }
        gpart += __shfl_xor(gpart, 32);
      }
      if (bok && lane < 32 && r < rows) {
        hp[((size_t)b * nb + c) * rows + r] = hpart;
        if (b <= c) {
          Gm[((size_t)r * nb + b) * nb + c] = gpart;
          Gm[((size_t)r * nb + c) * nb + b] = gpart;
        }
      }
    }
  }
}

// rhs[r][c] = sum over b of hp[b][c][r], in fp64 and in the order of b.
__global__ void rhs_sum_kernel(const float* __restrict__ hp, int64_t rows, int nb, float* __restrict__ rhs,
                               const int32_t* __restrict__ dev_info) {
  if (*dev_info != 0) return;
  const int c = blockIdx.y;
  for (int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; r < rows; r += (int64_t)gridDim.x * blockDim.x) {
    double s = 0.0;
    int b = 0;
    for (; b + 8 <= nb; b += 8) {  // eight loads in flight, then the adds in the order of b
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = hp[((size_t)(b + u) * nb + c) * rows + r];
#pragma unroll
      for (int u = 0; u < 8; ++u) s += (double)v[u];
    }
    for (; b < nb; ++b) s += (double)hp[((size_t)b * nb + c) * rows + r];
    rhs[(size_t)r * nb + c] = (float)s;
  }
}

__device__ __forceinline__ double wave_bcast_f64(double v, int lane) {
  const int64_t u = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane((int)(u & 0xffffffff), lane);
  const int hi = __builtin_amdgcn_readlane((int)(u >> 32), lane);
  return __longlong_as_double(((int64_t)hi << 32) | (uint32_t)lo);
}

__device__ __forceinline__ double rsqrt_refined(double d) {
  double r = (double)rsqrtf((float)d);
  r = r * (1.5 - 0.5 * d * r * r);
  r = r * (1.5 - 0.5 * d * r * r);
  return r;
}

// Per row, nb <= NB: (G + lambda mu I) s = h + lambda mu s0 in fp64, s -> fp16.  One wave per
// row (G full symmetric, row-major nb x nb fp32): lane i holds row i of the matrix in registers
// (identity rows past nb), the Cholesky factor L is formed in place with the pivot columns
// broadcast by readlane, z = L^-1 y by forward substitution in the same layout, then L goes
// through LDS once so that lane i holds column i for the back substitution L^T s = z.
template <int NB>
__global__ __launch_bounds__(64) void row_solve_wave_kernel(const float* __restrict__ Gm, const float* __restrict__ rhs,
                                                            int64_t rows, int nb, float lambda,
                                                            uint16_t* __restrict__ scales, float* __restrict__ raw,
                                                            const int32_t* __restrict__ dev_info) {
  __shared__ double lt[NB * (NB + 1)];
  if (*dev_info != 0) return;
  const int64_t row = blockIdx.x;
  const int lane = threadIdx.x;
  const bool live = lane < nb;
  const float* g = Gm + (size_t)row * nb * nb;
  double tr = live ? (double)g[(size_t)lane * nb + lane] : 0.0;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) tr += __shfl_xor(tr, o);
  const double reg = (double)lambda * tr / nb;
  double a[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    double v = j == lane ? 1.0 : 0.0;
    if (live && j < nb) v = (double)g[(size_t)lane * nb + j] + (j == lane ? reg : 0.0);
    a[j] = v;
  }
  double y = live ? (double)rhs[(size_t)row * nb + lane] + reg * (double)f16_bits_to_f32(scales[(size_t)row * nb + lane])
                  : 0.0;
  bool bad = false;
#pragma unroll
  for (int k = 0; k < NB; ++k) {
    const double d = wave_bcast_f64(a[k], k);
    bad |= !(d > 0.0);
    const double l = a[k] * rsqrt_refined(d);  // lane k: L_kk; lanes below: L_ik
    a[k] = l;
#pragma unroll
    for (int j = k + 1; j < NB; ++j) a[j] = fma(-l, wave_bcast_f64(l, j), a[j]);
  }
  if (bad) return;  // only reachable with lambda == 0 and a singular G: keep the incoming scales
  // z = L^-1 y (lane i: row i of L)
#pragma unroll
  for (int k = 0; k < NB; ++k) {
    const double zk = wave_bcast_f64(y, k) / wave_bcast_f64(a[k], k);
    y = lane == k ? zk : (lane > k ? fma(-a[k], zk, y) : y);
  }
  // transpose L through LDS: lane i then holds L_ki (k >= i) in a[k]
  if (lane < NB) {
#pragma unroll
    for (int j = 0; j < NB; ++j) lt[lane * (NB + 1) + j] = j <= lane ? a[j] : 0.0;
  }
  __syncthreads();
  if (lane < NB) {
#pragma unroll
    for (int k = 0; k < NB; ++k) a[k] = lt[k * (NB + 1) + lane];
  }
  // L^T s = z, last unknown first
#pragma unroll
  for (int k = NB - 1; k >= 0; --k) {
    const double sk = wave_bcast_f64(y, k) / wave_bcast_f64(a[k], k);
    y = lane == k ? sk : (lane < k ? fma(-a[k], sk, y) : y);
  }
  if (live) {
    scales[(size_t)row * nb + lane] = f64_to_f16_bits_clamped(y);
    if (raw) raw[(size_t)row * nb + lane] = (float)y;
  }
}

// Per row: (G + lambda mu I) s = h + lambda mu s0 in fp64 (packed lower Cholesky in LDS), s -> fp16.
// One 256-thread workgroup per row: G is read row by row (coalesced) into the packed lower
// triangle; per pivot the column below it is scaled, then every element of the trailing triangle
// is updated once, thread (r, c) of a 16 x 16 grid taking the rows r (mod 16) and in them the
// columns c (mod 16); then the two substitutions.  The trace is a 64-lane butterfly in the first wave.
constexpr int RS_THREADS = 256;
__global__ __launch_bounds__(RS_THREADS) void row_solve_kernel(const float* __restrict__ Gm, const float* __restrict__ rhs,
                                                               int64_t rows, int nb, float lambda,
                                                               uint16_t* __restrict__ scales, float* __restrict__ raw,
                                                               const int32_t* __restrict__ dev_info) {
  extern __shared__ double sh[];
  if (*dev_info != 0) return;
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  double* a = sh;                               // packed lower: a[i(i+1)/2 + j]
  double* y = sh + (size_t)nb * (nb + 1) / 2;
  __shared__ int failed;
  __shared__ double sreg;
  const float* g = Gm + (size_t)row * nb * nb;
  if (tid < 64) {
    double tr = 0.0;
    for (int i = tid; i < nb; i += 64) tr += (double)g[(size_t)i * nb + i];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) tr += __shfl_xor(tr, o);
    if (tid == 0) {
      sreg = (double)lambda * tr / nb;
      failed = 0;
    }
  }
  __syncthreads();
  const double reg = sreg;
  // element (j, i), j >= i, of the lower triangle from G[i][j] (G symmetric: the upper half, read
  // along rows)
  for (int t = tid; t < nb * nb; t += RS_THREADS) {
    const int i = t / nb, j = t - i * nb;
    if (j >= i) a[(size_t)j * (j + 1) / 2 + i] = (double)g[t] + (i == j ? reg : 0.0);
  }
  for (int i = tid; i < nb; i += RS_THREADS)
    y[i] = (double)rhs[(size_t)row * nb + i] + reg * (double)f16_bits_to_f32(scales[(size_t)row * nb + i]);
  __syncthreads();
  for (int k = 0; k < nb; ++k) {
    const size_t kk = (size_t)k * (k + 1) / 2 + k;
    if (tid == 0) {
      const double d = a[kk];
      if (!(d > 0.0)) failed = 1;
      else a[kk] = sqrt(d);
    }
    __syncthreads();
    if (failed) return;  // only reachable with lambda == 0 and a singular G: keep the incoming scales
    const double dk = a[kk];
    for (int i = k + 1 + tid; i < nb; i += RS_THREADS) a[(size_t)i * (i + 1) / 2 + k] /= dk;
    __syncthreads();
    const int m = nb - k - 1;  // trailing rows and columns k + 1 .. nb - 1
    for (int ii = tid >> 4; ii < m; ii += RS_THREADS / 16) {  // rows ii = tid / 16 (mod 16)
      const int i = k + 1 + ii;
      const size_t ri = (size_t)i * (i + 1) / 2;
      const double aik = a[ri + k];
      for (int jj = tid & 15; jj <= ii; jj += 16) {  // columns jj = tid (mod 16)
        const int j = k + 1 + jj;
        a[ri + j] -= aik * a[(size_t)j * (j + 1) / 2 + k];
      }
    }
    __syncthreads();
  }
  // L z = y
  for (int k = 0; k < nb; ++k) {
    if (tid == 0) y[k] /= a[(size_t)k * (k + 1) / 2 + k];
    __syncthreads();
    const double zk = y[k];
    for (int i = k + 1 + tid; i < nb; i += RS_THREADS) y[i] -= a[(size_t)i * (i + 1) / 2 + k] * zk;
    __syncthreads();
  }
  // L^T s = z
  for (int k = nb - 1; k >= 0; --k) {
    if (tid == 0) y[k] /= a[(size_t)k * (k + 1) / 2 + k];
    __syncthreads();
    const double uk = y[k];
    for (int i = tid; i < k; i += RS_THREADS) y[i] -= a[(size_t)k * (k + 1) / 2 + i] * uk;
    __syncthreads();
  }
  for (int i = tid; i < nb; i += RS_THREADS) {
    scales[(size_t)row * nb + i] = f64_to_f16_bits_clamped(y[i]);
    if (raw) raw[(size_t)row * nb + i] = (float)y[i];
  }
}

// Per row, 64 < nb <= 160: the same solve blocked by 16 on the fp64 matrix cores.  One 256-thread
// workgroup per row; the lower 16 x 16 blocks of A = G + lambda mu I (fp64, padded to a multiple of
// 16 with the identity) sit in LDS at a pitch of 17 doubles, next to the inverted diagonal factor
// blocks.  Per block column K: the panel L_IK = A_IK X_K^T (X_K = L_KK^-1) on the matrix cores, one
// block per wave in turn, and z_K = X_K y_K (the forward substitution carried as an extra column);
// then wave 0 updates the next diagonal block and factors and inverts it in registers while waves
// 1-3 update the other trailing blocks, A_IJ -= L_IK L_JK^T, and y_I -= L_IK z_K.  The back
// substitution L^T s = z runs block by block from the last one, s_K = X_K^T z_K followed by
// z_J -= L_KJ^T s_K.  Two barriers per block column instead of a few per pivot.
constexpr int RB_P = 17;             // row pitch of an LDS block, doubles (rows on different banks)
constexpr int RB_BLK = 16 * RB_P;    // doubles per block
constexpr int RB_MAXK = 10;          // block rows: up to 160 unknowns
__device__ __forceinline__ int rb_idx(int I, int J) { return I * (I + 1) / 2 + J; }

__global__ __launch_bounds__(256) void row_solve_blk_kernel(const float* __restrict__ Gm, const float* __restrict__ rhs,
                                                            int64_t rows, int nb, float lambda,
                                                            uint16_t* __restrict__ scales, float* __restrict__ raw,
                                                            const int32_t* __restrict__ dev_info) {
  extern __shared__ double sh[];
  __shared__ double sreg;
  __shared__ int failed;
  if (*dev_info != 0) return;
  const int nbk = (nb + 15) >> 4, nbp = 16 * nbk;
  double* Ab = sh;                                  // lower blocks, rb_idx order
  double* Xb = sh + (size_t)nbk * (nbk + 1) / 2 * RB_BLK;  // X_K = L_KK^-1
  double* y = Xb + (size_t)nbk * RB_BLK;            // right-hand side, then z, then s
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const f64x4 zero = {0.0, 0.0, 0.0, 0.0};
  const float* g = Gm + (size_t)row * nb * nb;
  if (tid < 64) {
    double tr = 0.0;
    for (int i = tid; i < nb; i += 64) tr += (double)g[(size_t)i * nb + i];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) tr += __shfl_xor(tr, o);
    if (tid == 0) {
      sreg = (double)lambda * tr / nb;
      failed = 0;
    }
  }
  __syncthreads();
  const double reg = sreg;
  for (int t = tid; t < nbp * nbp; t += 256) {
    const int i = t / nbp, j = t - i * nbp;
    if (j > i) continue;
    double v = i == j ? 1.0 : 0.0;
    if (i < nb) v = (double)g[(size_t)i * nb + j] + (i == j ? reg : 0.0);
    Ab[rb_idx(i >> 4, j >> 4) * RB_BLK + (i & 15) * RB_P + (j & 15)] = v;
  }
  for (int i = tid; i < nbp; i += 256)
    y[i] = i < nb ? (double)rhs[(size_t)row * nb + i] + reg * (double)f16_bits_to_f32(scales[(size_t)row * nb + i])
                  : 0.0;
  __syncthreads();
  if (wave == 0) {
    const int b = chol16_inv_pitch<RB_P>(Ab, Xb, lane);
    if (b >= 0 && lane == 0) failed = 1;
  }
  __syncthreads();
  for (int K = 0; K < nbk; ++K) {
    if (failed) return;  // only reachable with lambda == 0 and a singular G: keep the incoming scales
    const double* XK = Xb + K * RB_BLK;
    for (int I = K + 1 + wave; I < nbk; I += 4) {
      double* AIK = Ab + rb_idx(I, K) * RB_BLK;
      const f64x4 acc = mma16<true>(AIK, RB_P, 0, XK, RB_P, 0, 16, zero, lane);
#pragma unroll
      for (int v = 0; v < 4; ++v) AIK[((lane >> 4) + 4 * v) * RB_P + (lane & 15)] = acc[v];
    }
    // z_K = X_K y_K by exactly one wave (it reads y_K and then overwrites it): the first wave
    // without a panel block, or wave 3 (the last panel blocks' wave) when all four have one
    if (wave == (nbk - K - 1 < 4 ? nbk - K - 1 : 3)) {
      double z = 0.0;
      if (lane < 16) {
#pragma unroll
        for (int c = 0; c < 16; ++c) z = fma(XK[lane * RB_P + c], y[16 * K + c], z);
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      if (lane < 16) y[16 * K + lane] = z;
    }
    __syncthreads();
    if (wave == 0) {
      if (K + 1 < nbk) {
        double* D = Ab + rb_idx(K + 1, K + 1) * RB_BLK;
        const double* P = Ab + rb_idx(K + 1, K) * RB_BLK;
        const f64x4 acc = mma16<true>(P, RB_P, 0, P, RB_P, 0, 16, zero, lane);
#pragma unroll
        for (int v = 0; v < 4; ++v) D[((lane >> 4) + 4 * v) * RB_P + (lane & 15)] -= acc[v];
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        const int b = chol16_inv_pitch<RB_P>(D, Xb + (K + 1) * RB_BLK, lane);
        if (b >= 0 && lane == 0) failed = 1;
      }
    } else {
      int t = 0;
      for (int J = K + 1; J < nbk; ++J)
        for (int I = J; I < nbk; ++I) {
          if (I == K + 1 && J == K + 1) continue;
          if (t++ % 3 != wave - 1) continue;
          const f64x4 acc = mma16<true>(Ab + rb_idx(I, K) * RB_BLK, RB_P, 0, Ab + rb_idx(J, K) * RB_BLK, RB_P, 0, 16,
                                        zero, lane);
          double* C = Ab + rb_idx(I, J) * RB_BLK;
#pragma unroll
          for (int v = 0; v < 4; ++v) C[((lane >> 4) + 4 * v) * RB_P + (lane & 15)] -= acc[v];
        }
      for (int i = 16 * (K + 1) + tid - 64; i < nbp; i += 192) {
        const double* Li = Ab + rb_idx(i >> 4, K) * RB_BLK + (i & 15) * RB_P;
        double acc = 0.0;
#pragma unroll
        for (int c = 0; c < 16; ++c) acc = fma(Li[c], y[16 * K + c], acc);
        y[i] -= acc;
      }
    }
    __syncthreads();
  }
  if (failed) return;
  for (int K = nbk - 1; K >= 0; --K) {
    if (wave == 0) {  // s_K = X_K^T z_K
      const double* XK = Xb + K * RB_BLK;
      double sk = 0.0;
      if (lane < 16) {
#pragma unroll
        for (int c = 0; c < 16; ++c) sk = fma(XK[c * RB_P + lane], y[16 * K + c], sk);
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      if (lane < 16) y[16 * K + lane] = sk;
    }
    __syncthreads();
    for (int j = tid; j < 16 * K; j += 256) {  // z_J -= L_KJ^T s_K for the blocks J < K
      const double* LKJ = Ab + rb_idx(K, j >> 4) * RB_BLK + (j & 15);
      double acc = 0.0;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc = fma(LKJ[r * RB_P], y[16 * K + r], acc);
      y[j] -= acc;
    }
    __syncthreads();
  }
  for (int i = tid; i < nb; i += 256) {
    scales[(size_t)row * nb + i] = f64_to_f16_bits_clamped(y[i]);
    if (raw) raw[(size_t)row * nb + i] = (float)y[i];
  }
}

static size_t row_solve_blk_lds_bytes(int64_t nb) {
  const int64_t k = (nb + 15) / 16;
  return ((size_t)(k * (k + 1) / 2 + k) * RB_BLK + 16 * k) * sizeof(double);
}

// Block scale search (the finisher "nearest-point codes + block scale search"): for each block
// of G weights of T, the candidate scales s_k = fp16((1 - k/64) max|t| / L), k = 0..31, each with
// the nearest codes of t / s_k (IEEE division, as in the recode); the candidate with the least
// squared error of the block wins, the smaller k on a tie.  One half-wave (32 lanes, lane = k)
// per block, eight blocks per workgroup, the block's targets staged in LDS; the scale is
// formed in fp64 and rounded once to fp16; the error is summed in fp64.  Nothing is written
// when dev_info is already set (a non-finite target).
template <int G>
__global__ __launch_bounds__(256) void scale_search_kernel(const float* __restrict__ T, int64_t rows, int n,
                                                           const uint8_t* __restrict__ bits, uint8_t* __restrict__ codes,
                                                           uint16_t* __restrict__ scales,
                                                           const int32_t* __restrict__ dev_info) {
  if (*dev_info != 0) return;
  __shared__ float sT[8][G];
  const int nb = n / G;
  const int64_t blocks = rows * nb;
  const int tid = threadIdx.x, k = tid & 31, bl = tid >> 5;
  const int64_t blk0 = (int64_t)blockIdx.x * 8;
  for (int i = tid; i < 8 * G; i += 256) {
    const int bb = i / G, j = i % G;
    const int64_t blk = blk0 + bb;
    float v = 0.0f;
    if (blk < blocks) {
      const int64_t r = blk / nb;
      v = T[r * n + (blk - r * nb) * G + j];
    }
    sT[bb][j] = v;
  }
  __syncthreads();
  const int64_t blk = blk0 + bl;
  const bool live = blk < blocks;
  const int64_t r = live ? blk / nb : 0;
  const int b = live ? (int)(blk - r * nb) : 0;
  const int L = (1 << bits[r]) - 1;
  float amax = 0.0f;
  for (int j = 0; j < G; ++j) amax = fmaxf(amax, fabsf(sT[bl][j]));
  auto cand = [&](int kk) { return f16_bits_to_f32(f64_to_f16_bits_clamped((1.0 - kk / 64.0) * (double)amax / L)); };
  const float s = cand(k);
  double err = 0.0;
  for (int j = 0; j < G; ++j) {
    const float w = sT[bl][j];
    const int c = nearest_code(s > 0.0f ? w / s : 0.0f, L);
    const double d = (double)w - (double)s * (double)(2 * c - L);
    err = fma(d, d, err);
  }
  double be = err;
  int bk = k;
#pragma unroll
  for (int o = 1; o < 32; o <<= 1) {
    const double oe = __shfl_xor(be, o);
    const int ok = __shfl_xor(bk, o);
    if (oe < be || (oe == be && ok < bk)) {
      be = oe;
      bk = ok;
    }
  }
  if (!live) return;
  const float sb = cand(bk);
  constexpr int PER = G / 32;
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int j = k * PER + q;
    const float w = sT[bl][j];
    codes[r * n + (int64_t)b * G + j] = (uint8_t)nearest_code(sb > 0.0f ? w / sb : 0.0f, L);
  }
  if (k == 0) scales[r * nb + b] = f64_to_f16_bits_clamped((double)sb);
}

}  // namespace wr

using namespace wr;

struct WringLayout {
  size_t T, Lev, T0, T1, T2, H0, H1, H2, Gm, rhs, hp, Bf, Af, total;
};

static WringLayout wring_layout(int64_t rows, int64_t n, int32_t group, int32_t rank) {
  WringLayout l{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += (bytes + 255) & ~(size_t)255;
    return o;
  };
  const int64_t nb = n / group;
  const bool lh = group == 64;  // gram_lh_kernel: no split target, per-block shares of h
  l.T = take((size_t)rows * n * 4);
  l.Lev = take((size_t)rows * n * 2);
  l.T0 = take(lh ? 0 : (size_t)rows * n * 2);
  l.T1 = take(lh ? 0 : (size_t)rows * n * 2);
  l.T2 = take(lh ? 0 : (size_t)rows * n * 2);
  l.hp = take(lh ? (size_t)nb * nb * rows * 4 : 0);
  l.H0 = take((size_t)n * n * 2);
  l.H1 = take((size_t)n * n * 2);
  l.H2 = take((size_t)n * n * 2);
  l.Gm = take((size_t)rows * nb * nb * 4);
  l.rhs = take((size_t)rows * nb * 4);
  l.Bf = take((size_t)rows * (rank > 0 ? rank : 0) * 4);
  l.Af = take((size_t)n * (rank > 0 ? rank : 0) * 4);
  l.total = off;
  return l;
}

size_t wr_wring_ws_bytes(int64_t rows, int64_t n, int32_t group, int32_t rank) {
  return wring_layout(rows, n, group, rank).total;
}

size_t wr_gptq_ws_bytes(int64_t rows, int64_t n);
int wr_gptq_sweep_impl(wr_ctx* ctx, const void* W, int w_dtype, int64_t rows, int64_t n64, int64_t ldw,
                       const float* H, int64_t ldh, const uint8_t* bits, int32_t group, int32_t lazy_batch,
                       uint8_t* codes, uint16_t* scales, int32_t* dev_info);

static size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

// Workspace of the wring with GPTQ codes: the target T (rows x n fp32) kept across the sweep,
// then room for the larger of the sweep's and the joint solve's own workspaces.
size_t wr_wring_gptq_ws_bytes(int64_t rows, int64_t n, int32_t group, int32_t rank) {
  const size_t a = wr_gptq_ws_bytes(rows, n), b = wring_layout(rows, n, group, rank).total;
  return align256((size_t)rows * n * 4) + (a > b ? a : b);
}

// LDS of the per-row solve above 64 blocks: the packed factor and the right-hand side in fp64.
static size_t row_solve_lds_bytes(int64_t nb) { return ((size_t)nb * (nb + 1) / 2 + nb) * sizeof(double); }

// The joint solve on workspace ws.  With T_only the target T is formed there (codes and
// scales untouched) and nothing else is done; reset_info = false keeps a status already in
// dev_info (the later kernels do nothing when it is nonzero).
static int wring_core(wr_ctx* ctx, char* ws, size_t ws_bytes, const void* target, int t_dtype, int64_t ldt,
                      const void* B, const void* A, int32_t rank, float alpha, int ab_dtype, const float* H,
                      int64_t ldh, int64_t rows, int64_t n64, const uint8_t* bits, int32_t group, float lambda,
                      int flags, bool reset_info, float* T_only, uint8_t* codes, uint16_t* scales, int32_t* dev_info) {
  if (group != 32 && group != 64 && group != 128) return WR_EUNSUPPORTED;
  const bool adapter = B && A && rank > 0;
  const WringLayout lay = wring_layout(rows, n64, group, adapter ? rank : 0);
  if (ws_bytes < lay.total) return WR_EWORKSPACE;
  const int n = (int)n64;
  const int nb = n / group;
  hipStream_t st = ctx->stream;
  float* T = T_only ? T_only : reinterpret_cast<float*>(ws + lay.T);
  uint16_t* Lev = reinterpret_cast<uint16_t*>(ws + lay.Lev);
  const bool lh = group == 64;
  uint16_t* T0 = lh ? nullptr : reinterpret_cast<uint16_t*>(ws + lay.T0);
  uint16_t* T1 = lh ? nullptr : reinterpret_cast<uint16_t*>(ws + lay.T1);
  uint16_t* T2 = lh ? nullptr : reinterpret_cast<uint16_t*>(ws + lay.T2);
  uint16_t* H0 = reinterpret_cast<uint16_t*>(ws + lay.H0);
  uint16_t* H1 = reinterpret_cast<uint16_t*>(ws + lay.H1);
  uint16_t* H2 = reinterpret_cast<uint16_t*>(ws + lay.H2);
  float* Gm = reinterpret_cast<float*>(ws + lay.Gm);
  float* rh = reinterpret_cast<float*>(ws + lay.rhs);
  float* raw = ctx->scale_trace;  // unprojected scales for the measures, when the caller asked for them

  if (reset_info) {
    hipLaunchKernelGGL(set_int_kernel, dim3(1), dim3(1), 0, st, dev_info, 0);
    WR_CHECK_LAUNCH();
  }
  if (rows == 0) return WR_OK;
  const unsigned gx = (unsigned)std::min<int64_t>((n + 255) / 256, 16);
  const bool fused = lh && (!adapter || (ab_dtype == WR_BF16 && rank % 16 == 0 &&
                                         reinterpret_cast<uintptr_t>(B) % 16 == 0));
  if (fused) {
    uint16_t* At = reinterpret_cast<uint16_t*>(ws + lay.Af);
    if (adapter) {
      hipLaunchKernelGGL(transpose_ab_kernel, dim3((unsigned)std::min((n + 255) / 256, 64), (unsigned)rank), dim3(256),
                         0, st, static_cast<const uint16_t*>(A), rank, n, At);
      WR_CHECK_LAUNCH();
    }
    const dim3 pgrid((unsigned)((n + 63) / 64), (unsigned)((rows + 63) / 64));
    hipLaunchKernelGGL(wring_prep_kernel, pgrid, dim3(256), 0, st, target, t_dtype, ldt,
                       static_cast<const uint16_t*>(B), At, adapter ? rank : 0, adapter ? alpha / (float)rank : 0.0f,
                       bits, rows, n, (flags & WR_RECODE_NEAREST) ? 1 : 0, codes, scales, T, Lev, dev_info);
    WR_CHECK_LAUNCH();
  } else {
    hipLaunchKernelGGL(target_kernel, dim3(gx, (unsigned)rows), dim3(256), 0, st, target, t_dtype, ldt, codes, scales,
                       bits, rows, n, group, T);
    WR_CHECK_LAUNCH();
    if (adapter) {
      float* Bf = reinterpret_cast<float*>(ws + lay.Bf);
      float* Af = reinterpret_cast<float*>(ws + lay.Af);
      hipLaunchKernelGGL(to_f32_kernel, dim3(256), dim3(256), 0, st, B, ab_dtype, rows * rank, Bf);
      WR_CHECK_LAUNCH();
      hipLaunchKernelGGL(to_f32_kernel, dim3(256), dim3(256), 0, st, A, ab_dtype, (int64_t)rank * n, Af);
      WR_CHECK_LAUNCH();
      const int rc = wr_gemm_f32(st, (int)rows, n, rank, Bf, rank, Af, n, true, T, n, alpha / (float)rank, true, false,
                                 nullptr);
      if (rc) return rc;
    }
    hipLaunchKernelGGL(recode_residual_kernel, dim3(gx, (unsigned)rows), dim3(256), 0, st, T, codes, scales, bits, rows,
                       n, group, (flags & WR_RECODE_NEAREST) ? 1 : 0, Lev, T0, T1, T2, dev_info);
    WR_CHECK_LAUNCH();
  }
  if (T_only) return WR_OK;
  if (n % 8 == 0 && ldh % 4 == 0 && (reinterpret_cast<uintptr_t>(H) & 15) == 0)
    hipLaunchKernelGGL(split_h_vec_kernel, dim3(2048), dim3(256), 0, st, H, ldh, n, H0, H1, H2);
  else
    hipLaunchKernelGGL(split_h_kernel, dim3(gx, (unsigned)n), dim3(256), 0, st, H, ldh, n, H0, H1, H2);
  WR_CHECK_LAUNCH();
  dim3 ggrid((unsigned)((rows + 127) / 128), (unsigned)nb);
  if (lh) {
    if (!lds_limit(reinterpret_cast<const void*>(gram_lh_kernel), 2 * LH_STAGE)) return WR_EHIP;
    float* hp = reinterpret_cast<float*>(ws + lay.hp);
    hipLaunchKernelGGL(gram_lh_kernel, dim3(gram_lh_grid(rows, nb)), dim3(512), 2 * LH_STAGE, st, Lev, T, rows, n,
                       H0, H1, H2, Gm, hp, dev_info);
    WR_CHECK_LAUNCH();
    const unsigned sx = (unsigned)std::min<int64_t>((rows + 255) / 256, 64);
    hipLaunchKernelGGL(rhs_sum_kernel, dim3(sx, (unsigned)nb), dim3(256), 0, st, hp, rows, nb, rh, dev_info);
  } else if (group == 32) {
    hipLaunchKernelGGL(gram_kernel<32>, ggrid, dim3(256), 0, st, Lev, T0, T1, T2, rows, n, H0, H1, H2, Gm, rh, dev_info);
  } else {
    hipLaunchKernelGGL(gram_kernel<128>, ggrid, dim3(256), 0, st, Lev, T0, T1, T2, rows, n, H0, H1, H2, Gm, rh, dev_info);
  }
  WR_CHECK_LAUNCH();
  if (nb <= 64) {
    const dim3 grid((unsigned)rows);
    // the unrolled factorization costs NB^2 broadcasts and fmas whatever nb is: buckets of 8
    // (40 blocks for a 2560-wide layer with groups of 64)
    if (nb <= 16)
      hipLaunchKernelGGL(row_solve_wave_kernel<16>, grid, dim3(64), 0, st, Gm, rh, rows, nb, lambda, scales, raw, dev_info);
    else if (nb <= 24)
      hipLaunchKernelGGL(row_solve_wave_kernel<24>, grid, dim3(64), 0, st, Gm, rh, rows, nb, lambda, scales, raw, dev_info);
    else if (nb <= 32)
      hipLaunchKernelGGL(row_solve_wave_kernel<32>, grid, dim3(64), 0, st, Gm, rh, rows, nb, lambda, scales, raw, dev_info);
    else if (nb <= 40)
      hipLaunchKernelGGL(row_solve_wave_kernel<40>, grid, dim3(64), 0, st, Gm, rh, rows, nb, lambda, scales, raw, dev_info);
    else if (nb <= 48)
      hipLaunchKernelGGL(row_solve_wave_kernel<48>, grid, dim3(64), 0, st, Gm, rh, rows, nb, lambda, scales, raw, dev_info);
    else
      hipLaunchKernelGGL(row_solve_wave_kernel<64>, grid, dim3(64), 0, st, Gm, rh, rows, nb, lambda, scales, raw, dev_info);
    WR_CHECK_LAUNCH();
    return WR_OK;
  }
  if ((nb + 15) / 16 <= RB_MAXK) {
    const size_t bbytes = row_solve_blk_lds_bytes(nb);
    if (!lds_limit(reinterpret_cast<const void*>(row_solve_blk_kernel), (int)bbytes)) return WR_EHIP;
    hipLaunchKernelGGL(row_solve_blk_kernel, dim3((unsigned)rows), dim3(256), bbytes, st, Gm, rh, rows, nb, lambda,
                       scales, raw, dev_info);
    WR_CHECK_LAUNCH();
    return WR_OK;
  }
  const size_t shbytes = row_solve_lds_bytes(nb);
  if (shbytes > 160 * 1024) return WR_EUNSUPPORTED;  // refused by wr_wring_solve_impl before any launch
  if (shbytes > 64 * 1024 && !lds_limit(reinterpret_cast<const void*>(row_solve_kernel), (int)shbytes))
    return WR_EHIP;
  hipLaunchKernelGGL(row_solve_kernel, dim3((unsigned)rows), dim3(RS_THREADS), shbytes, st, Gm, rh, rows, nb, lambda,
                     scales, raw, dev_info);
  WR_CHECK_LAUNCH();
  return WR_OK;
}

namespace {
// Points the context's workspace at a sub-range for the duration of a call.
struct WorkspaceView {
  wr_ctx* c;
  void* ws;
  size_t bytes;
  WorkspaceView(wr_ctx* ctx, void* sub, size_t sub_bytes) : c(ctx), ws(ctx->ws), bytes(ctx->ws_bytes) {
    c->ws = sub;
    c->ws_bytes = sub_bytes;
  }
  ~WorkspaceView() {
    c->ws = ws;
    c->ws_bytes = bytes;
  }
};
}  // namespace

int wr_wring_solve_impl(wr_ctx* ctx, const void* target, int t_dtype, int64_t ldt, const void* B, const void* A,
                        int32_t rank, float alpha, int ab_dtype, const float* H, int64_t ldh, int64_t rows, int64_t n,
                        const uint8_t* bits, int32_t group, float lambda, int flags, uint8_t* codes, uint16_t* scales,
                        int32_t* dev_info) {
  // requests that the per-row solve cannot hold in LDS are refused before anything is launched
  if (!(flags & WR_RECODE_SEARCH) && n / group > 64 && row_solve_lds_bytes(n / group) > 160 * 1024)
    return WR_EUNSUPPORTED;
  if (ctx->scale_trace && ctx->scale_trace_count < rows * (n / group)) return WR_EINVAL;
  if (flags & WR_RECODE_SEARCH) {
    // the watered target into the joint solve's T slot, then the search (no joint solve)
    if (group != 32 && group != 64 && group != 128) return WR_EUNSUPPORTED;
    const bool adapter = B && A && rank > 0;
    const WringLayout lay = wring_layout(rows, n, group, adapter ? rank : 0);
    if (ctx->ws_bytes < lay.total) return WR_EWORKSPACE;
    char* ws = static_cast<char*>(ctx->ws);
    float* T = reinterpret_cast<float*>(ws + lay.T);
    int rc = wring_core(ctx, ws, ctx->ws_bytes, target, t_dtype, ldt, B, A, rank, alpha, ab_dtype, H, ldh, rows, n,
                        bits, group, lambda, 0, true, T, codes, scales, dev_info);
    if (rc || rows == 0) return rc;
    const dim3 grid((unsigned)((rows * (n / group) + 7) / 8));
    if (group == 32)
      hipLaunchKernelGGL(scale_search_kernel<32>, grid, dim3(256), 0, ctx->stream, T, rows, (int)n, bits, codes, scales,
                         dev_info);
    else if (group == 64)
      hipLaunchKernelGGL(scale_search_kernel<64>, grid, dim3(256), 0, ctx->stream, T, rows, (int)n, bits, codes, scales,
                         dev_info);
    else
      hipLaunchKernelGGL(scale_search_kernel<128>, grid, dim3(256), 0, ctx->stream, T, rows, (int)n, bits, codes,
                         scales, dev_info);
    WR_CHECK_LAUNCH();
    return WR_OK;
  }
  if (!(flags & WR_RECODE_GPTQ))
    return wring_core(ctx, static_cast<char*>(ctx->ws), ctx->ws_bytes, target, t_dtype, ldt, B, A, rank, alpha,
                      ab_dtype, H, ldh, rows, n, bits, group, lambda, flags, true, nullptr, codes, scales, dev_info);
  // GPTQ codes on the watered target: T = target or dequant, plus the adapter; the sweep of T
  // with H gives codes and scales; then the joint scales against T, the prior centred on the
  // sweep's scales.
  const bool adapter = B && A && rank > 0;
  if (ctx->ws_bytes < wr_wring_gptq_ws_bytes(rows, n, group, adapter ? rank : 0)) return WR_EWORKSPACE;
  char* ws = static_cast<char*>(ctx->ws);
  float* Tk = reinterpret_cast<float*>(ws);
  const size_t tb = align256((size_t)rows * n * 4);
  char* rest = ws + tb;
  const size_t rest_bytes = ctx->ws_bytes - tb;
  int rc = wring_core(ctx, rest, rest_bytes, target, t_dtype, ldt, B, A, rank, alpha, ab_dtype, H, ldh, rows, n, bits,
                      group, lambda, 0, true, Tk, codes, scales, dev_info);
  if (rc) return rc;
  if (rows == 0) return WR_OK;
  {
    WorkspaceView view(ctx, rest, rest_bytes);
    rc = wr_gptq_sweep_impl(ctx, Tk, WR_F32, rows, n, n, H, ldh, bits, group, 128, codes, scales, dev_info);
  }
  if (rc) return rc;
  return wring_core(ctx, rest, rest_bytes, Tk, WR_F32, n, nullptr, nullptr, 0, 0.0f, WR_F32, H, ldh, rows, n, bits,
                    group, lambda, 0, false, nullptr, codes, scales, dev_info);
}

// The watered target alone (the filled weights of the model cards): T_out (rows x n fp32,
// contiguous) = target, or dequant(codes, scales) when target is null, plus (alpha / rank) B A.
int wr_wring_target_impl(wr_ctx* ctx, const void* target, int t_dtype, int64_t ldt, const void* B, const void* A,
                         int32_t rank, float alpha, int ab_dtype, int64_t rows, int64_t n, const uint8_t* bits,
                         int32_t group, const uint8_t* codes, const uint16_t* scales, float* T_out,
                         int32_t* dev_info) {
  if (rows == 0) return WR_OK;
  return wring_core(ctx, static_cast<char*>(ctx->ws), ctx->ws_bytes, target, t_dtype, ldt, B, A, rank, alpha, ab_dtype,
                    nullptr, n, rows, n, bits, group, 0.0f, 0, true, T_out, const_cast<uint8_t*>(codes),
                    const_cast<uint16_t*>(scales), dev_info);
}
