// Calibration second moment S += X^T X (lower triangle).
//
// H is the average of x x^T over calibration inputs (Pingala-8 post, "Trick 2:
// round with error feedback"); delta is the Tikhonov damping of the GPTQ solve
// (Wringer news article, second paragraph).
//
// bf16 path: a SYRK on the bf16 matrix cores.  Each workgroup owns one 256x256
// tile of the lower triangle of S and a range of calibration rows; each of its
// eight waves owns a 128x64 part.  X is row-major (feature index contiguous),
// which is the wrong way round for an MFMA operand (8 consecutive calibration
// rows of one feature per lane), so the rows are copied untransposed into LDS by
// LDS-DMA loads (global_load_lds, no registers, several stages in flight) and
// transposed on the way out by the gfx950 transposing LDS read
// (ds_read_b64_tr_b16).  bf16 x bf16 products are exact in fp32; the MFMAs sum at
// most 32768 rows in fp32 before the sums reach S in fp64: either every
// workgroup adds its tile into S itself (one split per tile, when the tiles alone
// fill the chip; calls longer than 32768 rows become one launch per 32768-row
// slice), or the rows are cut into splits whose fp32 sums a second kernel adds
// into S in a fixed order.  Deterministic, no atomics.
#include <mutex>

#include "common.hpp"

namespace wr {

constexpr int SY_T = 256;                // tile edge
constexpr int SY_KT = 32;                // calibration rows per LDS stage
constexpr int SY_NS = 5;                 // stages in the LDS ring
constexpr int SY_PF = SY_NS;             // stages issued ahead of the one being consumed (every slot)
constexpr int SY_PANEL = SY_KT * SY_T * 2;            // one operand panel of a stage, bytes
constexpr int SY_STAGE_BYTES = 2 * SY_PANEL;
constexpr int SY_LDS_BYTES = SY_NS * SY_STAGE_BYTES;  // 160 KB
constexpr int SY_THREADS = 512;          // eight waves
constexpr int SY_DMA_PER_WAVE = (SY_STAGE_BYTES / 1024) / (SY_THREADS / 64);  // 1 KB per wave-wide DMA
constexpr int SY_XCD = 8;                // workgroups are dispatched round-robin over 8 XCDs
constexpr int SY_MAX_ROWS = 32768;       // rows summed in fp32 before the sums reach S in fp64
constexpr int SY_SPLIT_ROWS = 16384;     // rows per split when the tiles alone do not fill the chip

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Wave-wide LDS DMA: lane l copies 16 bytes from sbase + voff to LDS byte address
// m0 + 16 l.  Issued from inline assembly so that the compiler does not wait for it
// before unrelated LDS reads; completion is awaited with vm_wait.  The M0 write
// needs one wait state before the DMA.
__device__ __forceinline__ void lds_dma16(const void* sbase, uint32_t voff, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %2" ::"v"(voff), "s"(m0), "s"(sbase)
               : "memory", "m0");
}
template <int N>
__device__ __forceinline__ void vm_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// Workgroup barrier that the compiler cannot move LDS reads across.  Each wave's
// own LDS reads are complete (waited before the MFMAs that use them) and its own
// DMAs are waited with vm_wait, so after the barrier every wave sees every DMA.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Two transposing reads give one MFMA operand: 8 consecutive calibration rows of one feature.
__device__ __forceinline__ bf16x8 tr_frag(const lds_char* p, int half_stride) {
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + half_stride));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// S_lower += XA^T XB over rows [split * rows_per_split, ...) of the call (XA gives the
// tile's row features, XB its column features; both rows x n bf16, leading dimension
// ldx).  With ksplit == 1 the tile is added into S (fp64); otherwise its fp32 sums
// go to partial[split][tile][256][256].
//
// Eight waves (two per SIMD, so one issues MFMAs while the other waits on LDS or
// the barrier); wave w owns rows 128 (w / 4) .. +127 and columns 64 (w % 4) .. +63.
// LDS stage layout: panel A (row features) then panel B (column features), each 32
// calibration rows x 256 features, 512 bytes per row.  The 16-byte chunk c of row k
// sits at chunk position c ^ 4 (k & 3), so the four rows that one transposing read
// touches fall on disjoint bank groups.  Each DMA fills 1 KB (2 rows); every wave
// issues two per panel per stage.
__global__ __launch_bounds__(SY_THREADS, 1) void syrk_bf16_kernel(const uint16_t* __restrict__ XA,
                                                                  const uint16_t* __restrict__ XB, int64_t rows, int n,
                                                                  int64_t ldx, int64_t rows_per_split, int tiles,
                                                                  int ksplit, double* __restrict__ S,
                                                                  float* __restrict__ partial) {
  extern __shared__ __attribute__((aligned(1024))) char sy_lds[];
  lds_char* lds = (lds_char*)sy_lds;
  const uint32_t lds_base = (uint32_t)(uintptr_t)lds;

  // XCD-aware order (workgroup b runs on XCD b % 8).  Several splits: all workgroups of one row
  // split land on the same XCD, so the X rows they share are fetched into that XCD's L2 once.  One
  // split: each XCD takes a contiguous range of the tiles in blocked order, so the workgroups it
  // runs at once read few distinct panels of the same rows.  Tiles are numbered row-major over the
  // triangle for the partial sums.
  int t, split;
  {
    const int bid = blockIdx.x;
    if (ksplit == 1) {
      const int q = tiles / SY_XCD, rem = tiles % SY_XCD, x = bid % SY_XCD, slot = bid / SY_XCD;
      if (slot >= q + (x < rem ? 1 : 0)) return;  // the grid is rounded up to a multiple of 8
      split = 0;
      t = x * q + min(x, rem) + slot;
    } else if (ksplit % SY_XCD == 0) {
      const int per = SY_XCD * tiles;
      split = (bid % SY_XCD) + SY_XCD * (bid / per);
      t = (bid / SY_XCD) % tiles;
    } else {
      split = bid / tiles;
      t = bid % tiles;
    }
  }
  int I, J;
  blocked_tile<6, 6>(t, (n + SY_T - 1) / SY_T, I, J);
  const int tile = I * (I + 1) / 2 + J;
  const int64_t r0 = (int64_t)split * rows_per_split;
  const int64_t r1 = r0 + rows_per_split < rows ? r0 + rows_per_split : rows;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wi = wave >> 2, wj = wave & 3;

  // DMA sources: block b = 2 wave + u of a panel holds stage rows 2b, 2b + 1.
  uint32_t offA[2], offB[2], ldsoff[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int b = 2 * wave + u, row = 2 * b + (lane >> 5), c = (lane & 31) ^ (4 * (row & 3));
    offA[u] = (uint32_t)(row * ldx + min(SY_T * I + 8 * c, n - 8)) * 2u;
    offB[u] = (uint32_t)(row * ldx + min(SY_T * J + 8 * c, n - 8)) * 2u;
    ldsoff[u] = b * 1024 + lane * 16;
  }

  auto issue = [&](int64_t st, int slot) {
    const int64_t k0 = r0 + st * SY_KT;
    const uint32_t sbase = lds_base + slot * SY_STAGE_BYTES;
    if (k0 + SY_KT <= r1) {
      const uint16_t* ga = XA + k0 * ldx;
      const uint16_t* gb = XB + k0 * ldx;
#pragma unroll
      for (int u = 0; u < 2; ++u) lds_dma16(ga, offA[u], sbase + (2 * wave + u) * 1024);
#pragma unroll
      for (int u = 0; u < 2; ++u) lds_dma16(gb, offB[u], sbase + SY_PANEL + (2 * wave + u) * 1024);
    } else {
      // ragged last stage: bounds-checked loads through registers, zeros past r1
      lds_char* dst = lds + slot * SY_STAGE_BYTES;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int row = 2 * (2 * wave + u) + (lane >> 5);
        u32x4 va = u32x4{0u, 0u, 0u, 0u}, vb = va;
        if (k0 + row < r1) {
          va = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(XA + k0 * ldx) + offA[u]);
          vb = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(XB + k0 * ldx) + offB[u]);
        }
        *(__attribute__((address_space(3))) u32x4*)(dst + ldsoff[u]) = va;
        *(__attribute__((address_space(3))) u32x4*)(dst + SY_PANEL + ldsoff[u]) = vb;
      }
    }
  };

  // Transposing-read addresses.  Lane l (g = l / 16, t = (l / 4) % 4, q = l % 4) reads
  // row 8 (g / 2) + t (+ 4 for the second half) at features base + 16 (g % 2) + 4 q.
  uint32_t rdA[4], rdB[2];
  {
    const int g = lane >> 4, t = (lane >> 2) & 3, q = lane & 3;
    const int krow = 8 * (g >> 1) + t;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int f = 128 * wi + 32 * x + 16 * (g & 1) + 4 * q;
      rdA[x] = krow * (SY_T * 2) + (((f >> 3) ^ (4 * t)) << 4) + (f & 7) * 2;
    }
#pragma unroll
    for (int y = 0; y < 2; ++y) {
      const int f = 64 * wj + 32 * y + 16 * (g & 1) + 4 * q;
      rdB[y] = SY_PANEL + krow * (SY_T * 2) + (((f >> 3) ^ (4 * t)) << 4) + (f & 7) * 2;
    }
  }

  static_assert(SY_KT == 32, "two 16-row steps per stage");
  // Operand double buffer: set 0 holds rows 0..15 of a stage, set 1 rows 16..31.
  bf16x8 a0[4], b0[2], a1[4], b1[2];
  auto read_frags = [&](int slot, int u, bf16x8 (&fa)[4], bf16x8 (&fb)[2]) {
    const lds_char* st = lds + slot * SY_STAGE_BYTES + 16 * u * (SY_T * 2);
#pragma unroll
    for (int x = 0; x < 4; ++x) fa[x] = tr_frag(st + rdA[x], 4 * SY_T * 2);
#pragma unroll
    for (int y = 0; y < 2; ++y) fb[y] = tr_frag(st + rdB[y], 4 * SY_T * 2);
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y) acc[x][y] = f32x16{};
  auto mfma_step = [&](const bf16x8 (&fa)[4], const bf16x8 (&fb)[2]) {
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int y = 0; y < 2; ++y) acc[x][y] = mfma32x32x16_bf16(fa[x], fb[y], acc[x][y]);
  };

  // Pipeline: DMAs run SY_PF stages ahead; the operands of the first 16 rows of
  // stage s + 1 are read (after the barrier that publishes that stage) while the
  // MFMAs of the last 16 rows of stage s execute.
  const int64_t nst = r1 > r0 ? (r1 - r0 + SY_KT - 1) / SY_KT : 0;
  for (int64_t p = 0; p < SY_PF && p < nst; ++p) issue(p, (int)p);
  if (nst > 0) {
    if (nst - 1 > SY_PF - 1) {
      vm_wait<SY_DMA_PER_WAVE * (SY_PF - 1)>();
    } else {
      vm_wait<0>();
    }
    lds_barrier();
    read_frags(0, 0, a0, b0);
  }
  int slot = 0;
  for (int64_t s = 0; s < nst; ++s) {
    read_frags(slot, 1, a1, b1);
    mfma_step(a0, b0);
    const int next = slot == SY_NS - 1 ? 0 : slot + 1;
    if (s + 1 < nst) {
      // Stage s + 1 has landed once at most the DMAs of stages s + 2 .. s + SY_PF - 1
      // are outstanding; those are all full DMA stages unless the ragged last one
      // (or a stage past the end) is among them.
      if (s + SY_PF - 1 <= nst - 2) {
        vm_wait<SY_DMA_PER_WAVE * (SY_PF - 2)>();
      } else {
        vm_wait<0>();
      }
      lds_barrier();
      // the slot of stage s is free: every wave finished its reads of it before this barrier (the
      // second half was read at the top of this iteration, the first half in the previous one)
      // waves 0-3 refill the slot now, waves 4-7 (the other wave on each SIMD) after their MFMAs, so
      // that one wave of a SIMD issues matrix work while the other waits to hand over its DMAs
      if (s + SY_PF < nst && wave < 4) issue(s + SY_PF, slot);
      read_frags(next, 0, a0, b0);
    }
    mfma_step(a1, b1);
    if (s + 1 < nst && s + SY_PF < nst && wave >= 4) issue(s + SY_PF, slot);
    slot = next;
  }

#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int ii = 128 * wi + 32 * x + acc_row(v, lane);
        const int jj = 64 * wj + 32 * y + (lane & 31);
        if (partial) {
          partial[(((size_t)split * tiles + tile) * SY_T + ii) * SY_T + jj] = acc[x][y][v];
        } else {
          const int gi = SY_T * I + ii, gj = SY_T * J + jj;
          if (gi < n && gj < n && gi >= gj) S[(size_t)gi * n + gj] += (double)acc[x][y][v];
        }
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
__global__ void syrk_reduce_kernel(const float* __restrict__ partial, int ksplit, int tiles, int n,
                                   double* __restrict__ S) {
  const int tile = blockIdx.y;
  int I, J;
  tri_tile(tile, I, J);
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= SY_T * SY_T) return;
  const int ii = e / SY_T, jj = e - ii * SY_T;
  const int gi = SY_T * I + ii, gj = SY_T * J + jj;
  if (gi >= n || gj >= n || gi < gj) return;
  const size_t stride = (size_t)tiles * SY_T * SY_T;
  const float* p = partial + (size_t)tile * SY_T * SY_T + e;
  double acc = 0.0;
  int s = 0;
  for (; s + 4 <= ksplit; s += 4) {
    const float a = p[(size_t)s * stride], b = p[(size_t)(s + 1) * stride], c = p[(size_t)(s + 2) * stride],
                d = p[(size_t)(s + 3) * stride];
    acc += (double)a;
    acc += (double)b;
    acc += (double)c;
    acc += (double)d;
  }
  for (; s < ksplit; ++s) acc += (double)p[(size_t)s * stride];
  S[(size_t)gi * n + gj] += acc;
}

__global__ void zero_lower_kernel(double* S, int n) {
  const int i = blockIdx.x;
  for (int j = threadIdx.x; j <= i; j += blockDim.x) S[(size_t)i * n + j] = 0.0;
}

}  // namespace wr

using namespace wr;

// Row splits are chosen for a 256-CU part so the workspace size does not depend on the device.
static constexpr int kSplitCUs = 256;

// Workgroups of a launch: one per tile and split; with one split rounded up to a multiple of the XCD
// count (the surplus workgroups return at once).
static int syrk_grid(int tiles, int ks) { return ks == 1 ? (tiles + SY_XCD - 1) / SY_XCD * SY_XCD : tiles * ks; }

static int syrk_tiles(int64_t n) {
  const int nt = (int)((n + SY_T - 1) / SY_T);
  return nt * (nt + 1) / 2;
}

// Number of row splits.  A split is summed in fp32 by the MFMAs over at most 32768 rows.  When
// the lower 256 x 256 tiles alone give at least one workgroup per CU there is one split per tile
// and each workgroup adds its sums into S (fp64) itself: no partial buffer (the host then
// launches once per 32768-row slice).
// Otherwise the rows are cut into enough splits to fill the CUs (and to keep each at most 16384
// rows); from 8 splits up their number is a multiple of the XCD count (each XCD works through its
// own rows).  With `precise` (the fp32-input path, whose six passes rebuild an fp32-accurate S)
// a split is at most 512 rows.
static int syrk_ksplit(int64_t rows, int64_t n, int num_cu, bool precise) {
  if (rows <= 0) return 1;
  if (precise) return (int)std::min<int64_t>(64, (rows + 511) / 512);
  const int tiles = syrk_tiles(n);
  if (tiles >= num_cu) return 1;
  if (rows < SY_XCD * 1024) return (int)std::max<int64_t>(1, rows / 1024);
  int64_t ks = std::max<int64_t>((rows + SY_SPLIT_ROWS - 1) / SY_SPLIT_ROWS, (num_cu + tiles - 1) / tiles);
  if (ks >= SY_XCD) {
    ks = (ks + SY_XCD - 1) / SY_XCD * SY_XCD;
    while (ks < 64 && tiles * ks < num_cu && rows / (ks + SY_XCD) >= 1024) ks += SY_XCD;
  }
  return (int)std::min<int64_t>(ks, 64);
}

static size_t partial_bytes(int64_t rows, int64_t n, bool precise) {
  const int ks = syrk_ksplit(rows, n, kSplitCUs, precise);
  return ks > 1 ? (size_t)ks * syrk_tiles(n) * SY_T * SY_T * sizeof(float) : 0;
}

size_t wr_hessian_ws_bytes(int64_t rows, int64_t n, int x_dtype, int num_cu) {
  (void)num_cu;
  size_t bytes = 256 + ((partial_bytes(rows, n, x_dtype == WR_F32) + 255) & ~(size_t)255);
  if (x_dtype == WR_F32) bytes += 3 * (((size_t)rows * n * 2 + 255) & ~(size_t)255);
  return bytes;
}

// One SYRK pass S_lower += XA^T XB (bf16 sources, ld ldx), with its split-K reduction.
static int syrk_pass(wr_ctx* ctx, const uint16_t* XA, const uint16_t* XB, int64_t rows, int64_t n, int64_t ldx,
                     double* S, float* partial, bool precise, int ks_cap = 64) {
  if (!lds_limit((const void*)syrk_bf16_kernel, SY_LDS_BYTES)) return WR_EHIP;
  hipStream_t st = ctx->stream;
  const int tiles = syrk_tiles(n);
  const int ks = std::min(syrk_ksplit(rows, n, kSplitCUs, precise), std::max(ks_cap, 1));
  if (ks == 1 && rows > SY_MAX_ROWS) {
    for (int64_t r0 = 0; r0 < rows; r0 += SY_MAX_ROWS) {
      const int64_t rc = std::min<int64_t>(SY_MAX_ROWS, rows - r0);
      hipLaunchKernelGGL(syrk_bf16_kernel, dim3((unsigned)syrk_grid(tiles, 1)), dim3(SY_THREADS), SY_LDS_BYTES, st,
                         XA + r0 * ldx, XB + r0 * ldx, rc, (int)n, ldx, rc, tiles, 1, S, nullptr);
      WR_CHECK_LAUNCH();
    }
    return WR_OK;
  }
  const int64_t rps = ((rows + ks - 1) / ks + SY_KT - 1) / SY_KT * SY_KT;
  hipLaunchKernelGGL(syrk_bf16_kernel, dim3((unsigned)syrk_grid(tiles, ks)), dim3(SY_THREADS), SY_LDS_BYTES, st, XA, XB,
                     rows, (int)n, ldx, rps, tiles, ks, S, ks > 1 ? partial : nullptr);
  WR_CHECK_LAUNCH();
  if (ks > 1) {
    dim3 rgrid((unsigned)((SY_T * SY_T + 255) / 256), (unsigned)tiles);
    hipLaunchKernelGGL(syrk_reduce_kernel, rgrid, dim3(256), 0, st, partial, ks, tiles, (int)n, S);
    WR_CHECK_LAUNCH();
  }
  return WR_OK;
}

int wr_hessian_accumulate_impl(wr_ctx* ctx, const void* X, int x_dtype, int64_t rows, int64_t n, int64_t ldx,
                               double* S, int flags) {
  hipStream_t st = ctx->stream;
  if (rows > 0 && ctx->ws_bytes < wr_hessian_ws_bytes(rows, n, x_dtype, kSplitCUs)) return WR_EWORKSPACE;
  if (flags & WR_H_ZERO) {
    hipLaunchKernelGGL(zero_lower_kernel, dim3((unsigned)n), dim3(256), 0, st, S, (int)n);
    WR_CHECK_LAUNCH();
  }
  if (rows == 0) return WR_OK;
  char* ws = static_cast<char*>(ctx->ws);
  float* partial = reinterpret_cast<float*>(ws + 256);
  if (x_dtype == WR_BF16) {
    const uint16_t* Xb = static_cast<const uint16_t*>(X);
    return syrk_pass(ctx, Xb, Xb, rows, n, ldx, S, partial, false);
  }
  const size_t plane = ((size_t)rows * n * 2 + 255) & ~(size_t)255;
  uint16_t* P[3];
  for (int k = 0; k < 3; ++k)
    P[k] = reinterpret_cast<uint16_t*>(ws + 256 + ((partial_bytes(rows, n, true) + 255) & ~(size_t)255) + k * plane);
  const unsigned gx = (unsigned)std::min<int64_t>((n + 255) / 256, 16);
  hipLaunchKernelGGL(split3_kernel, dim3(gx, (unsigned)rows), dim3(256), 0, st, static_cast<const float*>(X), rows,
                     (int)n, ldx, P[0], P[1], P[2]);
  WR_CHECK_LAUNCH();
  static const int terms[6][2] = {{2, 0}, {1, 1}, {0, 2}, {1, 0}, {0, 1}, {0, 0}};  // small terms first
  for (const auto& t : terms) {
    const int rc = syrk_pass(ctx, P[t[0]], P[t[1]], rows, n, n, S, partial, true);
    if (rc) return rc;
  }
  return WR_OK;
}

// ---------------------------------------------------------------- allocation-free variant
// Device scratch of the allocation-free accumulate: a file-scope array, one copy per GPU, held
// until the process ends.  In host code `scratch` names a host-side stand-in, never the device
// memory: its device address comes from hipGetSymbolAddress, taken once per device (with that
// device current) by wr_static_scratch_init, which wr_create calls; only that address reaches
// the kernels.
static __device__ __align__(256) unsigned char scratch[WR_STATIC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

int wr_static_scratch_init(int device) {
  if (device < 0 || device >= kMaxDevices) return WR_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[device]) return WR_OK;
  int prev = -1;
  if (hipGetDevice(&prev) != hipSuccess) return WR_EHIP;
  if (prev != device && hipSetDevice(device) != hipSuccess) return WR_EHIP;
  void* ptr = nullptr;
  const hipError_t err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (prev != device) (void)hipSetDevice(prev);
  if (err != hipSuccess || !ptr) return WR_EHIP;
  g_scratch_ptr[device] = ptr;
  return WR_OK;
}

static void* static_scratch(int device) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  return device >= 0 && device < kMaxDevices ? g_scratch_ptr[device] : nullptr;
}

// Partial-sum bytes of k row splits of the fp32 path (a single split adds into S directly).
static size_t f32_partial_bytes(int64_t k, int64_t n) {
  return k > 1 ? (((size_t)k * syrk_tiles(n) * SY_T * SY_T * sizeof(float) + 255) & ~(size_t)255) : 0;
}

// Rows of fp32 input whose three bf16 planes and split partials fit in `bytes` (512 k rows for
// k splits of 512 rows, the split length of the fp32 path), or 0 when not even 512 rows fit.
static int64_t f32_rows_fitting(int64_t n, size_t bytes) {
  for (int64_t k = 64; k >= 1; k /= 2) {
    const int64_t c = 512 * k;
    const size_t need = 256 + f32_partial_bytes(k, n) + 3 * (((size_t)c * n * 2 + 255) & ~(size_t)255);
    if (need <= bytes) return c;
  }
  return 0;
}

// Same result as wr_hessian_accumulate_impl (bit-identical when its workspace need fits the static
// scratch), with the scratch taken from the per-device static array: bf16 input with fewer row
// splits at a time when their partials would not fit (each split still sums at most 32768 rows in
// fp32), fp32 input in row slices whose bf16 planes and partials fit.
int wr_hessian_accumulate_static_impl(wr_ctx* ctx, const void* X, int x_dtype, int64_t rows, int64_t n,
                                      int64_t ldx, double* S, int flags) {
  char* ws = static_cast<char*>(static_scratch(ctx->device));
  if (!ws) return WR_EHIP;
  const size_t cap = WR_STATIC_SCRATCH_BYTES;
  hipStream_t st = ctx->stream;
  if (rows > 0 && x_dtype == WR_F32 && f32_rows_fitting(n, cap) == 0) return WR_ESCRATCH;
  if (flags & WR_H_ZERO) {
    hipLaunchKernelGGL(zero_lower_kernel, dim3((unsigned)n), dim3(256), 0, st, S, (int)n);
    WR_CHECK_LAUNCH();
  }
  if (rows == 0) return WR_OK;
  float* partial = reinterpret_cast<float*>(ws + 256);
  const size_t part = (size_t)syrk_tiles(n) * SY_T * SY_T * sizeof(float);
  if (x_dtype == WR_BF16) {
    const uint16_t* Xb = static_cast<const uint16_t*>(X);
    const int ks_fit = (int)std::min<size_t>(64, (cap - 256) / part);
    if (ks_fit >= syrk_ksplit(rows, n, kSplitCUs, false))
      return syrk_pass(ctx, Xb, Xb, rows, n, ldx, S, partial, false);
    if (ks_fit < 2) return syrk_pass(ctx, Xb, Xb, rows, n, ldx, S, partial, false, 1);
    const int64_t slice = (int64_t)ks_fit * SY_MAX_ROWS;
    for (int64_t r0 = 0; r0 < rows; r0 += slice) {
      const int rc = syrk_pass(ctx, Xb + r0 * ldx, Xb + r0 * ldx, std::min(slice, rows - r0), n, ldx, S, partial,
                               false, ks_fit);
      if (rc) return rc;
    }
    return WR_OK;
  }
  const int64_t slice = f32_rows_fitting(n, cap);
  const size_t plane_cap = ((size_t)slice * n * 2 + 255) & ~(size_t)255;
  const int kmax = (int)(slice / 512);
  uint16_t* P[3];
  for (int k = 0; k < 3; ++k)
    P[k] = reinterpret_cast<uint16_t*>(ws + 256 + f32_partial_bytes(kmax, n) + k * plane_cap);
  const float* Xf = static_cast<const float*>(X);
  static const int terms[6][2] = {{2, 0}, {1, 1}, {0, 2}, {1, 0}, {0, 1}, {0, 0}};  // small terms first
  for (int64_t r0 = 0; r0 < rows; r0 += slice) {
    const int64_t rc_rows = std::min(slice, rows - r0);
    const unsigned gx = (unsigned)std::min<int64_t>((n + 255) / 256, 16);
    hipLaunchKernelGGL(split3_kernel, dim3(gx, (unsigned)rc_rows), dim3(256), 0, st, Xf + r0 * ldx, rc_rows, (int)n,
                       ldx, P[0], P[1], P[2]);
    WR_CHECK_LAUNCH();
    for (const auto& t : terms) {
      const int rc = syrk_pass(ctx, P[t[0]], P[t[1]], rc_rows, n, n, S, partial, true, kmax);
      if (rc) return rc;
    }
  }
  return WR_OK;
}
