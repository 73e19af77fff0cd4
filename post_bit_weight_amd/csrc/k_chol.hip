// Factorisation for the error-feedback sweep: H = M D M^T with M unit upper.
//
// LDLQ (Pingala-8 post, "Trick 2: round with error feedback") pushes each
// column's rounding error onto the later columns in proportions set by H; the
// proportions are the entries of the unit upper factor M of H = M D M^T.  With J
// the reversal permutation, L = chol_lower(J H J) gives H = V V^T for the upper
// V = J L J, and M = V diag(V)^-1: only a Cholesky factorisation is needed, no
// inverse of the whole matrix.
//
// fp64 blocked right-looking Cholesky, block CB = 64.  A diagonal block is
// factored by one workgroup in 16 x 16 blocks: each diagonal 16 x 16 block is
// factored and its factor inverted at once by one wave in registers (rows of A
// and columns of the identity side by side in the lanes, pivot columns broadcast
// with readlane), the rest are fp64 MFMA products in LDS.  Per block column kb one
// kernel, chol_step_kernel: every workgroup solves for the blocks of the factor's
// block column kb that it needs (a blocked triangular solve with the inverted
// 16 x 16 diagonal blocks, on the fp64 matrix cores), then workgroup 0 updates and
// factors the next diagonal block while the others update one trailing tile each,
// A_ij -= L_ik L_jk^T.  Recomputing a block column's solve per tile costs fp64
// matrix-core time that runs in parallel; it removes a dependent launch, a global
// round trip and a reload from the serial chain of diagonal blocks.
// A pivot that is not positive sets dev_info (1-based pivot of J H J) and every
// later kernel returns at once.
#include "chol16.hpp"

namespace wr {

constexpr int CB = 64;        // block edge
constexpr int CP = CB + 1;    // LDS row pitch in doubles: rows start on different banks
constexpr int CU_XCD = 8;     // workgroups are dispatched round-robin over 8 XCDs

__device__ __forceinline__ void lds_sync() { lds_sync_f64(); }

// Copy a 64 x 64 fp64 block (rows r0.., columns c0.. of a matrix with leading dimension ld)
// into LDS at pitch CP; entries outside [0, nr) x [0, nc) read as zero.  256 threads,
// each moving 8 pairs of doubles: every load is issued before the first LDS store.
__device__ __forceinline__ void load_block64(const double* __restrict__ G, int64_t ld, int r0, int c0, int nr, int nc,
                                             double* sM, int tid) {
  double2 v[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int e = tid + 256 * q;  // pair index: row e / 32, columns 2 (e % 32) .. +1
    const int r = e >> 5, c = 2 * (e & 31);
    const bool ok = r0 + r < nr && c0 + c + 1 < nc;  // nc is even
    const int64_t off = ok ? (int64_t)(r0 + r) * ld + c0 + c : 0;
    v[q] = *reinterpret_cast<const double2*>(G + off);
    if (!ok) v[q] = double2{0.0, 0.0};
  }
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int e = tid + 256 * q;
    const int r = e >> 5, c = 2 * (e & 31);
    sM[r * CP + c] = v[q].x;
    sM[r * CP + c + 1] = v[q].y;
  }
}

__device__ __forceinline__ int chol16_inv_wave(double* sM, double* sX, int o, int lane) {
  return chol16_inv_pitch<CP>(sM + o * CP + o, sX + o * CP + o, lane);
}

// acc[x][y] += A_x B_y^T over K for the 16 x 16 blocks A_x = rows r0 + 16 x of SA and B_y = rows
// c0 + 16 y of SB (both at pitch CP, k along the row): per k step the two row and two column
// fragments feed four independent MFMAs (each accumulator still sums its k steps in order).
__device__ __forceinline__ void mma16_2x2(const double* SA, int r0, const double* SB, int c0, int K,
                                          f64x4 (&acc)[2][2], int lane) {
  const int li = lane & 15, lk = lane >> 4;
#pragma unroll 4
  for (int k0 = 0; k0 < K; k0 += 4) {
    double fa[2], fb[2];
#pragma unroll
    for (int x = 0; x < 2; ++x) fa[x] = SA[(r0 + 16 * x + li) * CP + k0 + lk];
#pragma unroll
    for (int y = 0; y < 2; ++y) fb[y] = SB[(c0 + 16 * y + li) * CP + k0 + lk];
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int y = 0; y < 2; ++y) acc[x][y] = __builtin_amdgcn_mfma_f64_16x16x4f64(fa[x], fb[y], acc[x][y], 0, 0, 0);
  }
}

// Factor the 64 x 64 diagonal block at kb held in sA (lower part valid, strict upper
// part zero, identity past n) as L_kk, by 16 x 16 blocks: per block column s, wave 0
// factors the diagonal block and inverts its factor (X_ss), the blocks below become
// L_is = A_is X_ss^T, and the trailing blocks take A_ij -= L_is L_js^T on the fp64
// matrix cores.  Wave 0 updates and factors the next diagonal block while waves 1-3
// update the rest.  L_kk goes to L; the four X_ss to Xinv ([4][16][16], compact).
// With first_done, wave 0 has already factored the first 16 x 16 block (its first bad
// pivot, or -1, in bad0).  sX needs no initial contents.  A pivot that is not
// positive sets dev_info (first failure wins).
__device__ __forceinline__ void diag_factor(double* sA, double* sX, int n, int kb, double* L, double* Xinv,
                                            int32_t* dev_info, int tid, bool first_done = false, int bad0 = -1,
                                            int nthr = 256) {
  const int lane = tid & 63, wave = tid >> 6;
  const f64x4 zero = {0.0, 0.0, 0.0, 0.0};
  int bad = bad0;
  if (!first_done) {
    if (wave == 0) bad = chol16_inv_wave(sA, sX, 0, lane);
    lds_sync();
  }
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int o = 16 * s;
    if (wave < 3 - s) {  // L_is = A_is X_ss^T
      const int i0 = 16 * (s + 1 + wave);
      const f64x4 acc = mma16<true>(sA + o, CP, i0, sX + o, CP, o, 16, zero, lane);
#pragma unroll
      for (int v = 0; v < 4; ++v) sA[(i0 + (lane >> 4) + 4 * v) * CP + o + (lane & 15)] = acc[v];
    }
    lds_sync();
    if (s == 3) break;
    const int nx = 16 * (s + 1);
    if (wave == 0) {
      const f64x4 acc = mma16<true>(sA + o, CP, nx, sA + o, CP, nx, 16, zero, lane);
#pragma unroll
      for (int v = 0; v < 4; ++v) sA[(nx + (lane >> 4) + 4 * v) * CP + nx + (lane & 15)] -= acc[v];
      const int b = chol16_inv_wave(sA, sX, nx, lane);
      if (bad < 0 && b >= 0) bad = nx + b;
    } else {
      // trailing blocks (i, j), s + 1 <= j <= i <= 3, other than (s + 1, s + 1)
      int t = 0;
      for (int i = s + 1; i < 4; ++i)
        for (int j = s + 1; j <= i; ++j) {
          if (i == s + 1 && j == s + 1) continue;
          if (t++ % 3 != wave - 1) continue;
          const f64x4 acc = mma16<true>(sA + o, CP, 16 * i, sA + o, CP, 16 * j, 16, zero, lane);
#pragma unroll
          for (int v = 0; v < 4; ++v) sA[(16 * i + (lane >> 4) + 4 * v) * CP + 16 * j + (lane & 15)] -= acc[v];
        }
    }
    lds_sync();
  }
  if (wave == 0 && lane == 0 && bad >= 0) atomicCAS(dev_info, 0, kb + bad + 1);
  for (int e = tid; e < 4 * 256; e += nthr) {  // X_ss, compact: [s][16][16]
    const int b = e >> 8, r = (e >> 4) & 15, c = e & 15;
    Xinv[e] = sX[(16 * b + r) * CP + 16 * b + c];
  }
  for (int e = tid; e < CB * CB; e += nthr) {
    const int r = e / CB, c = e % CB;
    if (c <= r && kb + r < n) L[(int64_t)(kb + r) * n + kb + c] = sA[r * CP + c];
  }
}

// The inverted diagonal 16 x 16 blocks, stored compactly as [4][16][16], into sX at (16 s, 16 s).
__device__ __forceinline__ void load_xd(const double* __restrict__ Xc, double* sX, int tid) {
  double2 v[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) v[q] = *reinterpret_cast<const double2*>(Xc + 2 * (tid + 256 * q));
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int e = 2 * (tid + 256 * q), b = e >> 8, r = (e >> 4) & 15, c = e & 15;
    sX[(16 * b + r) * CP + 16 * b + c] = v[q].x;
    sX[(16 * b + r) * CP + 16 * b + c + 1] = v[q].y;
  }
}

// Rows past n of the last, partial block: the identity.  (Entries above the diagonal
// of a diagonal block are never read into the lower part, so they need no clearing.)
__device__ __forceinline__ void pad_diag(double* sA, int n, int kb, int tid, int nthr = 256) {
  if (kb + CB <= n) return;
  for (int e = tid; e < CB * CB; e += nthr) {
    const int r = e / CB, c = e % CB;
    if (kb + r >= n && c <= r) sA[r * CP + c] = r == c ? 1.0 : 0.0;
  }
}

// The diagonal block at kb (its trailing update done): factor it (L) and invert its 16 x 16 blocks.
__global__ __launch_bounds__(256) void chol_diag_kernel(const double* __restrict__ A, int n, int kb, double* __restrict__ L,
                                                        double* __restrict__ Xinv, int32_t* __restrict__ dev_info) {
  if (*dev_info != 0) return;
  __shared__ double sA[CB * CP];
  __shared__ double sX[CB * CP];
  const int tid = threadIdx.x;
  load_block64(A, n, kb, kb, n, n, sA, tid);
  __syncthreads();
  pad_diag(sA, n, kb, tid);
  __syncthreads();
  diag_factor(sA, sX, n, kb, L, Xinv, dev_info, tid);
}

// Blocked triangular solve P L_kk^T = A in place for rows 16 w .. 16 w + 15 of a 64-row
// tile in sP (one wave): P_s = (A_s - sum_{t<s} P_t L_st^T) X_ss^T per 16-column block,
// with L_kk in sL and its inverted diagonal 16 x 16 blocks X_ss in sX.  The wave only
// touches its own rows of sP.
__device__ __forceinline__ void panel_rows(double* sP, const double* sL, const double* sX, int wave, int lane) {
  const int w0 = 16 * wave;
  const f64x4 zero = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int o = 16 * s;
    f64x4 acc;
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[v] = sP[(w0 + (lane >> 4) + 4 * v) * CP + o + (lane & 15)];
#pragma unroll
    for (int t = 0; t < s; ++t) acc = mma16<true, true>(sP + 16 * t, CP, w0, sL + 16 * t, CP, o, 16, acc, lane);
#pragma unroll
    for (int v = 0; v < 4; ++v) sP[(w0 + (lane >> 4) + 4 * v) * CP + o + (lane & 15)] = acc[v];
    acc = mma16<true>(sP + o, CP, w0, sX + o, CP, o, 16, zero, lane);
#pragma unroll
    for (int v = 0; v < 4; ++v) sP[(w0 + (lane >> 4) + 4 * v) * CP + o + (lane & 15)] = acc[v];
  }
}

// Store the 64 x 64 block sM to L at (r0, c0) (rows past n skipped).
__device__ __forceinline__ void store_block64(const double* sM, double* __restrict__ L, int n, int r0, int c0, int tid) {
  for (int e = tid; e < CB * CB; e += 256) {
    const int r = e / CB, c = e % CB;
    if (r0 + r < n) L[(int64_t)(r0 + r) * n + c0 + c] = sM[r * CP + c];
  }
}

// The block column kb of the factor below the diagonal, L_ik = A_ik L_kk^-T for every block row
// i > k, one workgroup per block row, written to L: the first phase of a step whose trailing
// matrix has many tiles (then chol_step_kernel reads the panels instead of solving them in
// every tile).
__global__ __launch_bounds__(256) void chol_panel_kernel(const double* __restrict__ A, double* __restrict__ L,
                                                         const double* __restrict__ Xin, int n, int kb,
                                                         const int32_t* __restrict__ dev_info) {
  if (*dev_info != 0) return;
  __shared__ double sL[CB * CP];
  __shared__ double sX[CB * CP];
  __shared__ double sP[CB * CP];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i0 = kb + CB + CB * blockIdx.x;
  load_xd(Xin, sX, tid);
  load_block64(L, n, kb, kb, n, n, sL, tid);
  load_block64(A, n, i0, kb, n, n, sP, tid);
  lds_sync();
  panel_rows(sP, sL, sX, wave, lane);
  lds_sync();
  store_block64(sP, L, n, i0, kb, tid);
}

// Step kb, after the diagonal block kb is factored (L_kk in L, its inverted 16 x 16
// diagonal blocks in Xin).  Every workgroup solves for the factor's blocks that it needs
// from the block column A[.., kb..kb+63] itself, so no workgroup waits for another; with
// panels_ready those blocks are already in L (chol_panel_kernel) and are read instead.
//   workgroup 0:   L_{k+1,k}, then the next diagonal block A_{k+1,k+1} - L_{k+1,k} L_{k+1,k}^T,
//                  factored and inverted (to L and Xout), then L_{k+1,k} to L;
//   workgroup t:   trailing lower tile (ti, tj) != (0, 0): L_ik, L_jk, A_ij -= L_ik L_jk^T;
//                  the tiles of the first trailing column (tj = 0) also write L_ik.
// Xin and Xout are different buffers (workgroup 0 writes Xout while the others read Xin).
__global__ __launch_bounds__(256) void chol_step_kernel(double* __restrict__ A, double* __restrict__ L,
                                                        const double* __restrict__ Xin, double* __restrict__ Xout,
                                                        int n, int kb, int panels_ready, int wcols,
                                                        int32_t* __restrict__ dev_info) {
  if (*dev_info != 0) return;
  __shared__ double sL[CB * CP];
  __shared__ double sX[CB * CP];
  __shared__ double sP[CB * CP];
  __shared__ double sQ[CB * CP];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int base = kb + CB;
  const f64x4 zero = {0.0, 0.0, 0.0, 0.0};
  if (blockIdx.x == 0) {
    if (panels_ready) {
      load_block64(L, n, base, kb, n, n, sP, tid);
      load_block64(A, n, base, base, n, n, sQ, tid);
      lds_sync();
      pad_diag(sQ, n, base, tid);
    } else {
      load_xd(Xin, sX, tid);
      load_block64(L, n, kb, kb, n, n, sL, tid);
      load_block64(A, n, base, kb, n, n, sP, tid);
      load_block64(A, n, base, base, n, n, sQ, tid);
      lds_sync();
      pad_diag(sQ, n, base, tid);
      panel_rows(sP, sL, sX, wave, lane);
      lds_sync();
      store_block64(sP, L, n, base, kb, tid);  // L_{k+1,k}; nothing in this kernel reads it back
    }
    // next diagonal block sQ -= sP sP^T: wave 0 takes the first 16 x 16 block and factors it
    // at once, waves 1-3 take the other nine lower blocks
    int bad0 = -1;
    if (wave == 0) {
      const f64x4 acc = mma16<true>(sP, CP, 0, sP, CP, 0, CB, zero, lane);
#pragma unroll
      for (int v = 0; v < 4; ++v) sQ[((lane >> 4) + 4 * v) * CP + (lane & 15)] -= acc[v];
      bad0 = chol16_inv_wave(sQ, sX, 0, lane);
    } else {
      for (int t = wave; t < 10; t += 3) {
        const int bi = t < 3 ? 1 : t < 6 ? 2 : 3;
        const int bj = t - bi * (bi + 1) / 2;
        const f64x4 acc = mma16<true>(sP, CP, 16 * bi, sP, CP, 16 * bj, CB, zero, lane);
#pragma unroll
        for (int v = 0; v < 4; ++v) sQ[(16 * bi + (lane >> 4) + 4 * v) * CP + 16 * bj + (lane & 15)] -= acc[v];
      }
    }
    lds_sync();
    diag_factor(sQ, sX, n, base, L, Xout, dev_info, tid, true, bad0);
    return;
  }
  int ti, tj;
  {
    // lower tiles in row-major order, only the first wcols tile columns; tile 0 is the diagonal
    // block above
    const int t = blockIdx.x, tri = wcols * (wcols + 1) / 2;
    if (t < tri) {
      int i = (int)((sqrtf(8.0f * (float)t + 1.0f) - 1.0f) * 0.5f);
      while (i * (i + 1) / 2 > t) --i;
      while ((i + 1) * (i + 2) / 2 <= t) ++i;
      ti = i;
      tj = t - i * (i + 1) / 2;
    } else {
      ti = wcols + (t - tri) / wcols;
      tj = (t - tri) % wcols;
    }
  }
  const int i0 = base + CB * ti, j0 = base + CB * tj;
  const bool diag = ti == tj;
  const int wi = wave >> 1, wj = wave & 1;
  const bool active = !(diag && wj > wi);  // strictly upper 32 x 32 quarter of a diagonal tile: nothing to do
  // the wave's 32 x 32 part of A_ij, fetched first so that its latency overlaps the solves
  double cur[2][2][4];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int gi = i0 + 32 * wi + 16 * x + (lane >> 4) + 4 * v;
        const int gj = j0 + 32 * wj + 16 * y + (lane & 15);
        cur[x][y][v] = active && gi < n && gj < n ? A[(int64_t)gi * n + gj] : 0.0;
      }
  if (panels_ready) {
    load_block64(L, n, i0, kb, n, n, sP, tid);
    if (!diag) load_block64(L, n, j0, kb, n, n, sQ, tid);
    lds_sync();
  } else {
    load_xd(Xin, sX, tid);
    load_block64(L, n, kb, kb, n, n, sL, tid);
    load_block64(A, n, i0, kb, n, n, sP, tid);
    if (!diag) load_block64(A, n, j0, kb, n, n, sQ, tid);
    lds_sync();
    panel_rows(sP, sL, sX, wave, lane);
    if (!diag) panel_rows(sQ, sL, sX, wave, lane);
    lds_sync();
    if (tj == 0) store_block64(sP, L, n, i0, kb, tid);
  }
  if (!active) return;
  const double* Pj = diag ? sP : sQ;
  f64x4 acc[2][2] = {{zero, zero}, {zero, zero}};
  mma16_2x2(sP, 32 * wi, Pj, 32 * wj, CB, acc, lane);
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int gi = i0 + 32 * wi + 16 * x + (lane >> 4) + 4 * v;
        const int gj = j0 + 32 * wj + 16 * y + (lane & 15);
        if (gi < n && gj < n && gj <= gi) A[(int64_t)gi * n + gj] = cur[x][y][v] - acc[x][y][v];
      }
}

// The deferred trailing update of a panel of w block columns kb0 .. kb0 + 64 w - 1, all of whose
// factor blocks are in L: A_ij -= sum_c L_ic L_jc^T for every lower tile of the trailing matrix
// from base = kb0 + 64 w on, one tile per workgroup (each wave a 32 x 32 quarter), the sum over the
// w block columns accumulated on the fp64 matrix cores with the two factor blocks of each column
// staged in LDS (two buffers: two workgroups per CU).  Workgroup 0 takes the diagonal tile at base,
// applies the same update and factors it (L and the inverted 16 x 16 blocks to Xout), which starts
// the next panel.  Applying a panel's w columns together reads and writes the trailing matrix
// once per panel instead of once per block column.
__global__ __launch_bounds__(256) void chol_update_kernel(double* __restrict__ A, double* __restrict__ L,
                                                          double* __restrict__ Xout, int n, int kb0, int w,
                                                          int32_t* __restrict__ dev_info) {
  if (*dev_info != 0) return;
  __shared__ double sP[CB * CP];
  __shared__ double sQ[CB * CP];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int base = kb0 + CB * w;
  const f64x4 zero = {0.0, 0.0, 0.0, 0.0};
  int t, ti, tj;
  {
    // each XCD (workgroup b runs on XCD b % 8) takes a contiguous range of the tiles in blocked
    // order, so the workgroups it runs at once read the factor rows of few tile rows and columns
    const int nt = (n - base + CB - 1) / CB, tiles = nt * (nt + 1) / 2, bid = blockIdx.x;
    const int q = tiles / CU_XCD, rem = tiles % CU_XCD, x = bid % CU_XCD, slot = bid / CU_XCD;
    if (slot >= q + (x < rem ? 1 : 0)) return;  // the grid is rounded up to a multiple of 8
    t = x * q + min(x, rem) + slot;
    blocked_tile<4, 8>(t, nt, ti, tj);
  }
  const int i0 = base + CB * ti, j0 = base + CB * tj;
  const bool diag = ti == tj;
  const int wi = wave >> 1, wj = wave & 1;
  const bool active = !(diag && wj > wi);
  double cur[2][2][4];
  f64x4 acc[2][2];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y) {
      acc[x][y] = zero;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int gi = i0 + 32 * wi + 16 * x + (lane >> 4) + 4 * v;
        const int gj = j0 + 32 * wj + 16 * y + (lane & 15);
        cur[x][y][v] = active && gi < n && gj < n ? A[(int64_t)gi * n + gj] : 0.0;
      }
    }
  for (int c = 0; c < w; ++c) {
    load_block64(L, n, i0, kb0 + CB * c, n, n, sP, tid);
    if (!diag) load_block64(L, n, j0, kb0 + CB * c, n, n, sQ, tid);
    lds_sync();
    const double* Pj = diag ? sP : sQ;
    if (active) mma16_2x2(sP, 32 * wi, Pj, 32 * wj, CB, acc, lane);
    lds_sync();
  }
  if (t == 0) {
    // the next diagonal block: updated lower quarters into sP (the strictly upper 16 x 16 parts
    // of the diagonal quarters are never read by the factorisation), identity past n, factor
    if (active) {
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y)
#pragma unroll
          for (int v = 0; v < 4; ++v)
            sP[(32 * wi + 16 * x + (lane >> 4) + 4 * v) * CP + 32 * wj + 16 * y + (lane & 15)] =
                cur[x][y][v] - acc[x][y][v];
    }
    lds_sync();
    pad_diag(sP, n, base, tid);
    lds_sync();
    diag_factor(sP, sQ, n, base, L, Xout, dev_info, tid);
    return;
  }
  if (!active) return;
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int gi = i0 + 32 * wi + 16 * x + (lane >> 4) + 4 * v;
        const int gj = j0 + 32 * wj + 16 * y + (lane & 15);
        if (gi < n && gj < n && gj <= gi) A[(int64_t)gi * n + gj] = cur[x][y][v] - acc[x][y][v];
      }
}

// The same deferred update on 128 x 128 tiles for trailing matrices of many tiles: twice the
// multiply-adds per factor byte fetched, and 8 MFMAs per 6 fragment reads.  Eight waves (two per
// SIMD), each a 64 x 32 part of the tile (4 x 2 blocks of 16 x 16); one workgroup per CU (the two
// 128-row factor blocks of a column take 130 KB of LDS), the next column's blocks fetched into
// registers while the current one is multiplied, and the tile of A while the last one is; tiles in
// blocked order, a contiguous range per XCD.
// Workgroup 0 (tile (0, 0), dispatched first) also factors the next panel's first diagonal block,
// the top-left 64 x 64 block of its tile, as chol_update_kernel does: that block goes to LDS instead
// of A, and its factor and inverted 16 x 16 blocks to L and Xout.
constexpr int CB2 = 128;
constexpr int CU2_LDS = 2 * CB2 * CP * (int)sizeof(double);

__device__ __forceinline__ void fetch_block128(const double* __restrict__ G, int64_t ld, int r0, int c0, int nr, int nc,
                                               double2 (&v)[8], int tid) {
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int e = tid + 512 * q;  // pair index: row e / 32, columns 2 (e % 32) .. +1
    const int r = e >> 5, c = 2 * (e & 31);
    const bool ok = r0 + r < nr && c0 + c + 1 < nc;  // nc is even
    const int64_t off = ok ? (int64_t)(r0 + r) * ld + c0 + c : 0;
    v[q] = *reinterpret_cast<const double2*>(G + off);
    if (!ok) v[q] = double2{0.0, 0.0};
  }
}

__device__ __forceinline__ void put_block128(const double2 (&v)[8], double* sM, int tid) {
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int e = tid + 512 * q;
    const int r = e >> 5, c = 2 * (e & 31);
    sM[r * CP + c] = v[q].x;
    sM[r * CP + c + 1] = v[q].y;
  }
}

__global__ __launch_bounds__(512) void chol_update128_kernel(double* __restrict__ A, double* __restrict__ L,
                                                             double* __restrict__ Xout, int n, int kb0, int w,
                                                             int32_t* __restrict__ dev_info) {
  if (*dev_info != 0) return;
  extern __shared__ double cu2_lds[];
  double* sP = cu2_lds;
  double* sQ = cu2_lds + CB2 * CP;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int base = kb0 + CB * w;
  const f64x4 zero = {0.0, 0.0, 0.0, 0.0};
  int ti, tj;
  {
    const int nt2 = (n - base + CB2 - 1) / CB2, tiles = nt2 * (nt2 + 1) / 2, bid = blockIdx.x;
    const int q = tiles / CU_XCD, rem = tiles % CU_XCD, x = bid % CU_XCD, slot = bid / CU_XCD;
    if (slot >= q + (x < rem ? 1 : 0)) return;  // the grid is rounded up to a multiple of 8
    blocked_tile<4, 8>(x * q + min(x, rem) + slot, nt2, ti, tj);
  }
  const int i0 = base + CB2 * ti, j0 = base + CB2 * tj;
  const bool diag = ti == tj;
  const int wi = wave >> 2, wj = wave & 3;
  const bool active = !(diag && 32 * wj >= 64 * wi + 64);  // parts wholly above the diagonal: nothing
  const int li = lane & 15, lk = lane >> 4;
  f64x4 acc[4][2];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y) acc[x][y] = zero;
  double2 pv[8], qv[8];
  fetch_block128(L, n, i0, kb0, n, n, pv, tid);
  if (!diag) fetch_block128(L, n, j0, kb0, n, n, qv, tid);
  const double* Pj = diag ? sP : sQ;
  auto multiply = [&]() {
    if (!active) return;
#pragma unroll 2
    for (int k0 = 0; k0 < CB; k0 += 4) {
      double fa[4], fb[2];
#pragma unroll
      for (int x = 0; x < 4; ++x) fa[x] = sP[(64 * wi + 16 * x + li) * CP + k0 + lk];
#pragma unroll
      for (int y = 0; y < 2; ++y) fb[y] = Pj[(32 * wj + 16 * y + li) * CP + k0 + lk];
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y) acc[x][y] = __builtin_amdgcn_mfma_f64_16x16x4f64(fa[x], fb[y], acc[x][y], 0, 0, 0);
    }
  };
  for (int c = 0; c + 1 < w; ++c) {
    if (c > 0) lds_sync();  // every wave is done with column c - 1
    put_block128(pv, sP, tid);
    if (!diag) put_block128(qv, sQ, tid);
    lds_sync();
    fetch_block128(L, n, i0, kb0 + CB * (c + 1), n, n, pv, tid);
    if (!diag) fetch_block128(L, n, j0, kb0 + CB * (c + 1), n, n, qv, tid);
    multiply();
  }
  if (w > 1) lds_sync();
  put_block128(pv, sP, tid);
  if (!diag) put_block128(qv, sQ, tid);
  lds_sync();
  // the wave's part of A_ij, fetched while the last column is multiplied (in the registers the
  // factor blocks used)
  double cur[4][2][4];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int gi = i0 + 64 * wi + 16 * x + lk + 4 * v;
        const int gj = j0 + 32 * wj + 16 * y + li;
        cur[x][y][v] = active && gi < n && gj < n ? A[(int64_t)gi * n + gj] : 0.0;
      }
  multiply();
  const bool first = diag && ti == 0;  // tile (0, 0): its top-left 64 x 64 block is the next diagonal block
  if (!first && !active) return;
  if (active) {
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int y = 0; y < 2; ++y)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int gi = i0 + 64 * wi + 16 * x + lk + 4 * v;
          const int gj = j0 + 32 * wj + 16 * y + li;
          const double val = cur[x][y][v] - acc[x][y][v];
          const bool in_block = first && wi == 0 && wj < 2;
          if (!in_block && gi < n && gj < n && gj <= gi) A[(int64_t)gi * n + gj] = val;
          cur[x][y][v] = val;
        }
  }
  if (!first) return;
  // workgroup 0 only, every wave to the end (the barriers below count all eight): waves 0 and 1 hold
  // the block's lower part (strictly upper parts are never read by the factorisation); it goes to
  // LDS once every wave is done with the factor blocks there, then identity past n, then the factor
  double* sA = sP;
  double* sX = sP + CB * CP;
  lds_sync();
  if (wi == 0 && wj < 2) {
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int y = 0; y < 2; ++y)
#pragma unroll
        for (int v = 0; v < 4; ++v) sA[(16 * x + lk + 4 * v) * CP + 32 * wj + 16 * y + li] = cur[x][y][v];
  }
  lds_sync();
  pad_diag(sA, n, base, tid, 512);
  lds_sync();
  diag_factor(sA, sX, n, base, L, Xout, dev_info, tid, false, -1, 512);
}

// Block columns per panel of deferred trailing updates.
static const int kPanel = 4;
// Trailing matrices of at least this many 64-wide tile rows take the 128 x 128 tile update.
static const int kBigUpdate = 40;

// A = J H J (lower triangle), widened to fp64.
__global__ void reverse_copy_kernel(const float* __restrict__ H, int64_t ldh, int n, double* __restrict__ A) {
  const int i = blockIdx.x;
  for (int j = threadIdx.x; j <= i; j += blockDim.x)
    A[(int64_t)i * n + j] = (double)H[(int64_t)(n - 1 - i) * ldh + (n - 1 - j)];
}

// M[i][j] = L[n-1-i][n-1-j] / L[n-1-j][n-1-j] for i < j; 0 on and below the diagonal
// (the unit diagonal is implicit).
__global__ __launch_bounds__(256) void build_m_kernel(const double* __restrict__ L, int n, float* __restrict__ M,
                                                      const int32_t* __restrict__ dev_info) {
  // one 64 x 64 tile of M per workgroup; the 64 diagonal entries its columns divide by are read
  // once into LDS (they lie on 64 different rows of L)
  if (*dev_info != 0) return;
  __shared__ double dg[64];
  const int i0 = 64 * blockIdx.y, j0 = 64 * blockIdx.x;
  const int c = threadIdx.x & 63;
  if (threadIdx.x < 64) {
    const int64_t rj = n - 1 - (j0 + c);
    dg[c] = j0 + c < n ? L[rj * n + rj] : 1.0;
  }
  __syncthreads();
  for (int r = threadIdx.x >> 6; r < 64; r += 4) {
    const int i = i0 + r, j = j0 + c;
    if (i < n && j < n) {
      float v = 0.0f;
      if (j > i) v = (float)(L[(int64_t)(n - 1 - i) * n + (n - 1 - j)] / dg[c]);
      M[(int64_t)i * n + j] = v;
    }
  }
}

}  // namespace wr

using namespace wr;

size_t wr_factor_ws_bytes(int64_t n) {
  return 2 * (size_t)n * n * sizeof(double) + 2 * 4 * 256 * sizeof(double);
}

// M (n x n fp32, row-major) from the damped H.  ws: wr_factor_ws_bytes(n) bytes.
int wr_factor_m(hipStream_t st, const float* H, int64_t ldh, int n, void* ws, float* M, int32_t* dev_info) {
  double* A = static_cast<double*>(ws);
  double* Lf = A + (size_t)n * n;
  double* Xinv[2] = {Lf + (size_t)n * n, Lf + (size_t)n * n + 4 * 256};  // alternate per block column
  hipLaunchKernelGGL(reverse_copy_kernel, dim3(n), dim3(256), 0, st, H, ldh, n, A);
  WR_CHECK_LAUNCH();
  hipLaunchKernelGGL(chol_diag_kernel, dim3(1), dim3(256), 0, st, A, n, 0, Lf, Xinv[0], dev_info);
  WR_CHECK_LAUNCH();
  // Panels of kPanel block columns: within a panel each block column updates only the panel's own
  // later block columns (every tile of its first trailing column also writes the factor blocks
  // L_ik); after the panel's last block column, its factor blocks below the panel are solved in one
  // launch and the whole trailing matrix takes the panel's update at once.
  const int nblk = (n + CB - 1) / CB;
  for (int k = 0; k + 1 < nblk; ++k) {
    const int kb = CB * k;
    const int s0 = k - k % kPanel, s1 = std::min(s0 + kPanel, nblk);
    const int nt = nblk - k - 1;
    const int w_rem = s1 - (k + 1);
    double* Xin = Xinv[k & 1];
    double* Xout = Xinv[(k + 1) & 1];
    if (w_rem >= 1) {
      const int wc = std::min(w_rem, nt);
      const int tiles = wc * (wc + 1) / 2 + (nt - wc) * wc;
      hipLaunchKernelGGL(chol_step_kernel, dim3(tiles), dim3(256), 0, st, A, Lf, Xin, Xout, n, kb, 0, wc, dev_info);
      WR_CHECK_LAUNCH();
    } else {
      hipLaunchKernelGGL(chol_panel_kernel, dim3(nt), dim3(256), 0, st, A, Lf, Xin, n, kb, dev_info);
      WR_CHECK_LAUNCH();
      if (nt >= kBigUpdate) {
        // 128 x 128 tiles; workgroup 0 factors the next panel's first diagonal block
        const int nt2 = (nt + 1) / 2, tiles = nt2 * (nt2 + 1) / 2;
        if (!lds_limit(reinterpret_cast<const void*>(chol_update128_kernel), CU2_LDS)) return WR_EHIP;
        hipLaunchKernelGGL(chol_update128_kernel, dim3((tiles + CU_XCD - 1) / CU_XCD * CU_XCD), dim3(512), CU2_LDS, st,
                           A, Lf, Xout, n, CB * s0, s1 - s0, dev_info);
      } else {
        const int tiles = nt * (nt + 1) / 2;
        hipLaunchKernelGGL(chol_update_kernel, dim3((tiles + CU_XCD - 1) / CU_XCD * CU_XCD), dim3(256), 0, st, A, Lf,
                           Xout, n, CB * s0, s1 - s0, dev_info);
      }
      WR_CHECK_LAUNCH();
    }
  }
  hipLaunchKernelGGL(build_m_kernel, dim3((unsigned)((n + 63) / 64), (unsigned)((n + 63) / 64)), dim3(256), 0, st, Lf, n,
                     M, dev_info);
  WR_CHECK_LAUNCH();
  return WR_OK;
}
