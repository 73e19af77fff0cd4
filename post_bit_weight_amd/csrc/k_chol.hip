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
// with readlane), the rest are fp64 MFMA products in LDS.  Per block column kb
// two kernels:
//   chol_panel_kernel  the block column below, P = A_panel L_kk^-T, as a blocked
//                      triangular solve with the inverted 16 x 16 diagonal
//                      blocks on the fp64 matrix cores (the factor's final
//                      block column, written to L);
//   chol_step_kernel   the trailing lower matrix, A_ij -= P_i P_j^T, one 64 x 64
//                      tile per workgroup on the fp64 matrix cores, while
//                      workgroup 0 updates and factors the next diagonal block
//                      (lookahead).
// A pivot that is not positive sets dev_info (1-based pivot of J H J) and every
// later kernel returns at once.
#include "common.hpp"

namespace wr {

constexpr int CB = 64;        // block edge
constexpr int CP = CB + 1;    // LDS row pitch in doubles: rows start on different banks

typedef double f64x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ double bcast_f64(double v, int lane) {
  const int64_t u = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane((int)(u & 0xffffffff), lane);
  const int hi = __builtin_amdgcn_readlane((int)(u >> 32), lane);
  return __longlong_as_double(((int64_t)hi << 32) | (uint32_t)lo);
}

// 1/sqrt(d) to fp64 precision: the hardware estimate (about 23 correct bits over the
// whole fp64 range), two Newton steps r <- r (3 - d r^2) / 2.
__device__ __forceinline__ double rsqrt_f64(double d) {
  const double h = 0.5 * d;
  double r = __builtin_amdgcn_rsq(d);
  r = r * fma(-h * r, r, 1.5);
  r = r * fma(-h * r, r, 1.5);
  return r;
}

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

// acc += sum_{k < K} A(r, k) B(k, c) for one 16 x 16 block (v_mfma_f64_16x16x4f64);
// acc -= ... when NEG.  A(r, k) = SA[(r0 + r) * lda + k].  B(k, c) = SB[(c0 + c) * ldb + k]
// when BT (the "A B^T" form), else SB[k * ldb + c0 + c].  Operand lane l supplies
// row/column l % 16 at k = l / 16; accumulator v of lane l is row l / 16 + 4 v, column l % 16.
template <bool BT, bool NEG = false>
__device__ __forceinline__ f64x4 mma16(const double* SA, int lda, int r0, const double* SB, int ldb, int c0, int K,
                                       f64x4 acc, int lane) {
  const int li = lane & 15, lk = lane >> 4;
#pragma unroll 4
  for (int k0 = 0; k0 < K; k0 += 4) {
    const double a = SA[(r0 + li) * lda + k0 + lk];
    const double b = BT ? SB[(c0 + li) * ldb + k0 + lk] : SB[(k0 + lk) * ldb + c0 + li];
    acc = __builtin_amdgcn_mfma_f64_16x16x4f64(NEG ? -a : a, b, acc, 0, 0, 0);
  }
  return acc;
}

// Cholesky of the 16 x 16 block of sM at (o, o) together with the inverse of its
// factor, by one wave.  Lanes 0-15 hold the rows of the block (row r = lane & 15),
// lanes 16-31 the columns of the identity; lanes 32-63 repeat lanes 0-31.  At pivot k
// every lane forms m = v[k] / L_kk and subtracts m times column k of L (broadcast
// from lanes k+1..15) from its later entries: for a row of A this is the
// right-looking Cholesky update, for a column e_c it is the column-oriented forward
// substitution of L x = e_c, so lanes 16-31 end with the columns of X = L^-1.  The
// next pivot is formed from values read before the update (the same arithmetic as
// the update itself), so its reciprocal square root overlaps the update.
// L goes back to sM (zeros above the diagonal), X to sX at (o, o) (zeros above).
// Returns the first pivot (0-based) that is not positive, or -1.  Wave-uniform.
__device__ __forceinline__ int chol16_inv_wave(double* sM, double* sX, int o, int lane) {
  const int r = lane & 15;
  const bool xcol = (lane & 16) != 0;
  double v[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) v[j] = xcol ? (j == r ? 1.0 : 0.0) : sM[(o + r) * CP + o + j];
  int bad = -1;
  double d = bcast_f64(v[0], 0);
  if (!(d > 0.0)) bad = 0;
  double rs = rsqrt_f64(d);
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    // All of this pivot's broadcasts are issued before its updates (a readlane result
    // is ready only ~16 ns after issue); at most 34 scalar registers are live.
    double an = 0.0, bn = 0.0;
    if (k + 1 < 16) {
      an = bcast_f64(v[k + 1], k + 1);  // next diagonal entry before this update
      bn = bcast_f64(v[k], k + 1);      // its entry in column k
    }
    const double m = v[k] * rs;  // rows: L_rk (L_kk on lane k); columns: x_k
    v[k] = m;
    double col[16];
#pragma unroll
    for (int j = k + 1; j < 16; ++j) col[j] = bcast_f64(m, j);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = k + 1; j < 16; ++j) v[j] = fma(-m, col[j], v[j]);
    if (k + 1 < 16) {
      const double t = bn * rs;
      d = fma(-t, t, an);  // equals the updated v[k + 1] of lane k + 1
      if (!(d > 0.0) && bad < 0) bad = k + 1;
      rs = rsqrt_f64(d);
    }
  }
  if (lane < 16) {
#pragma unroll
    for (int j = 0; j < 16; ++j) sM[(o + r) * CP + o + j] = j <= r ? v[j] : 0.0;
  } else if (lane < 32) {
#pragma unroll
    for (int i = 0; i < 16; ++i) sX[(o + i) * CP + o + r] = i >= r ? v[i] : 0.0;
  }
  return bad;
}

// Factor the 64 x 64 diagonal block at kb held in sA (lower part valid, strict upper
// part zero, identity past n) as L_kk, by 16 x 16 blocks: per block column s, wave 0
// factors the diagonal block and inverts its factor (X_ss), the blocks below become
// L_is = A_is X_ss^T, and the trailing blocks take A_ij -= L_is L_js^T on the fp64
// matrix cores.  Wave 0 updates and factors the next diagonal block while waves 1-3
// update the rest.  L_kk goes to L; the four X_ss to Xinv (64 x 64, zero outside the
// diagonal 16 x 16 blocks).  sX needs no initial contents.  A pivot that is not
// positive sets dev_info (first failure wins).
__device__ __forceinline__ void diag_factor(double* sA, double* sX, int n, int kb, double* L, double* Xinv,
                                            int32_t* dev_info, int tid) {
  const int lane = tid & 63, wave = tid >> 6;
  const f64x4 zero = {0.0, 0.0, 0.0, 0.0};
  int bad = -1;
  if (wave == 0) bad = chol16_inv_wave(sA, sX, 0, lane);
  __syncthreads();
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int o = 16 * s;
    if (wave < 3 - s) {  // L_is = A_is X_ss^T
      const int i0 = 16 * (s + 1 + wave);
      const f64x4 acc = mma16<true>(sA + o, CP, i0, sX + o, CP, o, 16, zero, lane);
#pragma unroll
      for (int v = 0; v < 4; ++v) sA[(i0 + (lane >> 4) + 4 * v) * CP + o + (lane & 15)] = acc[v];
    }
    __syncthreads();
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
    __syncthreads();
  }
  if (wave == 0 && lane == 0 && bad >= 0) atomicCAS(dev_info, 0, kb + bad + 1);
  for (int e = tid; e < CB * CB; e += 256) {
    const int r = e / CB, c = e % CB;
    Xinv[e] = (r >> 4) == (c >> 4) && c <= r ? sX[r * CP + c] : 0.0;
    if (c <= r && kb + r < n) L[(int64_t)(kb + r) * n + kb + c] = sA[r * CP + c];
  }
}

// Only the lower part of A is maintained: clear the strict upper part of the block in
// sA and pad rows past n with the identity.
__device__ __forceinline__ void prepare_diag(double* sA, int n, int kb, int tid) {
  for (int e = tid; e < CB * CB; e += 256) {
    const int r = e / CB, c = e % CB;
    if (c > r) sA[r * CP + c] = 0.0;
    else if (kb + r >= n) sA[r * CP + c] = r == c ? 1.0 : 0.0;
  }
}

// First diagonal block (kb = 0).
__global__ __launch_bounds__(256) void chol_diag_kernel(const double* __restrict__ A, int n, double* __restrict__ L,
                                                        double* __restrict__ Xinv, int32_t* __restrict__ dev_info) {
  if (*dev_info != 0) return;
  __shared__ double sA[CB * CP];
  __shared__ double sX[CB * CP];
  const int tid = threadIdx.x;
  load_block64(A, n, 0, 0, n, n, sA, tid);
  __syncthreads();
  prepare_diag(sA, n, 0, tid);
  __syncthreads();
  diag_factor(sA, sX, n, 0, L, Xinv, dev_info, tid);
}

// The factor's block column below the diagonal block at kb: P L_kk^T = A_panel for the
// 64 rows from row0, by 16-column blocks, P_s = (A_s - sum_{t<s} P_t L_st^T) X_ss^T with
// X_ss the inverted diagonal 16 x 16 blocks of L_kk (written to L).  Wave w owns rows
// 16 w .. 16 w + 15 of the panel and needs no other wave's results.
__global__ __launch_bounds__(256) void chol_panel_kernel(const double* __restrict__ A, int n, int kb,
                                                         const double* __restrict__ Xinv, double* __restrict__ L,
                                                         const int32_t* __restrict__ dev_info) {
  if (*dev_info != 0) return;
  __shared__ double sX[CB * CP];
  __shared__ double sL[CB * CP];
  __shared__ double sP[CB * CP];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row0 = kb + CB + CB * blockIdx.x;
  load_block64(Xinv, CB, 0, 0, CB, CB, sX, tid);
  load_block64(L, n, kb, kb, n, n, sL, tid);
  load_block64(A, n, row0, kb, n, n, sP, tid);
  __syncthreads();
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
    for (int v = 0; v < 4; ++v) {
      const int rl = w0 + (lane >> 4) + 4 * v;
      sP[rl * CP + o + (lane & 15)] = acc[v];
      if (row0 + rl < n) L[(int64_t)(row0 + rl) * n + kb + o + (lane & 15)] = acc[v];
    }
  }
}

// Step kb, after chol_panel_kernel has written the block column P = L[kb + 64.., kb..]:
// workgroup 0 updates the next diagonal block, A_00 - P_0 P_0^T (not stored back), and
// factors and inverts it (lookahead: the serial part of the next step overlaps this
// step's trailing update); every other workgroup owns one lower tile (ti, tj) != (0, 0)
// of the trailing matrix (rows/columns from kb + 64 on) and applies A_ij -= P_i P_j^T.
__global__ __launch_bounds__(256) void chol_step_kernel(double* __restrict__ A, double* __restrict__ L,
                                                        double* __restrict__ Xinv, int n, int kb,
                                                        int32_t* __restrict__ dev_info) {
  if (*dev_info != 0) return;
  __shared__ double sPi[CB * CP];
  __shared__ double sPj[CB * CP];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int base = kb + CB;
  const f64x4 zero = {0.0, 0.0, 0.0, 0.0};
  if (blockIdx.x == 0) {
    double* sA = sPi;  // the next diagonal block
    double* sP = sPj;  // its panel rows, later X
    load_block64(A, n, base, base, n, n, sA, tid);
    load_block64(L, n, base, kb, n, n, sP, tid);
    __syncthreads();
    const int wi = wave >> 1, wj = wave & 1;
    f64x4 acc[2][2];
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int y = 0; y < 2; ++y)
        acc[x][y] = wj > wi ? zero : mma16<true>(sP, CP, 32 * wi + 16 * x, sP, CP, 32 * wj + 16 * y, CB, zero, lane);
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int y = 0; y < 2; ++y)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          sA[(32 * wi + 16 * x + (lane >> 4) + 4 * v) * CP + 32 * wj + 16 * y + (lane & 15)] -= acc[x][y][v];
    __syncthreads();
    prepare_diag(sA, n, base, tid);
    __syncthreads();
    diag_factor(sA, sP, n, base, L, Xinv, dev_info, tid);
    return;
  }
  int ti, tj;
  {
    const int t = blockIdx.x;  // lower tiles in row-major order; tile 0 is the diagonal block above
    int i = (int)((sqrtf(8.0f * (float)t + 1.0f) - 1.0f) * 0.5f);
    while (i * (i + 1) / 2 > t) --i;
    while ((i + 1) * (i + 2) / 2 <= t) ++i;
    ti = i;
    tj = t - i * (i + 1) / 2;
  }
  const int i0 = base + CB * ti, j0 = base + CB * tj;
  const bool diag = ti == tj;
  const int wi = wave >> 1, wj = wave & 1;
  const bool active = !(diag && wj > wi);  // strictly upper 32 x 32 quarter of a diagonal tile: nothing to do
  // the wave's 32 x 32 part of A_ij, fetched before the panels so its latency overlaps the MFMAs
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
  load_block64(L, n, i0, kb, n, n, sPi, tid);
  if (!diag) load_block64(L, n, j0, kb, n, n, sPj, tid);
  __syncthreads();
  if (!active) return;
  const double* Pj = diag ? sPi : sPj;
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y) {
      const f64x4 acc = mma16<true>(sPi, CP, 32 * wi + 16 * x, Pj, CP, 32 * wj + 16 * y, CB,
                                    f64x4{0.0, 0.0, 0.0, 0.0}, lane);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int gi = i0 + 32 * wi + 16 * x + (lane >> 4) + 4 * v;
        const int gj = j0 + 32 * wj + 16 * y + (lane & 15);
        if (gi < n && gj < n && gj <= gi) A[(int64_t)gi * n + gj] = cur[x][y][v] - acc[v];
      }
    }
}

// A = J H J (lower triangle), widened to fp64.
__global__ void reverse_copy_kernel(const float* __restrict__ H, int64_t ldh, int n, double* __restrict__ A) {
  const int i = blockIdx.x;
  for (int j = threadIdx.x; j <= i; j += blockDim.x)
    A[(int64_t)i * n + j] = (double)H[(int64_t)(n - 1 - i) * ldh + (n - 1 - j)];
}

// M[i][j] = L[n-1-i][n-1-j] / L[n-1-j][n-1-j] for i < j; 0 on and below the diagonal
// (the unit diagonal is implicit).
__global__ void build_m_kernel(const double* __restrict__ L, int n, float* __restrict__ M,
                               const int32_t* __restrict__ dev_info) {
  if (*dev_info != 0) return;
  const int i = blockIdx.x;
  const int64_t ri = n - 1 - i;
  for (int j = threadIdx.x; j < n; j += blockDim.x) {
    float v = 0.0f;
    if (j > i) {
      const int64_t rj = n - 1 - j;
      v = (float)(L[ri * n + rj] / L[rj * n + rj]);
    }
    M[(int64_t)i * n + j] = v;
  }
}

}  // namespace wr

using namespace wr;

size_t wr_factor_ws_bytes(int64_t n) { return 2 * (size_t)n * n * sizeof(double) + (size_t)CB * CB * sizeof(double); }

// M (n x n fp32, row-major) from the damped H.  ws: wr_factor_ws_bytes(n) bytes.
int wr_factor_m(hipStream_t st, const float* H, int64_t ldh, int n, void* ws, float* M, int32_t* dev_info) {
  double* A = static_cast<double*>(ws);
  double* Lf = A + (size_t)n * n;
  double* Xinv = Lf + (size_t)n * n;
  hipLaunchKernelGGL(reverse_copy_kernel, dim3(n), dim3(256), 0, st, H, ldh, n, A);
  WR_CHECK_LAUNCH();
  hipLaunchKernelGGL(chol_diag_kernel, dim3(1), dim3(256), 0, st, A, n, Lf, Xinv, dev_info);
  WR_CHECK_LAUNCH();
  for (int kb = 0; kb + CB < n; kb += CB) {
    const int nt = (n - kb - CB + CB - 1) / CB;
    hipLaunchKernelGGL(chol_panel_kernel, dim3(nt), dim3(256), 0, st, A, n, kb, Xinv, Lf, dev_info);
    WR_CHECK_LAUNCH();
    hipLaunchKernelGGL(chol_step_kernel, dim3(nt * (nt + 1) / 2), dim3(256), 0, st, A, Lf, Xinv, n, kb, dev_info);
    WR_CHECK_LAUNCH();
  }
  hipLaunchKernelGGL(build_m_kernel, dim3(n), dim3(256), 0, st, Lf, n, M, dev_info);
  WR_CHECK_LAUNCH();
  return WR_OK;
}
