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
// factored and its factor inverted by one workgroup: two 32 x 32 halves, each
// factored and inverted by one wave in registers (rows in lanes, pivot columns
// broadcast with readlane), glued by fp64 MFMA products in LDS.  Per block
// column kb two kernels:
//   chol_panel_kernel  the block column below, P = A_panel L_kk^-T = A_panel X^T,
//                      on the fp64 matrix cores (the factor's final block
//                      column, written to L);
//   chol_step_kernel   the trailing lower matrix, A_ij -= P_i P_j^T, one 64 x 64
//                      tile per workgroup on the fp64 matrix cores, while
//                      workgroup 0 updates, factors and inverts the next
//                      diagonal block (lookahead).
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

// 1/sqrt(d) to fp64 precision: fp32 estimate, two Newton steps.
__device__ __forceinline__ double rsqrt_newton(double d) {
  double r = (double)rsqrtf((float)d);
  r = r * (1.5 - 0.5 * d * r * r);
  r = r * (1.5 - 0.5 * d * r * r);
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

// acc += sum_{k < K} A(r, k) B(k, c) for one 16 x 16 block (v_mfma_f64_16x16x4f64).
// A(r, k) = SA[(r0 + r) * lda + k].  B(k, c) = SB[(c0 + c) * ldb + k] when BT (the
// "A B^T" form), else SB[k * ldb + c0 + c].  Operand lane l supplies row/column
// l % 16 at k = l / 16; accumulator v of lane l is row l / 16 + 4 v, column l % 16.
template <bool BT>
__device__ __forceinline__ f64x4 mma16(const double* SA, int lda, int r0, const double* SB, int ldb, int c0, int K,
                                       f64x4 acc, int lane) {
  const int li = lane & 15, lk = lane >> 4;
#pragma unroll 4
  for (int k0 = 0; k0 < K; k0 += 4) {
    const double a = SA[(r0 + li) * lda + k0 + lk];
    const double b = BT ? SB[(c0 + li) * ldb + k0 + lk] : SB[(k0 + lk) * ldb + c0 + li];
    acc = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, acc, 0, 0, 0);
  }
  return acc;
}

// Cholesky of the 32 x 32 block of sM at (o, o) in place (lower part; the strict
// upper part is cleared).  One wave: lane i < 32 holds row i in registers; the
// column of pivot k is broadcast lane by lane; rinv[o + k] receives 1 / L_kk.
// Returns the first pivot (0-based) that is not positive, or -1.  Wave-uniform.
__device__ __forceinline__ int chol32_wave(double* sM, double* rinv, int o, int lane) {
  const int r = lane & 31;
  double a[32];
#pragma unroll
  for (int j = 0; j < 32; ++j) a[j] = sM[(o + r) * CP + o + j];
  int bad = -1;
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    const double d = bcast_f64(a[k], k);
    if (!(d > 0.0) && bad < 0) bad = k;
    const double rs = rsqrt_newton(d);
    const double l = a[k] * rs;  // lane k: sqrt(d); lanes below: L_ik
    a[k] = l;
    if (lane == 0) rinv[o + k] = rs;
#pragma unroll
    for (int j = k + 1; j < 32; ++j) a[j] = fma(-l, bcast_f64(l, j), a[j]);
  }
  if (lane < 32) {
#pragma unroll
    for (int j = 0; j < 32; ++j) sM[(o + r) * CP + o + j] = j <= r ? a[j] : 0.0;
  }
  return bad;
}

// X = L^-1 for the lower 32 x 32 block L of sM at (o, o), into sX at (o, o)
// (zeros above the diagonal); rinv[i] = 1 / L_ii.  One wave: lane c < 32 solves
// L x = e_c by forward substitution (two interleaved partial sums shorten the
// dependency chain); the entries of L are read as LDS broadcasts.
__device__ __forceinline__ void inv32_wave(const double* sM, const double* rinv, double* sX, int o, int lane) {
  const int c = lane & 31;
  double x[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    double s0 = i == c ? 1.0 : 0.0, s1 = 0.0;
#pragma unroll
    for (int m = 0; m + 1 < i; m += 2) {
      s0 = fma(-sM[(o + i) * CP + o + m], x[m], s0);
      s1 = fma(-sM[(o + i) * CP + o + m + 1], x[m + 1], s1);
    }
    if (i & 1) s0 = fma(-sM[(o + i) * CP + o + i - 1], x[i - 1], s0);
    x[i] = (s0 + s1) * rinv[o + i];
  }
  if (lane < 32) {
#pragma unroll
    for (int i = 0; i < 32; ++i) sX[(o + i) * CP + o + c] = x[i];
  }
}

// Factor and invert the 64 x 64 diagonal block at kb held in sA (lower part valid,
// strict upper part zero, identity past n): L_kk goes to L and X = L_kk^-1 (64 x 64,
// zeros above the diagonal) to Xinv.  Two 32 x 32 halves: L00 = chol(A00),
// X00 = L00^-1, L10 = A10 X00^T, A11 -= L10 L10^T, L11 = chol(A11), X11 = L11^-1,
// X10 = -X11 (L10 X00).  sX needs no initial contents; the product L10 X00 is kept
// in the unused upper right quarter of sA.  A pivot that is not positive sets
// dev_info (first failure wins).
__device__ __forceinline__ void diag_factor(double* sA, double* sX, double* rinv, int n, int kb, double* L,
                                            double* Xinv, int32_t* dev_info, int tid) {
  const int lane = tid & 63, wave = tid >> 6;
  int bad = -1;
  if (wave == 0) {
    bad = chol32_wave(sA, rinv, 0, lane);
    inv32_wave(sA, rinv, sX, 0, lane);
  }
  __syncthreads();
  // L10 = A10 X00^T
  const int bi = wave >> 1, bj = wave & 1;
  const f64x4 zero = {0.0, 0.0, 0.0, 0.0};
  f64x4 acc = mma16<true>(sA, CP, 32 + 16 * bi, sX, CP, 16 * bj, 32, zero, lane);
  __syncthreads();
#pragma unroll
  for (int v = 0; v < 4; ++v) sA[(32 + 16 * bi + (lane >> 4) + 4 * v) * CP + 16 * bj + (lane & 15)] = acc[v];
  __syncthreads();
  // A11 -= L10 L10^T (reads columns 0..31, writes columns 32..63)
  acc = mma16<true>(sA, CP, 32 + 16 * bi, sA, CP, 32 + 16 * bj, 32, zero, lane);
#pragma unroll
  for (int v = 0; v < 4; ++v) sA[(32 + 16 * bi + (lane >> 4) + 4 * v) * CP + 32 + 16 * bj + (lane & 15)] -= acc[v];
  __syncthreads();
  // wave 0: L11 = chol(A11), X11 = L11^-1; waves 1-3 meanwhile: T = L10 X00 into sA[0..31][32..63]
  if (wave == 0) {
    const int b2 = chol32_wave(sA, rinv, 32, lane);
    if (bad < 0 && b2 >= 0) bad = 32 + b2;
    inv32_wave(sA, rinv, sX, 32, lane);
  } else {
    for (int blk = wave - 1; blk < 4; blk += 3) {
      const int ti = blk >> 1, tj = blk & 1;
      const f64x4 t = mma16<false>(sA, CP, 32 + 16 * ti, sX, CP, 16 * tj, 32, zero, lane);
#pragma unroll
      for (int v = 0; v < 4; ++v) sA[(16 * ti + (lane >> 4) + 4 * v) * CP + 32 + 16 * tj + (lane & 15)] = t[v];
    }
  }
  __syncthreads();
  // X10 = -X11 T
  acc = mma16<false>(sX + 32 * CP + 32, CP, 16 * bi, sA + 32, CP, 16 * bj, 32, zero, lane);
#pragma unroll
  for (int v = 0; v < 4; ++v) sX[(32 + 16 * bi + (lane >> 4) + 4 * v) * CP + 16 * bj + (lane & 15)] = -acc[v];
  if (wave == 0 && lane == 0 && bad >= 0) atomicCAS(dev_info, 0, kb + bad + 1);
  __syncthreads();
  for (int e = tid; e < CB * CB; e += 256) {
    const int r = e / CB, c = e % CB;
    Xinv[e] = c <= r ? sX[r * CP + c] : 0.0;
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
  __shared__ double rinv[CB];
  const int tid = threadIdx.x;
  load_block64(A, n, 0, 0, n, n, sA, tid);
  __syncthreads();
  prepare_diag(sA, n, 0, tid);
  __syncthreads();
  diag_factor(sA, sX, rinv, n, 0, L, Xinv, dev_info, tid);
}

// P = A[rows, kb..kb+63] X^T for the 64 rows below the diagonal block at `row0`:
// the factor's block column (written to L).
__global__ __launch_bounds__(256) void chol_panel_kernel(const double* __restrict__ A, int n, int kb,
                                                         const double* __restrict__ Xinv, double* __restrict__ L,
                                                         const int32_t* __restrict__ dev_info) {
  if (*dev_info != 0) return;
  __shared__ double sX[CB * CP];
  __shared__ double sP[CB * CP];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row0 = kb + CB + CB * blockIdx.x;
  load_block64(Xinv, CB, 0, 0, CB, CB, sX, tid);
  load_block64(A, n, row0, kb, n, n, sP, tid);
  __syncthreads();
  f64x4 acc[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
    acc[cb] = mma16<true>(sP, CP, 16 * wave, sX, CP, 16 * cb, CB, f64x4{0.0, 0.0, 0.0, 0.0}, lane);
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int r = row0 + 16 * wave + (lane >> 4) + 4 * v, c = kb + 16 * cb + (lane & 15);
      if (r < n && c < n) L[(int64_t)r * n + c] = acc[cb][v];
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
  __shared__ double rinv[CB];
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
    diag_factor(sA, sP, rinv, n, base, L, Xinv, dev_info, tid);
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
