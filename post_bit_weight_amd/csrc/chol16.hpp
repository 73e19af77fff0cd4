// fp64 helpers shared by the factorisation of H and the per-row scale solves: broadcasts, the
// reciprocal square root, the 16 x 16 fp64 matrix-core product and the Cholesky factor plus
// inverse of a 16 x 16 block by one wave.
#pragma once
#include "common.hpp"

namespace wr {

typedef double f64x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ double bcast_f64(double v, int lane) {
  const int64_t u = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane((int)(u & 0xffffffff), lane);
  const int hi = __builtin_amdgcn_readlane((int)(u >> 32), lane);
  return __longlong_as_double(((int64_t)hi << 32) | (uint32_t)lo);
}

// Workgroup barrier for data exchanged through LDS only: each wave waits for its own LDS
// operations, not for its global stores (which no other wave of the kernel reads).
__device__ __forceinline__ void lds_sync_f64() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// 1/sqrt(d) to fp64 precision: the hardware estimate (about 23 correct bits over the
// whole fp64 range), two Newton steps r <- r (3 - d r^2) / 2.
__device__ __forceinline__ double rsqrt_f64(double d) {
  const double h = 0.5 * d;
  double r = __builtin_amdgcn_rsq(d);
  r = r * fma(-h * r, r, 1.5);
  r = r * fma(-h * r, r, 1.5);
  return r;
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

// Cholesky of the 16 x 16 block at sM (row pitch P doubles) together with the inverse of its
// factor, by one wave.  Lanes 0-15 hold the rows of the block (row r = lane & 15),
// lanes 16-31 the columns of the identity; lanes 32-63 repeat lanes 0-31.  At pivot k
// every lane forms m = v[k] / L_kk and subtracts m times column k of L (broadcast
// from lanes k+1..15) from its later entries: for a row of A this is the
// right-looking Cholesky update, for a column e_c it is the column-oriented forward
// substitution of L x = e_c, so lanes 16-31 end with the columns of X = L^-1.  The
// next pivot is formed from values read before the update (the same arithmetic as
// the update itself), so its reciprocal square root overlaps the update.
// L goes back to sM (zeros above the diagonal), X to sX (same pitch, zeros above).
// Returns the first pivot (0-based) that is not positive, or -1.  Wave-uniform.
template <int P>
__device__ __forceinline__ int chol16_inv_pitch(double* sM, double* sX, int lane) {
  const int r = lane & 15;
  const bool xcol = (lane & 16) != 0;
  double v[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) v[j] = xcol ? (j == r ? 1.0 : 0.0) : sM[r * P + j];
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
    for (int j = 0; j < 16; ++j) sM[r * P + j] = j <= r ? v[j] : 0.0;
  } else if (lane < 32) {
#pragma unroll
    for (int i = 0; i < 16; ++i) sX[i * P + r] = i >= r ? v[i] : 0.0;
  }
  return bad;
}

}  // namespace wr
