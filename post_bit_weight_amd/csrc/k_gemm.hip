// fp32 GEMM tile kernel on the fp32 matrix cores (v_mfma_f32_32x32x2f32).
//
//   C[tile] = (accumulate ? C : 0) + alpha * A * op(B)
//
// A is M x K row-major (lda), op(B) is K x N: either B stored K x N (B_KN) or
// B stored N x K (transposed use).  64x64 output tile per workgroup of four
// waves, each wave owning one 32x32 MFMA block; K staged 16 at a time in LDS.
// With lower_tiles the grid enumerates only tiles on or below the diagonal.
// Used for the blocked Cholesky (triangular solve and trailing update) and the
// lazy-batch trailing update of the GPTQ sweep.  Leading dimensions, K and N
// must be multiples of 4 and the pointers 16-byte aligned.
#include "common.hpp"

namespace wr {

constexpr int GM_T = 64;
constexpr int GM_K = 16;

__device__ __forceinline__ void gm_tile_from_linear(int t, int& ti, int& tj) {
  int i = (int)((sqrtf(8.0f * (float)t + 1.0f) - 1.0f) * 0.5f);
  while (i * (i + 1) / 2 > t) --i;
  while ((i + 1) * (i + 2) / 2 <= t) ++i;
  ti = i;
  tj = t - i * (i + 1) / 2;
}

template <bool B_KN>
__global__ __launch_bounds__(256) void gemm_f32_kernel(int M, int N, int K, const float* __restrict__ A, int64_t lda,
                                                       const float* __restrict__ B, int64_t ldb, float* C, int64_t ldc,
                                                       float alpha, int accumulate, int lower_tiles,
                                                       const int32_t* __restrict__ dev_info) {
  if (dev_info && *dev_info != 0) return;
  __shared__ float sA[GM_K][GM_T + 4];
  __shared__ float sB[GM_K][GM_T + 4];
  int tm, tn;
  if (lower_tiles) {
    gm_tile_from_linear(blockIdx.x, tm, tn);
  } else {
    tm = blockIdx.y;
    tn = blockIdx.x;
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wi = wave >> 1, wj = wave & 1;
  const int64_t i0 = (int64_t)tm * GM_T, j0 = (int64_t)tn * GM_T;
  f32x16 acc = {};
  const int arow = tid >> 2, akq = (tid & 3) * 4;     // A loader: 64 rows x 16 k
  const int bk = tid >> 4, bjq = (tid & 15) * 4;      // B (K x N) loader: 16 k x 64 j
  for (int k0 = 0; k0 < K; k0 += GM_K) {
    {
      const int64_t i = i0 + arow;
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
      if (i < M && k0 + akq < K) v = *reinterpret_cast<const f32x4*>(A + i * lda + k0 + akq);
#pragma unroll
      for (int e = 0; e < 4; ++e) sA[akq + e][arow] = v[e];
    }
    if (B_KN) {
      const int64_t j = j0 + bjq;
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
      if (k0 + bk < K && j < N) v = *reinterpret_cast<const f32x4*>(B + (int64_t)(k0 + bk) * ldb + j);
      *reinterpret_cast<f32x4*>(&sB[bk][bjq]) = v;
    } else {
      const int64_t j = j0 + arow;
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
      if (j < N && k0 + akq < K) v = *reinterpret_cast<const f32x4*>(B + j * ldb + k0 + akq);
#pragma unroll
      for (int e = 0; e < 4; ++e) sB[akq + e][arow] = v[e];
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < GM_K; kk += 2) {
      const float a = sA[kk + (lane >> 5)][32 * wi + (lane & 31)];
      const float b = sB[kk + (lane >> 5)][32 * wj + (lane & 31)];
      acc = mfma32x32x2_f32(a, b, acc);
    }
    __syncthreads();
  }
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int64_t i = i0 + 32 * wi + acc_row(v, lane);
    const int64_t j = j0 + 32 * wj + (lane & 31);
    if (i < M && j < N) {
      float* p = C + i * ldc + j;
      *p = (accumulate ? *p : 0.0f) + alpha * acc[v];
    }
  }
}

}  // namespace wr

using namespace wr;

// C (M x N) = [C +] alpha * A (M x K) * op(B); b_kn selects B stored K x N.
int wr_gemm_f32(hipStream_t st, int M, int N, int K, const float* A, int64_t lda, const float* B, int64_t ldb,
                bool b_kn, float* C, int64_t ldc, float alpha, bool accumulate, bool lower_tiles,
                const int32_t* dev_info) {
  if (M <= 0 || N <= 0) return WR_OK;
  dim3 grid;
  if (lower_tiles) {
    const int nt = (M + GM_T - 1) / GM_T;
    grid = dim3((unsigned)(nt * (nt + 1) / 2));
  } else {
    grid = dim3((unsigned)((N + GM_T - 1) / GM_T), (unsigned)((M + GM_T - 1) / GM_T));
  }
  if (b_kn)
    hipLaunchKernelGGL(gemm_f32_kernel<true>, grid, dim3(256), 0, st, M, N, K, A, lda, B, ldb, C, ldc, alpha,
                       (int)accumulate, (int)lower_tiles, dev_info);
  else
    hipLaunchKernelGGL(gemm_f32_kernel<false>, grid, dim3(256), 0, st, M, N, K, A, lda, B, ldb, C, ldc, alpha,
                       (int)accumulate, (int)lower_tiles, dev_info);
  WR_CHECK_LAUNCH();
  return WR_OK;
}
