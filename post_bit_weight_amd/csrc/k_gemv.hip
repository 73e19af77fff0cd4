// Product of a packed module with input vectors (the decode-time use of the container of the
// Wringer model cards, "What is in this repo"): y = W_q R x_pad for the module stored in the
// rotated, zero-padded basis.  Two kernels:
//   gemv_prep_kernel  x' = R x_pad for each input vector (the Hadamard blocks in LDS), and the
//                     sum of x' over each 32-column chunk;
//   gemv_kernel       16 lanes per row, each walking 32-column chunks of the row: one 8/12/16-byte
//                     read of the chunk's codes, its fp16 scale, and
//                       s (2 sum_e c_e x'_e - L sum_e x'_e)
//                     per input vector (the level 2c - L split so that a weight costs one extract
//                     and one fma per vector); the lanes of a row add their partial sums by
//                     shuffles in a fixed order, so the result is deterministic.
#include "common.hpp"

namespace wr {

constexpr int GV_CHUNK = 32;

// one workgroup per (segment, vector): a Hadamard block of m columns (or 256 columns without a
// rotation); x' and the chunk sums go to the workspace
__global__ __launch_bounds__(256) void gemv_prep_kernel(const float* __restrict__ x, int64_t ldx, int n_in, int n_store,
                                                        int m, int log2m, const int8_t* __restrict__ signs, float scale,
                                                        float* __restrict__ xr, float* __restrict__ sums) {
  extern __shared__ float seg[];
  const int b = blockIdx.y;
  const int len = m > 0 ? m : 256;
  const int j0 = blockIdx.x * len;
  const float* xb = x + (int64_t)b * ldx;
  for (int i = threadIdx.x; i < len; i += blockDim.x) {
    const int j = j0 + i;
    float v = (j < n_in) ? xb[j] : 0.0f;
    if (m > 0) v *= (float)signs[j];
    seg[i] = v;
  }
  __syncthreads();
  for (int h = 1; m > 0 && h < m; h <<= 1) {
    for (int i = threadIdx.x; i < m / 2; i += blockDim.x) {
      const int lo = (i / h) * 2 * h + (i % h);
      const float a = seg[lo], c = seg[lo + h];
      seg[lo] = a + c;
      seg[lo + h] = a - c;
    }
    __syncthreads();
  }
  float* xo = xr + (int64_t)b * n_store;
  for (int i = threadIdx.x; i < len; i += blockDim.x) {
    if (j0 + i < n_store) {
      const float v = m > 0 ? seg[i] * scale : seg[i];
      seg[i] = v;
      xo[j0 + i] = v;
    }
  }
  __syncthreads();
  const int nch = n_store / GV_CHUNK;
  for (int c = threadIdx.x; c < len / GV_CHUNK; c += blockDim.x) {
    const int q = j0 / GV_CHUNK + c;
    if (q < nch) {
      float s = 0.0f;
      for (int e = 0; e < GV_CHUNK; ++e) s += seg[c * GV_CHUNK + e];
      sums[(int64_t)b * nch + q] = s;
    }
  }
}

template <int BITS, int BMAX>
__global__ __launch_bounds__(256) void gemv_kernel(const uint8_t* __restrict__ in, int64_t rows, int n_store, int group,
                                                   const float* __restrict__ xr, const float* __restrict__ sums,
                                                   int batch, float* __restrict__ y, int64_t ldy) {
  constexpr int L = (1 << BITS) - 1;
  const int l16 = threadIdx.x & 15;
  const int64_t row0 = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const bool live = row0 < rows;
  const int64_t row = live ? row0 : rows - 1;
  const int nch = n_store / GV_CHUNK;
  const int64_t rowbytes = (int64_t)(n_store / 8) * BITS;
  const uint8_t* cp = in + row * rowbytes;
  const uint8_t* sp = in + rows * rowbytes + row * (int64_t)(n_store / group) * 2;
  float acc[BMAX];
#pragma unroll
  for (int b = 0; b < BMAX; ++b) acc[b] = 0.0f;
  for (int q = l16; q < nch; q += 16) {
    uint32_t w[BITS];  // 32 codes of BITS bits = BITS dwords
    if constexpr (BITS == 2) {
      const uint2 v = *reinterpret_cast<const uint2*>(cp + 8 * q);
      w[0] = v.x;
      w[1] = v.y;
    } else if constexpr (BITS == 4) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(cp + 16 * q);
#pragma unroll
      for (int u = 0; u < 4; ++u) w[u] = v[u];
    } else {
      const uint32_t* p = reinterpret_cast<const uint32_t*>(cp + 12 * q);
#pragma unroll
      for (int u = 0; u < 3; ++u) w[u] = p[u];
    }
    const int gi = q * GV_CHUNK / group;
    const float s = f16_bits_to_f32((uint16_t)(sp[2 * gi] | (sp[2 * gi + 1] << 8)));
    float c[GV_CHUNK];
#pragma unroll
    for (int e = 0; e < GV_CHUNK; ++e) {
      const int bit = e * BITS;
      uint32_t v;
      if ((bit & 31) + BITS <= 32)
        v = (w[bit >> 5] >> (bit & 31)) & L;
      else
        v = ((w[bit >> 5] >> (bit & 31)) | (w[(bit >> 5) + 1] << (32 - (bit & 31)))) & L;
      c[e] = (float)v;
    }
#pragma unroll
    for (int b = 0; b < BMAX; ++b) {
      if (b < batch) {
        const float* xp = xr + (int64_t)b * n_store + q * GV_CHUNK;
        float d = 0.0f;
#pragma unroll
        for (int t = 0; t < GV_CHUNK / 4; ++t) {
          const f32x4 xv = *reinterpret_cast<const f32x4*>(xp + 4 * t);
#pragma unroll
          for (int e = 0; e < 4; ++e) d = fmaf(c[4 * t + e], xv[e], d);
        }
        acc[b] = fmaf(s, fmaf(2.0f, d, -(float)L * sums[(int64_t)b * nch + q]), acc[b]);
      }
    }
  }
#pragma unroll
  for (int b = 0; b < BMAX; ++b) {
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) acc[b] += __shfl_xor(acc[b], o);
    if (live && l16 == 0 && b < batch) y[(int64_t)b * ldy + row] = acc[b];
  }
}

}  // namespace wr

using namespace wr;

size_t wr_gemv_ws_bytes(int64_t n_store, int32_t batch) {
  const size_t a = ((size_t)batch * n_store * 4 + 255) & ~(size_t)255;
  return a + (size_t)batch * (n_store / GV_CHUNK) * 4;
}

int wr_packed_gemv_impl(wr_ctx* ctx, const uint8_t* in, int64_t rows, int64_t n_store, int32_t bits, int32_t group,
                        int32_t had_block, const int8_t* signs, const float* x, int64_t n_in, int64_t ldx, int32_t batch,
                        float* y, int64_t ldy) {
  if (ctx->ws_bytes < wr_gemv_ws_bytes(n_store, batch)) return WR_EWORKSPACE;
  float* xr = static_cast<float*>(ctx->ws);
  float* sums = reinterpret_cast<float*>(static_cast<char*>(ctx->ws) +
                                         (((size_t)batch * n_store * 4 + 255) & ~(size_t)255));
  const int m = had_block;
  int log2m = 0;
  while ((1 << log2m) < m) ++log2m;
  const int len = m > 0 ? m : 256;
  const dim3 pgrid((unsigned)((n_store + len - 1) / len), (unsigned)batch);
  hipLaunchKernelGGL(gemv_prep_kernel, pgrid, dim3(256), len * sizeof(float), ctx->stream, x, ldx, (int)n_in,
                     (int)n_store, m, log2m, signs, m > 0 ? 1.0f / std::sqrt((float)m) : 1.0f, xr, sums);
  WR_CHECK_LAUNCH();
  if (rows == 0) return WR_OK;
  const dim3 grid((unsigned)((rows + 15) / 16));
#define WR_GV(BT, BM)                                                                                               \
  hipLaunchKernelGGL((gemv_kernel<BT, BM>), grid, dim3(256), 0, ctx->stream, in, rows, (int)n_store, group, xr, sums, \
                     batch, y, ldy)
#define WR_GV_B(BT)                      \
  if (batch == 1) {                      \
    WR_GV(BT, 1);                        \
  } else if (batch <= 4) {               \
    WR_GV(BT, 4);                        \
  } else {                               \
    WR_GV(BT, 8);                        \
  }
  switch (bits) {
    case 2: WR_GV_B(2); break;
    case 3: WR_GV_B(3); break;
    default: WR_GV_B(4); break;
  }
#undef WR_GV_B
#undef WR_GV
  WR_CHECK_LAUNCH();
  return WR_OK;
}
