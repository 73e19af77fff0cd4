// Product of a packed module with input vectors (the decode-time use of the container of the
// Wringer model cards, "What is in this repo"): y = W_q R x_pad for the module stored in the
// rotated, zero-padded basis.  Two kernels:
//   gemv_prep_kernel  x' = R x_pad for each input vector (the Hadamard blocks in LDS), when x'
//                     does not fit in the product's LDS (otherwise the product forms it);
//   gemv_kernel       16 lanes per group of 4 rows, each walking 32-column chunks: per chunk and
//                     row one 8/12/16-byte read of the codes and the fp16 scale, and
//                       s (2 sum_e c_e x'_e - L sum_e x'_e)
//                     per input vector (the level 2c - L split so that a weight costs one extract
//                     and one fma per vector; one read of x' serves the 4 rows); the lanes of a
//                     row group add their partial sums by shuffles in a fixed order, so the
//                     result is deterministic.
#include "common.hpp"

namespace wr {

constexpr int GV_CHUNK = 32;
// threads of a product workgroup: 32 row groups of RPL rows, so that a module of a few tens of
// thousands of rows makes about one workgroup per CU and each forms x' once
constexpr int GV_THREADS = 512;

// one workgroup per (segment, vector): a Hadamard block of m columns (or 256 columns without a
// rotation); x' = R x_pad goes to the workspace (used when x' does not fit in LDS)
__global__ __launch_bounds__(256) void gemv_prep_kernel(const float* __restrict__ x, int64_t ldx, int n_in, int n_store,
                                                        int m, int log2m, const int8_t* __restrict__ signs, float scale,
                                                        float* __restrict__ xr) {
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
  for (int lh = 0; lh < log2m; ++lh) {
    const int h = 1 << lh;
    for (int i = threadIdx.x; i < m / 2; i += blockDim.x) {
      const int lo = ((i >> lh) << (lh + 1)) | (i & (h - 1));
      const float a = seg[lo], c = seg[lo + h];
      seg[lo] = a + c;
      seg[lo + h] = a - c;
    }
    __syncthreads();
  }
  float* xo = xr + (int64_t)b * n_store;
  for (int i = threadIdx.x; i < len; i += blockDim.x)
    if (j0 + i < n_store) xo[j0 + i] = m > 0 ? seg[i] * scale : seg[i];
}

// byte N of v as a float (v_cvt_f32_ubyteN; written out because the compiler otherwise folds
// the byte selection into a bit-field extract plus a conversion)
template <int N>
__device__ __forceinline__ float ubyte_f32(uint32_t v) {
  float r;
  if constexpr (N == 0)
    asm("v_cvt_f32_ubyte0 %0, %1" : "=v"(r) : "v"(v));
  else if constexpr (N == 1)
    asm("v_cvt_f32_ubyte1 %0, %1" : "=v"(r) : "v"(v));
  else if constexpr (N == 2)
    asm("v_cvt_f32_ubyte2 %0, %1" : "=v"(r) : "v"(v));
  else
    asm("v_cvt_f32_ubyte3 %0, %1" : "=v"(r) : "v"(v));
  return r;
}

// LDS position of element i of x' (vectors back to back, n_store % 32 == 0): float4 t of the
// 32-element chunk q is stored at slot t ^ (q & 7), so that 16 lanes reading float4 t of 16
// consecutive chunks hit 16 different bank groups
__device__ __forceinline__ int xswz(int i) { return (i & ~31) | ((((i >> 2) & 7) ^ ((i >> 5) & 7)) << 2) | (i & 3); }

// the 32 codes of one chunk as floats
template <int BITS>
__device__ __forceinline__ void chunk_codes(const uint32_t (&w)[BITS], float (&c)[GV_CHUNK]) {
  constexpr int L = (1 << BITS) - 1;
  if constexpr (BITS == 2) {
    // dword d holds codes 16 d .. 16 d + 15; (w >> 2k) & 0x03030303 gives codes k, k+4, k+8, k+12
#pragma unroll
    for (int d = 0; d < 2; ++d)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t v = (w[d] >> (2 * k)) & 0x03030303u;
        c[16 * d + k] = ubyte_f32<0>(v);
        c[16 * d + k + 4] = ubyte_f32<1>(v);
        c[16 * d + k + 8] = ubyte_f32<2>(v);
        c[16 * d + k + 12] = ubyte_f32<3>(v);
      }
  } else if constexpr (BITS == 4) {
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const uint32_t v = (w[d] >> (4 * k)) & 0x0F0F0F0Fu;
        c[8 * d + k] = ubyte_f32<0>(v);
        c[8 * d + k + 2] = ubyte_f32<1>(v);
        c[8 * d + k + 4] = ubyte_f32<2>(v);
        c[8 * d + k + 6] = ubyte_f32<3>(v);
      }
  } else {
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
  }
}

template <int BITS>
__device__ __forceinline__ void load_codes(const uint8_t* p, uint32_t (&w)[BITS]) {
  if constexpr (BITS == 2) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    w[0] = v.x;
    w[1] = v.y;
  } else if constexpr (BITS == 4) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int u = 0; u < 4; ++u) w[u] = v[u];
  } else {
#pragma unroll
    for (int u = 0; u < 3; ++u) w[u] = reinterpret_cast<const uint32_t*>(p)[u];
  }
}

// 16 lanes per group of RPL rows: lane l handles the chunks l, l + 16, ... of all RPL rows, so one
// read of x' serves RPL rows; the codes and scales of NG chunks (the HBM traffic) are requested
// together, x' (a few KB, in LDS or cache-resident) just before its use.  Workgroup: GV_THREADS / 16 row
// groups.
// With XLDS the workgroup forms x' = R x_pad itself, in LDS (batch x n_store floats; the host
// checks they fit): x is read from global memory, the Hadamard butterflies run three stages per
// pass through LDS, and 1/sqrt(m) is applied to the outputs (the product is linear in x').  The first chunk's
// codes are requested before that, so their latency overlaps the butterflies.  Without XLDS, x'
// (already scaled) comes from the workspace.  Either way the chunk's sum of x' is formed in the
// main loop, once for the RPL rows.
template <int BITS, int BMAX, bool XLDS>
__global__ __launch_bounds__(GV_THREADS) void gemv_kernel(const uint8_t* __restrict__ in, int64_t rows, int n_store, int group,
                                                   const float* __restrict__ xr_g, int batch, float* __restrict__ y,
                                                   int64_t ldy, const float* __restrict__ x, int64_t ldx, int n_in,
                                                   int log2m, const int8_t* __restrict__ signs, float out_scale) {
  constexpr int L = (1 << BITS) - 1;
  constexpr int RPL = 4;  // rows per lane: one read of x' serves them
  constexpr int NG = 2;   // chunks whose codes and scales are requested together
  extern __shared__ float xl[];
  const int l16 = threadIdx.x & 15;
  const int64_t rbase = ((int64_t)blockIdx.x * (GV_THREADS / 16) + (threadIdx.x >> 4)) * RPL;
  const int nch = n_store / GV_CHUNK;
  const int64_t rowbytes = (int64_t)(n_store / 8) * BITS;
  const int nb = n_store / group;
  const uint8_t* cp[RPL];
  const uint8_t* sp[RPL];
#pragma unroll
  for (int r = 0; r < RPL; ++r) {
    const int64_t row = min(rbase + r, rows - 1);
    cp[r] = in + row * rowbytes;
    sp[r] = in + rows * rowbytes + row * (int64_t)nb * 2;
  }
  uint32_t w[NG][RPL][BITS];
  uint32_t sb[NG][RPL];
  auto fetch_group = [&](int q0) {  // chunks q0, q0 + 16, ..., up to NG of them
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const int q = q0 + 16 * g;
      if (q < nch) {
        const int gi = q * GV_CHUNK / group;
#pragma unroll
        for (int r = 0; r < RPL; ++r) {
          load_codes<BITS>(cp[r] + (int64_t)q * (GV_CHUNK / 8) * BITS, w[g][r]);
          sb[g][r] = *reinterpret_cast<const uint16_t*>(sp[r] + 2 * gi);  // 2-aligned: rowbytes is even
        }
      }
    }
  };
  fetch_group(l16);
  const float* xr = xr_g;
  if constexpr (XLDS) {
    const int tot = batch * n_store;
    for (int i = threadIdx.x; i < tot; i += GV_THREADS) {
      const int bi = i / n_store, j = i - bi * n_store;
      float v = j < n_in ? x[(int64_t)bi * ldx + j] : 0.0f;
      if (log2m > 0) v *= (float)signs[j];
      xl[xswz(i)] = v;
    }
    __syncthreads();
    // up to three butterfly stages per pass, in registers: a thread takes the 2^ns elements
    // base + k h that those stages combine (blocks of m never straddle: m | n_store), so a
    // pass costs one barrier; every element sees the same additions as stage by stage
    auto pass = [&](auto ns_tag, int lh) __attribute__((always_inline)) {
      constexpr int NS = decltype(ns_tag)::value, G = 1 << NS;
      const int h = 1 << lh;
      for (int gi = threadIdx.x; gi < tot / G; gi += GV_THREADS) {
        const int base = ((gi >> lh) << (lh + NS)) | (gi & (h - 1));
        float v[G];
#pragma unroll
        for (int k = 0; k < G; ++k) v[k] = xl[xswz(base + k * h)];
#pragma unroll
        for (int st = 0; st < NS; ++st)
#pragma unroll
          for (int k = 0; k < G; ++k)
            if (!(k & (1 << st))) {
              const float a = v[k], c = v[k + (1 << st)];
              v[k] = a + c;
              v[k + (1 << st)] = a - c;
            }
#pragma unroll
        for (int k = 0; k < G; ++k) xl[xswz(base + k * h)] = v[k];
      }
      __syncthreads();
    };
    for (int lh = 0; lh < log2m; lh += 3) {
      if (log2m - lh >= 3)
        pass(std::integral_constant<int, 3>{}, lh);
      else if (log2m - lh == 2)
        pass(std::integral_constant<int, 2>{}, lh);
      else
        pass(std::integral_constant<int, 1>{}, lh);
    }
    xr = xl;
  }
  float acc[RPL][BMAX];
#pragma unroll
  for (int r = 0; r < RPL; ++r)
#pragma unroll
    for (int b = 0; b < BMAX; ++b) acc[r][b] = 0.0f;
  for (int q0 = l16; q0 < nch; q0 += 16 * NG) {
    if (q0 != l16) fetch_group(q0);
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const int q = q0 + 16 * g;
      if (q < nch) {
#pragma unroll
        for (int b = 0; b < BMAX; ++b) {
          if (b < batch) {
            const float* xp = xr + (int64_t)b * n_store + q * GV_CHUNK;
            f32x4 xv[GV_CHUNK / 4];
#pragma unroll
            for (int t = 0; t < GV_CHUNK / 4; ++t)  // in LDS float4 t of chunk b nch + q is at slot t ^ ((b nch + q) & 7)
              xv[t] = *reinterpret_cast<const f32x4*>(xp + 4 * (XLDS ? (t ^ ((b * nch + q) & 7)) : t));
            float xs = 0.0f;
#pragma unroll
            for (int t = 0; t < GV_CHUNK / 4; ++t)
#pragma unroll
              for (int e = 0; e < 4; ++e) xs += xv[t][e];
#pragma unroll
            for (int r = 0; r < RPL; ++r) {
              float c[GV_CHUNK];
              chunk_codes<BITS>(w[g][r], c);
              float dd = 0.0f;
#pragma unroll
              for (int t = 0; t < GV_CHUNK / 4; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e) dd = fmaf(c[4 * t + e], xv[t][e], dd);
              acc[r][b] = fmaf(f16_bits_to_f32((uint16_t)sb[g][r]), fmaf(2.0f, dd, -(float)L * xs), acc[r][b]);
            }
          }
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < RPL; ++r)
#pragma unroll
    for (int b = 0; b < BMAX; ++b) {
      float a = acc[r][b];
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) a += __shfl_xor(a, o);
      if (l16 == 0 && rbase + r < rows && b < batch) y[(int64_t)b * ldy + rbase + r] = a * out_scale;
    }
}

}  // namespace wr

using namespace wr;

size_t wr_gemv_ws_bytes(int64_t n_store, int32_t batch) { return (size_t)batch * n_store * 4; }

int wr_packed_gemv_impl(wr_ctx* ctx, const uint8_t* in, int64_t rows, int64_t n_store, int32_t bits, int32_t group,
                        int32_t had_block, const int8_t* signs, const float* x, int64_t n_in, int64_t ldx, int32_t batch,
                        float* y, int64_t ldy) {
  const int m = had_block;
  int log2m = 0;
  while ((1 << log2m) < m) ++log2m;
  const size_t lds = (size_t)batch * n_store * sizeof(float);
  const bool fused = lds <= 64 * 1024;
  if (!fused && ctx->ws_bytes < wr_gemv_ws_bytes(n_store, batch)) return WR_EWORKSPACE;
  float* xr = static_cast<float*>(ctx->ws);
  const float rs = m > 0 ? 1.0f / std::sqrt((float)m) : 1.0f;
  if (rows == 0) return WR_OK;
  if (!fused) {
    const int len = m > 0 ? m : 256;
    const dim3 pgrid((unsigned)((n_store + len - 1) / len), (unsigned)batch);
    hipLaunchKernelGGL(gemv_prep_kernel, pgrid, dim3(256), len * sizeof(float), ctx->stream, x, ldx, (int)n_in,
                       (int)n_store, m, log2m, signs, rs, xr);
    WR_CHECK_LAUNCH();
  }
  const dim3 grid((unsigned)((rows + GV_THREADS / 4 - 1) / (GV_THREADS / 4)));
#define WR_GV(BT, BM)                                                                                                 \
  if (fused)                                                                                                          \
    hipLaunchKernelGGL((gemv_kernel<BT, BM, true>), grid, dim3(GV_THREADS), lds, ctx->stream, in, rows, (int)n_store, group, \
                       xr, batch, y, ldy, x, ldx, (int)n_in, log2m, signs, rs);                                       \
  else                                                                                                                \
    hipLaunchKernelGGL((gemv_kernel<BT, BM, false>), grid, dim3(GV_THREADS), 0, ctx->stream, in, rows, (int)n_store, group,  \
                       xr, batch, y, ldy, x, ldx, (int)n_in, log2m, signs, 1.0f)
#define WR_GV_B(BT)        \
  if (batch == 1) {        \
    WR_GV(BT, 1);          \
  } else if (batch <= 4) { \
    WR_GV(BT, 4);          \
  } else {                 \
    WR_GV(BT, 8);          \
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
