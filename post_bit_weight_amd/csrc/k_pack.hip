// Bit-packing of codes and fp16 scales (Wringer model cards, "What is in this
// repo": the container holds packed codes plus fp16 block scales).  Layout:
// per row, code j occupies bits [j b, (j+1) b) of the row's bit stream, least
// significant bit first in little-endian bytes; then the scales as
// little-endian fp16, row-major.  One thread handles 8 codes = b bytes.
#include "common.hpp"

namespace wr {

__global__ void pack_codes_kernel(const uint8_t* __restrict__ codes, int64_t groups, int n8, int bits,
                                  uint8_t* __restrict__ out) {
  for (int64_t gidx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; gidx < groups;
       gidx += (int64_t)gridDim.x * blockDim.x) {
    const uint2 raw = *reinterpret_cast<const uint2*>(codes + gidx * 8);
    const uint32_t mask = (1u << bits) - 1u;
    uint32_t v = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t c = ((e < 4 ? raw.x : raw.y) >> (8 * (e & 3))) & 0xffu;
      v |= (c & mask) << (bits * e);
    }
    uint8_t* o = out + gidx * bits;
    for (int t = 0; t < bits; ++t) o[t] = (uint8_t)(v >> (8 * t));
  }
}

__global__ void unpack_codes_kernel(const uint8_t* __restrict__ in, int64_t groups, int n8, int n, int bits, int group,
                                    const uint8_t* __restrict__ scale_bytes, uint8_t* __restrict__ codes,
                                    uint16_t* __restrict__ dequant) {
  const int nb = n / group;
  const int L = (1 << bits) - 1;
  for (int64_t gidx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; gidx < groups;
       gidx += (int64_t)gridDim.x * blockDim.x) {
    const uint8_t* src = in + gidx * bits;
    uint32_t v = 0;
    for (int t = 0; t < bits; ++t) v |= (uint32_t)src[t] << (8 * t);
    const int64_t row = gidx / n8;
    const int col0 = (int)(gidx % n8) * 8;
    const int64_t sb = (row * nb + col0 / group) * 2;
    const uint16_t sbits = (uint16_t)(scale_bytes[sb] | (scale_bytes[sb + 1] << 8));
    const float s = f16_bits_to_f32(sbits);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t c = (v >> (bits * e)) & ((1u << bits) - 1u);
      if (codes) codes[gidx * 8 + e] = (uint8_t)c;
      if (dequant) dequant[gidx * 8 + e] = (uint16_t)f32_to_bf16_bits((float)(2 * (int)c - L) * s);
    }
  }
}

__global__ void pack_scales_kernel(const uint16_t* __restrict__ scales, int64_t count, uint8_t* __restrict__ out) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += (int64_t)gridDim.x * blockDim.x) {
    const uint16_t s = scales[i];
    out[2 * i] = (uint8_t)(s & 0xffu);
    out[2 * i + 1] = (uint8_t)(s >> 8);
  }
}

__global__ void unpack_scales_kernel(const uint8_t* __restrict__ in, int64_t count, uint16_t* __restrict__ scales) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += (int64_t)gridDim.x * blockDim.x)
    scales[i] = (uint16_t)(in[2 * i] | (in[2 * i + 1] << 8));
}

// Materialize one module.  One wave per (row, segment of 64 E columns): lane t holds the
// E consecutive columns t E .. t E + E - 1, reads their codes as one little-endian bit
// field and their scales, and dequantizes exactly.  With a rotation of block m (m = 64 E,
// or E = 1 and m < 64, the segment then holding 64 / m blocks) it applies
// R^T = diag(d) H_m / sqrt(m): the unnormalised Walsh-Hadamard butterflies in increasing
// distance below m (distances below E inside the lane, the others across lanes), then the
// scale and the signs.  The first n_out columns are rounded to bf16 once.  Workgroup:
// four waves on four (row, segment) pairs of one segment column.
template <int E>
__global__ __launch_bounds__(256) void materialize_kernel(const uint8_t* __restrict__ in, int64_t rows, int n_store,
                                                          int bits, int group, int rotate, int m,
                                                          const int8_t* __restrict__ signs, float scale, int n_out,
                                                          uint16_t* __restrict__ out, int64_t ldo) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.y * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const int j0 = blockIdx.x * (64 * E) + lane * E;
  const int L = (1 << bits) - 1;
  const int nb = n_store / group;
  const uint8_t* row = in + r * ((int64_t)n_store * bits / 8);
  const uint8_t* sc = in + rows * ((int64_t)n_store * bits / 8) + r * nb * 2;
  float v[E];
  if (j0 < n_store) {  // n_store % 8 == 0 and E columns never straddle n_store when E <= 8 ...
    const int64_t p0 = (int64_t)j0 * bits;  // ... and with a rotation n_store % (64 E) == 0
    const int nbits = E * bits;
    const int64_t byte0 = p0 >> 3;
    const int off = (int)(p0 & 7);
    const int nbytes = (off + nbits + 7) >> 3;
    uint64_t field[(E * 4 + 7) / 64 + 2] = {};
    for (int t = 0; t < nbytes; ++t) field[t >> 3] |= (uint64_t)row[byte0 + t] << (8 * (t & 7));
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int bp = off + e * bits;
      const int w = bp >> 6, sh = bp & 63;
      uint64_t x = field[w] >> sh;
      if (sh + bits > 64) x |= field[w + 1] << (64 - sh);
      const int c = (int)(x & (uint64_t)L);
      const int j = j0 + e;
      const int bj = (j < n_store ? j : n_store - 1) / group;
      const float s = f16_bits_to_f32((uint16_t)(sc[2 * bj] | (sc[2 * bj + 1] << 8)));
      v[e] = j < n_store ? (float)(2 * c - L) * s : 0.0f;  // exact: an fp16 scale times an odd integer below 16
    }
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) v[e] = 0.0f;
  }
  if (rotate) {
#pragma unroll
    for (int h = 1; h < E; h <<= 1)
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (!(e & h)) {
          const float a = v[e], b = v[e + h];
          v[e] = a + b;
          v[e + h] = a - b;
        }
#pragma unroll
    for (int lh = 1; lh < 64; lh <<= 1) {
      if (lh * E >= m) break;
      const bool upper = (lane & lh) != 0;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float o = __shfl_xor(v[e], lh);
        v[e] = upper ? o - v[e] : v[e] + o;
      }
    }
  }
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = j0 + e;
    if (rotate && j < n_store) v[e] = v[e] * scale * (float)signs[j];
  }
  uint16_t* o = out + r * ldo + j0;
  if (j0 + E <= n_out && (E % 8) == 0 && (reinterpret_cast<uintptr_t>(o) & 15) == 0) {
#pragma unroll
    for (int q = 0; q < E; q += 8) {
      u32x4 w;
#pragma unroll
      for (int u = 0; u < 4; ++u)
        w[u] = f32_to_bf16_bits(v[q + 2 * u]) | (f32_to_bf16_bits(v[q + 2 * u + 1]) << 16);
      *reinterpret_cast<u32x4*>(o + q) = w;
    }
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (j0 + e < n_out) o[e] = (uint16_t)f32_to_bf16_bits(v[e]);
  }
}

}  // namespace wr

using namespace wr;

static unsigned grid_for(int64_t work) { return (unsigned)std::max<int64_t>(1, std::min<int64_t>((work + 255) / 256, 8192)); }

int wr_pack_impl(wr_ctx* ctx, const uint8_t* codes, const uint16_t* scales, int64_t rows, int64_t n, int32_t bits,
                 int32_t group, uint8_t* out) {
  const int64_t groups = rows * (n / 8);
  const int64_t code_bytes = rows * n * bits / 8;
  if (groups > 0) {
    hipLaunchKernelGGL(pack_codes_kernel, dim3(grid_for(groups)), dim3(256), 0, ctx->stream, codes, groups, (int)(n / 8),
                       bits, out);
    WR_CHECK_LAUNCH();
  }
  const int64_t ns = rows * (n / group);
  if (ns > 0) {
    hipLaunchKernelGGL(pack_scales_kernel, dim3(grid_for(ns)), dim3(256), 0, ctx->stream, scales, ns, out + code_bytes);
    WR_CHECK_LAUNCH();
  }
  return WR_OK;
}

int wr_unpack_impl(wr_ctx* ctx, const uint8_t* in, int64_t rows, int64_t n, int32_t bits, int32_t group,
                   uint8_t* codes, uint16_t* scales, uint16_t* dequant) {
  const int64_t groups = rows * (n / 8);
  const int64_t code_bytes = rows * n * bits / 8;
  if (groups > 0 && (codes || dequant)) {
    hipLaunchKernelGGL(unpack_codes_kernel, dim3(grid_for(groups)), dim3(256), 0, ctx->stream, in, groups,
                       (int)(n / 8), (int)n, bits, group, in + code_bytes, codes, dequant);
    WR_CHECK_LAUNCH();
  }
  const int64_t ns = rows * (n / group);
  if (ns > 0 && scales) {
    hipLaunchKernelGGL(unpack_scales_kernel, dim3(grid_for(ns)), dim3(256), 0, ctx->stream, in + code_bytes, ns, scales);
    WR_CHECK_LAUNCH();
  }
  return WR_OK;
}

int wr_materialize_impl(wr_ctx* ctx, const uint8_t* in, int64_t rows, int64_t n_store, int32_t bits, int32_t group,
                        int32_t had_block, const int8_t* signs, int64_t n_out, uint16_t* out, int64_t ldo) {
  if (rows == 0) return WR_OK;
  // 64 E columns per wave: the Hadamard block with a rotation of 64..4096 columns, 64 for
  // smaller blocks, 512 without a rotation
  const int m = had_block > 0 ? had_block : 512;
  const int seg = m < 64 ? 64 : m;
  const int rotate = had_block > 0 ? 1 : 0;
  const float scale = rotate ? 1.0f / std::sqrt((float)m) : 1.0f;
  const dim3 grid((unsigned)((n_store + seg - 1) / seg), (unsigned)((rows + 3) / 4));
#define WR_MAT(EV)                                                                                                   \
  hipLaunchKernelGGL(materialize_kernel<EV>, grid, dim3(256), 0, ctx->stream, in, rows, (int)n_store, bits, group, \
                     rotate, m, signs, scale, (int)n_out, out, ldo)
  switch (seg) {
    case 64: WR_MAT(1); break;
    case 128: WR_MAT(2); break;
    case 256: WR_MAT(4); break;
    case 512: WR_MAT(8); break;
    case 1024: WR_MAT(16); break;
    case 2048: WR_MAT(32); break;
    default: WR_MAT(64); break;
  }
#undef WR_MAT
  WR_CHECK_LAUNCH();
  return WR_OK;
}
