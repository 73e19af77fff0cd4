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
