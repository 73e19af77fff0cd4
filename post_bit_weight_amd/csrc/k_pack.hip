// Bit-packing of codes and fp16 scales (Wringer model cards, "What is in this
// repo": the container holds packed codes plus fp16 block scales).  Layout:
// per row, code j occupies bits [j b, (j+1) b) of the row's bit stream, least
// significant bit first in little-endian bytes; then the scales as
// little-endian fp16, row-major.  One thread handles 8 codes = b bytes.
#include "common.hpp"

namespace wr {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

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

// Vector forms for aligned buffers (codes, packed stream and dequant output 16-byte aligned,
// rows x n a multiple of 32): rows are byte-aligned in the stream, so the codes of the whole
// module form one continuous bit stream and thread t packs codes 32 t .. 32 t + 31 into the B
// dwords t B .. t B + B - 1 (two 16-byte loads, B dword stores that the lanes of a wave lay end
// to end).  The same launch then copies the scales, which are stored in their own byte order
// (little-endian fp16), 16 bytes per thread when both ends allow it.
template <int B>
__device__ __forceinline__ void pack32(const u32x4 lo, const u32x4 hi, uint32_t (&d)[B]) {
  const uint32_t w[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
  for (int q = 0; q < B; ++q) d[q] = 0u;
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    const uint32_t c = (w[e >> 2] >> (8 * (e & 3))) & ((1u << B) - 1u);
    const int pos = B * e, q = pos >> 5, sh = pos & 31;
    d[q] |= c << sh;
    if (sh + B > 32) d[q + 1] |= c >> (32 - sh);
  }
}

__device__ __forceinline__ void copy_bytes(const uint8_t* __restrict__ src, int64_t nbytes, uint8_t* __restrict__ dst,
                                           int64_t tid, int64_t nthreads) {
  if ((((uintptr_t)src | (uintptr_t)dst) & 15) == 0) {
    const int64_t nv = nbytes / 16;
    for (int64_t i = tid; i < nv; i += nthreads)
      reinterpret_cast<u32x4*>(dst)[i] = reinterpret_cast<const u32x4*>(src)[i];
    for (int64_t i = 16 * nv + tid; i < nbytes; i += nthreads) dst[i] = src[i];
  } else {
    for (int64_t i = tid; i < nbytes; i += nthreads) dst[i] = src[i];
  }
}

template <int B>
__global__ __launch_bounds__(256) void pack_vec_kernel(const uint8_t* __restrict__ codes, int64_t n32,
                                                       const uint16_t* __restrict__ scales, int64_t scale_bytes,
                                                       uint8_t* __restrict__ out) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x, nthreads = (int64_t)gridDim.x * blockDim.x;
  for (int64_t t = tid; t < n32; t += nthreads) {
    const u32x4 lo = *reinterpret_cast<const u32x4*>(codes + 32 * t);
    const u32x4 hi = *reinterpret_cast<const u32x4*>(codes + 32 * t + 16);
    uint32_t d[B];
    pack32<B>(lo, hi, d);
    uint32_t* o = reinterpret_cast<uint32_t*>(out + 4 * B * t);
    if constexpr (B == 4) {
      *reinterpret_cast<u32x4*>(o) = u32x4{d[0], d[1], d[2], d[3]};
    } else if constexpr (B == 2) {
      *reinterpret_cast<u32x2*>(o) = u32x2{d[0], d[1]};
    } else {
#pragma unroll
      for (int q = 0; q < B; ++q) o[q] = d[q];
    }
  }
  copy_bytes(reinterpret_cast<const uint8_t*>(scales), scale_bytes, out + 4 * B * n32, tid, nthreads);
}

// Inverse: thread t reads the B dwords of codes 32 t .. 32 t + 31 and writes the codes (two
// 16-byte stores) and/or their dequantized bf16 values (four); with n and the group multiples of
// 32 the 32 codes share one row and one scale.  The same launch copies the scales out.
template <int B>
__global__ __launch_bounds__(256) void unpack_vec_kernel(const uint8_t* __restrict__ in, int64_t n32, int n, int group,
                                                         int64_t scale_bytes, uint8_t* __restrict__ codes,
                                                         uint16_t* __restrict__ scales, uint16_t* __restrict__ dequant) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x, nthreads = (int64_t)gridDim.x * blockDim.x;
  const uint8_t* sbytes = in + 4 * B * n32;
  const int nb = n / group, n32row = n / 32;
  constexpr int L = (1 << B) - 1;
  for (int64_t t = tid; t < n32; t += nthreads) {
    const uint32_t* src = reinterpret_cast<const uint32_t*>(in + 4 * B * t);
    uint32_t d[B + 1];
#pragma unroll
    for (int q = 0; q < B; ++q) d[q] = src[q];
    d[B] = 0u;
    uint32_t c[32];
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      const int pos = B * e, q = pos >> 5, sh = pos & 31;
      uint32_t v = d[q] >> sh;
      if (sh + B > 32) v |= d[q + 1] << (32 - sh);
      c[e] = v & (uint32_t)L;
    }
    if (codes) {
      u32x4 w0, w1;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        w0[q] = c[4 * q] | (c[4 * q + 1] << 8) | (c[4 * q + 2] << 16) | (c[4 * q + 3] << 24);
        w1[q] = c[16 + 4 * q] | (c[17 + 4 * q] << 8) | (c[18 + 4 * q] << 16) | (c[19 + 4 * q] << 24);
      }
      *reinterpret_cast<u32x4*>(codes + 32 * t) = w0;
      *reinterpret_cast<u32x4*>(codes + 32 * t + 16) = w1;
    }
    if (dequant) {
      const int64_t row = t / n32row;
      const int col = (int)(t - row * n32row) * 32;
      const int64_t sb = 2 * (row * nb + col / group);
      const float s = f16_bits_to_f32((uint16_t)(sbytes[sb] | (sbytes[sb + 1] << 8)));
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        u32x4 w;
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const int e = 8 * q + 2 * h;
          const uint32_t lo = f32_to_bf16_bits((float)(2 * (int)c[e] - L) * s);
          const uint32_t hi = f32_to_bf16_bits((float)(2 * (int)c[e + 1] - L) * s);
          w[h] = lo | (hi << 16);
        }
        *reinterpret_cast<u32x4*>(dequant + 32 * t + 8 * q) = w;
      }
    }
  }
  if (scales) copy_bytes(sbytes, scale_bytes, reinterpret_cast<uint8_t*>(scales), tid, nthreads);
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

// Lane exchange at distance LH inside a wave (partner lane = lane ^ LH): DPP for the
// distances inside a 16-lane row, a bpermute for 16 and 32.
template <int LH>
__device__ __forceinline__ float xor_lane(float x) {
  const int i = __float_as_int(x);
  if constexpr (LH == 1) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(i, 0xB1, 0xF, 0xF, true));  // quad_perm [1,0,3,2]
  } else if constexpr (LH == 2) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(i, 0x4E, 0xF, 0xF, true));  // quad_perm [2,3,0,1]
  } else if constexpr (LH == 4) {
    // half-row mirror (i -> 7 - i) then quad reverse (i -> i ^ 3): i -> i ^ 4
    const int t = __builtin_amdgcn_mov_dpp(i, 0x141, 0xF, 0xF, true);
    return __int_as_float(__builtin_amdgcn_mov_dpp(t, 0x1B, 0xF, 0xF, true));
  } else if constexpr (LH == 8) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(i, 0x128, 0xF, 0xF, true));  // row_ror:8
  } else {
    return __shfl_xor(x, LH);
  }
}

// acc += k * acc[partner], the partner's value taken by DPP inside the fma (one VALU op per
// element).  The s_nop keeps the two wait states a DPP read needs after a VALU write of its
// source register.
// Eight at a time, v[B .. B+7], behind one s_nop: inside the block no instruction writes a
// register that a later one reads.
#define WR_DPP1(i, CTRL) "\n\tv_fmac_f32_dpp %" #i ", %" #i ", %8 " CTRL " row_mask:0xf bank_mask:0xf bound_ctrl:1"
#define WR_FMAC_DPP8(v, B, k, CTRL)                                                                                  \
  asm volatile("s_nop 1" WR_DPP1(0, CTRL) WR_DPP1(1, CTRL) WR_DPP1(2, CTRL) WR_DPP1(3, CTRL) WR_DPP1(4, CTRL)        \
                   WR_DPP1(5, CTRL) WR_DPP1(6, CTRL) WR_DPP1(7, CTRL)                                               \
               : "+v"(v[B]), "+v"(v[B + 1]), "+v"(v[B + 2]), "+v"(v[B + 3]), "+v"(v[B + 4]), "+v"(v[B + 5]),       \
                 "+v"(v[B + 6]), "+v"(v[B + 7])                                                                     \
               : "v"(k))

typedef _Float16 h2v __attribute__((ext_vector_type(2)));
typedef float f32x2v __attribute__((ext_vector_type(2)));

// (x, y) -> (x + y, x - y) on the two halves of a packed fp16 register, in one op.
__device__ __forceinline__ h2v pk_half_butterfly(h2v a) {
  h2v r;
  asm("v_pk_add_f16 %0, %1, %1 op_sel:[0,1] op_sel_hi:[0,1] neg_hi:[0,1]" : "=v"(r) : "v"(a));
  return r;
}

// (x & mask) | bits in one op (the mask in a scalar register, the bits in a vector register).
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t mask, uint32_t bits) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(mask), "v"(bits));
  return r;
}
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

// Materialize, chunk form (n_store % 64 == 0, aligned buffers): lane i of the grid handles
// chunk i of the flattened (row, 64-column chunk) index, so the chunks of one Hadamard block
// of m = 64 A columns sit on A lanes of one wave (for A = 8 lane bits 2 and 3 trade places, so
// that the three exchanges are at lane distances 1, 2 and 8, one DPP pattern each).  The lane reads its 64 codes
// with one to three vector loads and its scales (one per chunk when the group is a multiple
// of 64, else G = group columns each), dequantizes exactly ((2c - L) s: a product of small
// integers and an fp16 value), runs the butterflies at distances below min(m, 64) in
// registers and the others across lanes: u = y + k y_partner with k = -1 on the upper lane of
// each pair, so that a lane holds its true value times (-1)^(number of exchanges in which it
// was the upper lane), a sign folded into the final scale by 1/sqrt(m); rounds pairs to bf16 with v_cvt_pk_bf16_f32 (round to nearest even), and puts
// the signs d_j into the bf16 sign bits (exact: a sign change commutes with the rounding).
// LOGA: log2(m / 64) for a rotation of block m >= 64 (the number of exchanges across lanes),
// -1 for no rotation.
template <int BITS, int G, int LOGA>
__global__ __launch_bounds__(64, (LOGA >= 5 ? 4 : 5)) void materialize_chunk_kernel(const uint8_t* __restrict__ in, int64_t rows,
                                                                int n_store, int group,
                                                                const int8_t* __restrict__ signs, float scale,
                                                                int n_out, uint16_t* __restrict__ out, int64_t ldo) {
  const int lane = threadIdx.x;
  constexpr bool SWAP23 = LOGA == 3;
  const int lane_log = SWAP23 ? ((lane & 0x33) | ((lane >> 1) & 4) | ((lane << 1) & 8)) : lane;
  const int nch = n_store >> 6;
  const int64_t total = rows * nch;
  const int64_t id0 = (int64_t)blockIdx.x * 64 + lane_log;
  const bool live = id0 < total;
  const int64_t id = live ? id0 : total - 1;  // every lane takes part in the exchanges
  const int64_t r = id / nch;
  const int q = (int)(id - r * nch);
  const int j0 = q << 6;
  const int64_t rowbytes = (int64_t)(n_store >> 3) * BITS;
  const uint8_t* cp = in + r * rowbytes + (int64_t)q * (8 * BITS);
  uint32_t w[2 * BITS];
  if constexpr (BITS == 3) {
#pragma unroll
    for (int t = 0; t < 3; ++t) {
      const uint2 x = *reinterpret_cast<const uint2*>(cp + 8 * t);
      w[2 * t] = x.x;
      w[2 * t + 1] = x.y;
    }
  } else {
#pragma unroll
    for (int t = 0; t < BITS / 2; ++t) {
      const u32x4 x = *reinterpret_cast<const u32x4*>(cp + 16 * t);
#pragma unroll
      for (int u = 0; u < 4; ++u) w[4 * t + u] = x[u];
    }
  }
  constexpr int NS = 64 / G;
  const uint8_t* sp = in + rows * rowbytes + r * (int64_t)(n_store / group) * 2;
  const int gi0 = j0 / group;
  float s[NS];
#pragma unroll
  for (int t = 0; t < NS; ++t)
    s[t] = f16_bits_to_f32(*reinterpret_cast<const uint16_t*>(sp + 2 * (gi0 + t)));  // rows start at even offsets
  constexpr bool rotate = LOGA >= 0;
  constexpr int L = (1 << BITS) - 1;
  float v[64];
  if constexpr (!rotate) {
#pragma unroll
    for (int e = 0; e < 64; ++e) {
      const int bit = e * BITS;
      uint32_t c;
      if ((bit & 31) + BITS <= 32)
        c = (w[bit >> 5] >> (bit & 31)) & L;
      else
        c = ((w[bit >> 5] >> (bit & 31)) | (w[(bit >> 5) + 1] << (32 - (bit & 31)))) & L;
      const float sc = s[e / G];
      v[e] = fmaf((float)c, 2.0f * sc, -(float)L * sc);  // exact
    }
  } else {
    // Butterflies at distances below the group G run on the codes c themselves, two per
    // packed fp16 register (exact: every partial sum is an integer of magnitude <= 64 L < 2048).
    // Register p holds the elements elo(p) and elo(p) + HB.  With FWHT_G(1) = G at index 0 of
    // each G-block, the transform of the levels is 2 P - G L [e % G == 0], times s: exact in fp32.
    constexpr int HB = BITS == 4 ? 4 : 8;
    auto elo = [](int p) { return (p & (HB - 1)) | ((p / HB) * (2 * HB)); };
    const h2v magic = __builtin_bit_cast(h2v, 0x64006400u);  // 1024, 1024
    const uint32_t magic_bits = __builtin_amdgcn_readfirstlane(0x64006400u) + 0u * lane;  // in a vector register
    h2v P[32];
#pragma unroll
    for (int p = 0; p < 32; ++p) {
      uint32_t pair;
      if constexpr (BITS == 2) {
        pair = and_or(w[p >> 3] >> (2 * (p & 7)), 0x00030003u, magic_bits);  // codes 16 d + k, 16 d + k + 8
      } else if constexpr (BITS == 4) {
        pair = and_or(w[p >> 2] >> (4 * (p & 3)), 0x000F000Fu, magic_bits);  // codes 8 d + k, 8 d + k + 4
      } else {
        uint32_t c2[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int bit = (elo(p) + u * HB) * 3;
          if ((bit & 31) + 3 <= 32)
            c2[u] = (w[bit >> 5] >> (bit & 31)) & 7u;
          else
            c2[u] = ((w[bit >> 5] >> (bit & 31)) | (w[(bit >> 5) + 1] << (32 - (bit & 31)))) & 7u;
        }
        pair = c2[0] | (c2[1] << 16) | 0x64006400u;
      }
      P[p] = __builtin_bit_cast(h2v, pair) - magic;
    }
    static_for<0, 6>([&](auto kc) {
      constexpr int h = 1 << decltype(kc)::value;
      if constexpr (h < G) {
        if constexpr (h == HB) {
#pragma unroll
          for (int p = 0; p < 32; ++p) P[p] = pk_half_butterfly(P[p]);
        } else {
          constexpr int dp = h < HB ? h : h / 2;
#pragma unroll
          for (int p = 0; p < 32; ++p)
            if (!(p & dp)) {
              const h2v a = P[p], b = P[p + dp];
              P[p] = a + b;
              P[p + dp] = a - b;
            }
        }
      }
    });
#pragma unroll
    for (int p = 0; p < 32; ++p) {
      v[elo(p)] = (float)P[p].x;
      v[elo(p) + HB] = (float)P[p].y;
    }
#pragma unroll
    for (int e = 0; e < 64; ++e) {
      const float sc = s[e / G];
      v[e] = (e % G == 0) ? fmaf(v[e], 2.0f * sc, -(float)(G * L) * sc) : v[e] * (2.0f * sc);
    }
#pragma unroll
    for (int h = G; h < 64; h <<= 1)
#pragma unroll
      for (int e = 0; e < 64; ++e)
        if (!(e & h)) {
          const float a = v[e], b = v[e + h];
          v[e] = a + b;
          v[e + h] = a - b;
        }
    static_for<0, (LOGA > 0 ? LOGA : 0)>([&](auto kc) {
      constexpr int i = decltype(kc)::value;
      constexpr int lh = (SWAP23 && i == 2) ? 8 : (1 << i);
      const float sgn = (lane & lh) ? -1.0f : 1.0f;
      if constexpr (lh == 1) {
        #pragma unroll
        for (int b = 0; b < 64; b += 8) WR_FMAC_DPP8(v, b, sgn, "quad_perm:[1,0,3,2]");
      } else if constexpr (lh == 2) {
        #pragma unroll
        for (int b = 0; b < 64; b += 8) WR_FMAC_DPP8(v, b, sgn, "quad_perm:[2,3,0,1]");
      } else if constexpr (lh == 8) {
        #pragma unroll
        for (int b = 0; b < 64; b += 8) WR_FMAC_DPP8(v, b, sgn, "row_ror:8");
      } else {
#pragma unroll
        for (int e = 0; e < 64; ++e) v[e] = fmaf(xor_lane<lh>(v[e]), sgn, v[e]);
      }
    });
#pragma unroll
    for (int e = 0; e < 64; ++e) v[e] *= scale;
  }
  uint32_t sg[16];
  if constexpr (rotate) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const u32x4 x = *reinterpret_cast<const u32x4*>(signs + j0 + 16 * t);
#pragma unroll
      for (int u = 0; u < 4; ++u) sg[4 * t + u] = x[u];
    }
    // the lane's sign from the exchanges joins the signs d_j (exact)
    const int upper = LOGA > 0 ? __builtin_popcount(lane & (SWAP23 ? 0xB : (1 << (LOGA > 0 ? LOGA : 0)) - 1)) : 0;
    const uint32_t flip = (upper & 1) ? 0x80808080u : 0u;
#pragma unroll
    for (int t = 0; t < 16; ++t) sg[t] ^= flip;
  }
  uint32_t o[32];
#pragma unroll
  for (int p = 0; p < 32; ++p) {
    o[p] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2v){v[2 * p], v[2 * p + 1]}, bf16x2v));
    if constexpr (rotate) {
      // bytes (2p, 2p + 1) of the signs -> bit 7 of each into bits 15 and 31
      const uint32_t D = sg[p >> 1];
      const uint32_t sel = (p & 1) ? 0x030C020Cu : 0x010C000Cu;
      o[p] ^= __builtin_amdgcn_perm(0u, D, sel) & 0x80008000u;
    }
  }
  if (n_out % 64 == 0) {
    // every chunk is stored whole: through LDS, so that each store instruction writes whole
    // 128-byte lines (8 lanes per chunk) instead of 16 bytes into each of 64 lines.  Piece t of
    // lane c sits at c * 128 + 16 (t ^ (c & 7)) bytes (XOR swizzle against bank conflicts).
    __shared__ u32x4 tile[64 * 8];
#pragma unroll
    for (int t = 0; t < 8; ++t) tile[lane * 8 + (t ^ (lane & 7))] = u32x4{o[4 * t], o[4 * t + 1], o[4 * t + 2], o[4 * t + 3]};
    __syncthreads();
    const int64_t base = (int64_t)blockIdx.x * 64;
    const int64_t r0 = base / nch;
    const int q0 = (int)(base - r0 * nch);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int c = 8 * t + (lane >> 3), k = lane & 7;
      const int cl = SWAP23 ? ((c & 0x33) | ((c >> 1) & 4) | ((c << 1) & 8)) : c;
      if (base + cl < total) {
        int qc = q0 + cl;
        int64_t rc = r0;
        while (qc >= nch) {
          qc -= nch;
          ++rc;
        }
        if (64 * qc < n_out)  // chunks past n_out are the cropped padding; streamed past the caches
          __builtin_nontemporal_store(tile[c * 8 + (k ^ (c & 7))],
                                      reinterpret_cast<u32x4*>(out + rc * ldo + 64 * qc + 8 * k));
      }
    }
  } else if (live) {
    uint16_t* op = out + r * ldo + j0;
    if (j0 + 64 <= n_out) {
#pragma unroll
      for (int t = 0; t < 8; ++t)
        *reinterpret_cast<u32x4*>(op + 8 * t) = u32x4{o[4 * t], o[4 * t + 1], o[4 * t + 2], o[4 * t + 3]};
    } else {
#pragma unroll
      for (int e = 0; e < 64; ++e)
        if (j0 + e < n_out) op[e] = (uint16_t)(o[e >> 1] >> (16 * (e & 1)));
    }
  }
}

}  // namespace wr

using namespace wr;

static unsigned grid_for(int64_t work) { return (unsigned)std::max<int64_t>(1, std::min<int64_t>((work + 255) / 256, 8192)); }

// The vector kernels take 16-byte aligned buffers and whole 32-code pieces; others take the
// byte forms.
static bool vec_ok(const void* a, const void* b, const void* c, int64_t n, int32_t group) {
  const uintptr_t m = (uintptr_t)a | (uintptr_t)b | (uintptr_t)c;
  return (m & 15) == 0 && n % 32 == 0 && group % 32 == 0;
}

int wr_pack_impl(wr_ctx* ctx, const uint8_t* codes, const uint16_t* scales, int64_t rows, int64_t n, int32_t bits,
                 int32_t group, uint8_t* out) {
  const int64_t groups = rows * (n / 8);
  const int64_t code_bytes = rows * n * bits / 8;
  const int64_t ns = rows * (n / group);
  if (rows > 0 && vec_ok(codes, out, nullptr, n, group)) {
    const int64_t n32 = rows * n / 32;
    const unsigned grid = grid_for(std::max<int64_t>(n32, 1));
    if (bits == 2) hipLaunchKernelGGL(pack_vec_kernel<2>, dim3(grid), dim3(256), 0, ctx->stream, codes, n32, scales, 2 * ns, out);
    else if (bits == 3) hipLaunchKernelGGL(pack_vec_kernel<3>, dim3(grid), dim3(256), 0, ctx->stream, codes, n32, scales, 2 * ns, out);
    else hipLaunchKernelGGL(pack_vec_kernel<4>, dim3(grid), dim3(256), 0, ctx->stream, codes, n32, scales, 2 * ns, out);
    WR_CHECK_LAUNCH();
    return WR_OK;
  }
  if (groups > 0) {
    hipLaunchKernelGGL(pack_codes_kernel, dim3(grid_for(groups)), dim3(256), 0, ctx->stream, codes, groups, (int)(n / 8),
                       bits, out);
    WR_CHECK_LAUNCH();
  }
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
  if (rows > 0 && (codes || scales || dequant) && vec_ok(in, codes, dequant, n, group) && (uintptr_t)scales % 16 == 0) {
    const int64_t n32 = rows * n / 32, sbytes = 2 * rows * (n / group);
    const unsigned grid = grid_for(std::max<int64_t>(n32, 1));
    if (bits == 2)
      hipLaunchKernelGGL(unpack_vec_kernel<2>, dim3(grid), dim3(256), 0, ctx->stream, in, n32, (int)n, group, sbytes, codes, scales, dequant);
    else if (bits == 3)
      hipLaunchKernelGGL(unpack_vec_kernel<3>, dim3(grid), dim3(256), 0, ctx->stream, in, n32, (int)n, group, sbytes, codes, scales, dequant);
    else
      hipLaunchKernelGGL(unpack_vec_kernel<4>, dim3(grid), dim3(256), 0, ctx->stream, in, n32, (int)n, group, sbytes, codes, scales, dequant);
    WR_CHECK_LAUNCH();
    return WR_OK;
  }
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
  const bool chunk = n_store % 64 == 0 && reinterpret_cast<uintptr_t>(in) % 16 == 0 &&
                     reinterpret_cast<uintptr_t>(out) % 16 == 0 && ldo % 8 == 0 && (group % 64 == 0 || group == 32) &&
                     (had_block == 0 || (had_block >= 64 && reinterpret_cast<uintptr_t>(signs) % 16 == 0));
  if (chunk) {
    const int64_t total = rows * (n_store / 64);
    const dim3 grid((unsigned)((total + 63) / 64));
    const float scale = had_block > 0 ? 1.0f / std::sqrt((float)had_block) : 1.0f;
    int loga = -1;
    if (had_block > 0)
      for (loga = 0; (64 << loga) < had_block; ++loga) {
      }
#define WR_MATC(B, GG, LA)                                                                                        \
  hipLaunchKernelGGL((materialize_chunk_kernel<B, GG, LA>), grid, dim3(64), 0, ctx->stream, in, rows,            \
                     (int)n_store, group, signs, scale, (int)n_out, out, ldo)
#define WR_MATC_A(B, GG)               \
  switch (loga) {                      \
    case -1: WR_MATC(B, GG, -1); break; \
    case 0: WR_MATC(B, GG, 0); break;   \
    case 1: WR_MATC(B, GG, 1); break;   \
    case 2: WR_MATC(B, GG, 2); break;   \
    case 3: WR_MATC(B, GG, 3); break;   \
    case 4: WR_MATC(B, GG, 4); break;   \
    case 5: WR_MATC(B, GG, 5); break;   \
    default: WR_MATC(B, GG, 6); break;  \
  }
#define WR_MATC_G(B)           \
  if (group % 64 == 0) {       \
    WR_MATC_A(B, 64)           \
  } else {                     \
    WR_MATC_A(B, 32)           \
  }
    switch (bits) {
      case 2: WR_MATC_G(2); break;
      case 3: WR_MATC_G(3); break;
      default: WR_MATC_G(4); break;
    }
#undef WR_MATC_G
#undef WR_MATC_A
#undef WR_MATC
    WR_CHECK_LAUNCH();
    return WR_OK;
  }
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
