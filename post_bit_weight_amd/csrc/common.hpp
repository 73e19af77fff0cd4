// Shared device helpers for the gfx950 quantization-solve kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <set>
#include <type_traits>
#include <utility>

#include "../../include/wringer.h"

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct wr_ctx {
  int device;
  hipStream_t stream;
  void* ws;
  size_t ws_bytes;
  int num_cu;
  float* scale_trace;         // wr_set_scale_trace: unprojected joint scales, or null
  int64_t scale_trace_count;  // its capacity in elements
};

#define WR_CHECK_LAUNCH()                                       \
  do {                                                          \
    if (hipGetLastError() != hipSuccess) return WR_EHIP;        \
  } while (0)

namespace wr {

constexpr int kWave = 64;

// Raise a kernel's dynamic LDS limit to `bytes` on the current device, once per (kernel, device,
// size); thread-safe.  Returns false if the runtime refuses.
inline bool lds_limit(const void* kernel, int bytes) {
  static std::mutex mu;
  static std::set<std::pair<std::pair<const void*, int>, int>> done;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  std::lock_guard<std::mutex> lock(mu);
  const auto key = std::make_pair(std::make_pair(kernel, dev), bytes);
  if (done.count(key)) return true;
  if (hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes) != hipSuccess) return false;
  done.insert(key);
  return true;
}

// ---------------------------------------------------------------- conversions
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// IEEE round-to-nearest-even fp32 -> bf16 bit pattern (NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float f16_bits_to_f32(uint16_t h) {
  _Float16 v = __builtin_bit_cast(_Float16, h);
  return (float)v;
}

// fp32 -> fp16 round-to-nearest-even, clamped to the finite range +-65504.
__device__ __forceinline__ uint16_t f32_to_f16_bits_clamped(float f) {
  f = fminf(fmaxf(f, -65504.0f), 65504.0f);
  _Float16 v = (_Float16)f;
  return __builtin_bit_cast(uint16_t, v);
}

// fp64 -> fp16 round-to-nearest-even with a single rounding, clamped to +-65504.
// The fp16 quantum q of |d| is a power of two; |d|/q is exact and rint() rounds it
// to nearest even, so r = rint(|d|/q) q is the correctly rounded value.
__device__ __forceinline__ uint16_t f64_to_f16_bits_clamped(double d) {
  if (d != d) return 0x7e00u;
  double a = fabs(d);
  uint16_t sign = d < 0.0 ? 0x8000u : 0u;
  if (a >= 65504.0) return sign | 0x7bffu;
  int e = ilogb(a);                       // a in [2^e, 2^(e+1))
  if (a == 0.0 || e < -14) e = -14;       // subnormal range shares the quantum 2^-24
  double q = ldexp(1.0, e - 10);
  double r = rint(a / q) * q;             // exact in fp16 (possibly the next binade)
  if (r > 65504.0) r = 65504.0;
  _Float16 v = (_Float16)(float)r;        // exact conversion
  return sign | __builtin_bit_cast(uint16_t, v);
}

// fp64 -> bf16 round-to-nearest-even with a single rounding (normal range: |d| in [2^-126, 2^128)).
// The bf16 quantum q of |d| is a power of two, |d|/q is exact and rint() rounds it to nearest even.
__device__ __forceinline__ uint32_t f64_to_bf16_bits(double d) {
  if (d != d) return 0x7fc0u;
  const uint32_t sign = d < 0.0 || (d == 0.0 && signbit(d)) ? 0x8000u : 0u;
  const double a = fabs(d);
  if (a == 0.0) return sign;
  const double q = ldexp(1.0, ilogb(a) - 7);
  const float r = (float)(rint(a / q) * q);  // exact: 8 significant bits
  return sign | (__float_as_uint(r) >> 16);
}

// x = x0 + x1 + x2 with each part rounded to bf16 in turn (exact for any fp32 x whose
// parts stay in the normal range): 24 significant bits as three bf16 matrix-core operands.
__device__ __forceinline__ void split3(float x, uint16_t& p0, uint16_t& p1, uint16_t& p2) {
  const uint32_t a = f32_to_bf16_bits(x);
  const float r1 = x - bf16_bits_to_f32(a);
  const uint32_t b = f32_to_bf16_bits(r1);
  const float r2 = r1 - bf16_bits_to_f32(b);
  p0 = (uint16_t)a;
  p1 = (uint16_t)b;
  p2 = (uint16_t)f32_to_bf16_bits(r2);
}

// ---------------------------------------------------------------- grid
// Nearest code for t in level units: clamp(floor((t + L)/2 + 1/2), 0, L).
__device__ __forceinline__ int nearest_code(float t, int L) {
  float c = floorf(fmaf(t, 0.5f, 0.5f * (float)(L + 1)));
  c = fminf(fmaxf(c, 0.0f), (float)L);
  return (int)c;
}

// ---------------------------------------------------------------- unrolling
// f(integral_constant<int, I>) for I = B .. E-1, each with I a compile-time constant
// (for lane indices of DPP and readlane that must be immediates).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// ---------------------------------------------------------------- MFMA
__device__ __forceinline__ f32x16 mfma32x32x16_bf16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32x32x2_f32(float a, float b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}
// Accumulator register v of lane l of a 32x32 MFMA block holds row acc_row(v, l), column l % 32.
__device__ __forceinline__ int acc_row(int v, int lane) { return 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3); }

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& u) { return __builtin_bit_cast(bf16x8, u); }

// Lower-triangle tile t -> (I, J), J <= I, row-major over the block triangle.
__device__ __forceinline__ void tri_tile(int t, int& I, int& J) {
  int i = (int)((sqrtf(8.0f * (float)t + 1.0f) - 1.0f) * 0.5f);
  while (i * (i + 1) / 2 > t) --i;
  while ((i + 1) * (i + 2) / 2 <= t) ++i;
  I = i;
  J = t - i * (i + 1) / 2;
}

// Tile t (0 <= t < nt (nt + 1) / 2) of the lower triangle of nt x nt tiles, in blocked order: bands of
// BH tile rows, each band in chunks of CW tile columns (BH * CW tiles that read the operand rows of
// only BH + CW tile rows and columns), row-major inside a chunk; the columns a band has past its last
// full chunk, and a last band of fewer than BH rows, row-major.  Tile 0 is (0, 0).
template <int BH, int CW>
__device__ __forceinline__ void blocked_tile(int t, int nt, int& I, int& J) {
  auto before = [](int b) { return BH * b * (BH * b + 1) / 2; };  // tiles in bands 0 .. b-1
  int b = (int)((sqrtf(2.0f * (float)t + 0.25f) - 0.5f) * (1.0f / BH));
  while (b > 0 && before(b) > t) --b;
  while (before(b + 1) <= t) ++b;
  int r = t - before(b);
  int c0 = 0;
  if (BH * b + BH <= nt) {
    const int nfull = BH * b >= CW - 1 ? (BH * b - (CW - 1)) / CW + 1 : 0;  // chunks on or below the diagonal
    if (r < BH * CW * nfull) {
      I = BH * b + (r % (BH * CW)) / CW;
      J = CW * (r / (BH * CW)) + r % CW;
      return;
    }
    r -= BH * CW * nfull;
    c0 = CW * nfull;
  }
  for (int i = BH * b;; ++i) {
    const int cnt = i + 1 - c0;
    if (r < cnt) {
      I = i;
      J = c0 + r;
      return;
    }
    r -= cnt;
  }
}

}  // namespace wr
