// C ABI entry points: argument checks on the host, then launches on the context's stream.
#include <new>

#include "common.hpp"

size_t wr_hessian_ws_bytes(int64_t rows, int64_t n, int x_dtype, int num_cu);
size_t wr_gptq_ws_bytes(int64_t rows, int64_t n);
size_t wr_wring_ws_bytes(int64_t rows, int64_t n, int32_t group, int32_t rank);
size_t wr_wring_gptq_ws_bytes(int64_t rows, int64_t n, int32_t group, int32_t rank);
int wr_hessian_accumulate_impl(wr_ctx*, const void*, int, int64_t, int64_t, int64_t, double*, int);
int wr_hessian_accumulate_static_impl(wr_ctx*, const void*, int, int64_t, int64_t, int64_t, double*, int);
int wr_static_scratch_init(int device);
int wr_hessian_finalize_impl(wr_ctx*, const double*, int64_t, int64_t, float, int64_t, float*, int64_t, float*, int32_t,
                             const int8_t*);
size_t wr_finalize_ws_bytes(int64_t n_store);
int wr_hadamard_rotate_impl(wr_ctx*, float*, int64_t, int64_t, int64_t, int32_t, const int8_t*, int);
int wr_gptq_sweep_impl(wr_ctx*, const void*, int, int64_t, int64_t, int64_t, const float*, int64_t, const uint8_t*,
                       int32_t, int32_t, uint8_t*, uint16_t*, int32_t*);
int wr_wring_solve_impl(wr_ctx*, const void*, int, int64_t, const void*, const void*, int32_t, float, int, const float*,
                        int64_t, int64_t, int64_t, const uint8_t*, int32_t, float, int, uint8_t*, uint16_t*, int32_t*);
int wr_pack_impl(wr_ctx*, const uint8_t*, const uint16_t*, int64_t, int64_t, int32_t, int32_t, uint8_t*);
int wr_unpack_impl(wr_ctx*, const uint8_t*, int64_t, int64_t, int32_t, int32_t, uint8_t*, uint16_t*, uint16_t*);
size_t wr_trellis_ws_bytes(int64_t rows, int64_t n, int32_t states);
size_t wr_gemv_ws_bytes(int64_t n_store, int32_t batch);
size_t wr_stats_ws_bytes(int64_t rows);
int wr_quant_stats_impl(wr_ctx*, const float*, int64_t, const uint8_t*, const uint16_t*, const uint8_t*, int64_t,
                        int64_t, int32_t, const uint8_t*, const float*, double*);
int wr_wring_target_impl(wr_ctx*, const void*, int, int64_t, const void*, const void*, int32_t, float, int, int64_t,
                         int64_t, const uint8_t*, int32_t, const uint8_t*, const uint16_t*, float*, int32_t*);
int wr_packed_gemv_impl(wr_ctx*, const uint8_t*, int64_t, int64_t, int32_t, int32_t, int32_t, const int8_t*, const float*,
                        int64_t, int64_t, int32_t, float*, int64_t);
int wr_trellis_quantize_impl(wr_ctx*, const float*, int64_t, int64_t, int64_t, int32_t, int32_t, const float*, int32_t,
                             uint8_t*, int64_t, float*, int64_t, double*);
int wr_materialize_impl(wr_ctx*, const uint8_t*, int64_t, int64_t, int32_t, int32_t, int32_t, const int8_t*, int64_t,
                        uint16_t*, int64_t);

namespace {

constexpr int kDefaultCUs = 256;

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
bool valid_dtype(int d) { return d == WR_F32 || d == WR_BF16; }
bool pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }
size_t dsize(int d) { return d == WR_F32 ? 4 : 2; }

// Guard: make the context's device current for the duration of a call.
struct DeviceScope {
  int prev = -1;
  bool ok = true;
  explicit DeviceScope(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    if (prev != dev) ok = hipSetDevice(dev) == hipSuccess;
  }
  ~DeviceScope() {
    if (prev >= 0) (void)hipSetDevice(prev);
  }
};

}  // namespace

extern "C" {

int wr_create(wr_ctx** out, int device, void* hip_stream) {
  if (!out) return WR_EINVAL;
  *out = nullptr;
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess) return WR_EHIP;
  if (device < 0 || device >= count) return WR_EINVAL;
  int cus = kDefaultCUs;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess) return WR_EHIP;
  wr_ctx* c = new (std::nothrow) wr_ctx;
  if (!c) return WR_EHIP;
  c->device = device;
  c->stream = static_cast<hipStream_t>(hip_stream);
  c->ws = nullptr;
  c->ws_bytes = 0;
  c->num_cu = cus > 0 ? cus : kDefaultCUs;
  c->scale_trace = nullptr;
  c->scale_trace_count = 0;
  // device address of the allocation-free entry point's static scratch, once per device (a
  // failure here is reported by that entry point, which tries again)
  (void)wr_static_scratch_init(device);
  *out = c;
  return WR_OK;
}

int wr_destroy(wr_ctx* ctx) {
  if (!ctx) return WR_EINVAL;
  delete ctx;
  return WR_OK;
}

size_t wr_workspace_bytes(int op, int64_t rows, int64_t n, int32_t group, int32_t rank, int32_t lazy_batch) {
  (void)lazy_batch;
  if (rows < 0 || n <= 0) return 0;
  switch (op) {
    case WR_OP_HESSIAN: {
      // the larger of the bf16 and fp32 input paths
      const size_t a = wr_hessian_ws_bytes(rows, n, WR_BF16, kDefaultCUs);
      const size_t b = wr_hessian_ws_bytes(rows, n, WR_F32, kDefaultCUs);
      return a > b ? a : b;
    }
    case WR_OP_GPTQ: return wr_gptq_ws_bytes(rows, n);
    case WR_OP_FINALIZE: return wr_finalize_ws_bytes(n);
    case WR_OP_WRING: return group > 0 ? wr_wring_ws_bytes(rows, n, group, rank > 0 ? rank : 0) : 0;
    case WR_OP_WRING_GPTQ: return group > 0 ? wr_wring_gptq_ws_bytes(rows, n, group, rank > 0 ? rank : 0) : 0;
    case WR_OP_TRELLIS: return group >= 2 && group <= 16 ? wr_trellis_ws_bytes(rows, n, group) : 0;
    case WR_OP_GEMV: return rows >= 1 && rows <= 8 ? wr_gemv_ws_bytes(n, (int32_t)rows) : 0;
    case WR_OP_STATS: return wr_stats_ws_bytes(rows > 0 ? rows : 1);
    default: return 0;
  }
}

int wr_set_workspace(wr_ctx* ctx, void* dev_ptr, size_t bytes) {
  if (!ctx || (bytes > 0 && !dev_ptr) || (dev_ptr && !aligned(dev_ptr, 256))) return WR_EINVAL;
  ctx->ws = dev_ptr;
  ctx->ws_bytes = dev_ptr ? bytes : 0;
  return WR_OK;
}

int wr_hessian_accumulate(wr_ctx* ctx, const void* X, int x_dtype, int64_t rows, int64_t n, int64_t ldx, double* S,
                          int flags) {
  if (!ctx || !S || !valid_dtype(x_dtype) || rows < 0 || n <= 0 || n > 65536 || ldx < n || (flags & ~WR_H_ZERO))
    return WR_EINVAL;
  if (rows > 0 && !X) return WR_EINVAL;
  if (n % 8 != 0) return WR_EINVAL;
  if (rows > 0 && x_dtype == WR_BF16 && (ldx % 8 != 0 || !aligned(X, 16))) return WR_EINVAL;
  if (rows > 65535 * 4096) return WR_EINVAL;
  if (ldx > ((int64_t)1 << 24)) return WR_EUNSUPPORTED;
  if (!aligned(S, 8)) return WR_EINVAL;
  DeviceScope ds(ctx->device);
  if (!ds.ok) return WR_EHIP;
  return wr_hessian_accumulate_impl(ctx, X, x_dtype, rows, n, ldx, S, flags);
}

int wr_hessian_accumulate_noalloc(wr_ctx* ctx, const void* X, int x_dtype, int64_t rows, int64_t n, int64_t ldx,
                                  double* S, int flags) {
  if (!ctx || !S || !valid_dtype(x_dtype) || rows < 0 || n <= 0 || n > 65536 || ldx < n || (flags & ~WR_H_ZERO))
    return WR_EINVAL;
  if (rows > 0 && !X) return WR_EINVAL;
  if (n % 8 != 0) return WR_EINVAL;
  if (rows > 0 && x_dtype == WR_BF16 && (ldx % 8 != 0 || !aligned(X, 16))) return WR_EINVAL;
  if (rows > 65535 * 4096) return WR_EINVAL;
  if (ldx > ((int64_t)1 << 24)) return WR_EUNSUPPORTED;
  if (!aligned(S, 8)) return WR_EINVAL;
  DeviceScope ds(ctx->device);
  if (!ds.ok) return WR_EHIP;
  if (wr_static_scratch_init(ctx->device) != WR_OK) return WR_EHIP;
  return wr_hessian_accumulate_static_impl(ctx, X, x_dtype, rows, n, ldx, S, flags);
}

int wr_hessian_finalize(wr_ctx* ctx, const double* S, int64_t n, int64_t total_rows, float damp_frac, int64_t n_store,
                        float* H, int64_t ldh, float* delta_out, int32_t had_block, const int8_t* signs) {
  if (!ctx || !S || !H || n <= 0 || n > 65536 || total_rows <= 0 || n_store < n || n_store > 65535 || ldh < n_store ||
      !(damp_frac >= 0.0f))
    return WR_EINVAL;
  if (had_block != 0 && (!signs || !pow2(had_block) || had_block < 2 || had_block > 4096 || n_store % had_block != 0))
    return WR_EINVAL;
  DeviceScope ds(ctx->device);
  if (!ds.ok) return WR_EHIP;
  return wr_hessian_finalize_impl(ctx, S, n, total_rows, damp_frac, n_store, H, ldh, delta_out, had_block, signs);
}

int wr_hadamard_rotate(wr_ctx* ctx, float* M, int64_t rows, int64_t n, int64_t ld, int32_t had_block,
                       const int8_t* signs, int mode) {
  if (!ctx || !M || !signs || rows < 0 || n <= 0 || ld < n || !pow2(had_block) || had_block < 2 || had_block > 4096 ||
      n % had_block != 0)
    return WR_EINVAL;
  if (mode != WR_ROT_ROWS && mode != WR_ROT_ROWS_INVERSE && mode != WR_ROT_SYM) return WR_EINVAL;
  if (mode == WR_ROT_SYM && rows != n) return WR_EINVAL;
  if (rows > 65535 || n / had_block > 65535) return WR_EINVAL;
  if (rows == 0) return WR_OK;
  DeviceScope ds(ctx->device);
  if (!ds.ok) return WR_EHIP;
  return wr_hadamard_rotate_impl(ctx, M, rows, n, ld, had_block, signs, mode);
}

int wr_gptq_sweep(wr_ctx* ctx, const void* W, int w_dtype, int64_t rows, int64_t n, int64_t ldw, const float* H,
                  int64_t ldh, const uint8_t* bits, int32_t group, int32_t lazy_batch, uint8_t* codes,
                  uint16_t* scales, int32_t* dev_info) {
  if (!ctx || !H || !dev_info || !valid_dtype(w_dtype) || rows < 0 || n <= 0 || n > 65536 || ldh < n || group <= 0 ||
      n % group != 0 || group % 8 != 0 || lazy_batch < group || lazy_batch % group != 0 || n % 4 != 0)
    return WR_EINVAL;
  if (rows > 0 && (!W || !bits || !codes || !scales || ldw < n)) return WR_EINVAL;
  if (rows > 2147483647 / 4) return WR_EINVAL;
  if (!aligned(H, 16) || ldh % 4 != 0) return WR_EINVAL;
  DeviceScope ds(ctx->device);
  if (!ds.ok) return WR_EHIP;
  return wr_gptq_sweep_impl(ctx, W, w_dtype, rows, n, ldw, H, ldh, bits, group, lazy_batch, codes, scales, dev_info);
}

int wr_wring_solve(wr_ctx* ctx, const void* target, int t_dtype, int64_t ldt, const void* B, const void* A,
                   int32_t rank, float alpha, int ab_dtype, const float* H, int64_t ldh, int64_t rows, int64_t n,
                   const uint8_t* bits, int32_t group, float lambda, int flags, uint8_t* codes, uint16_t* scales,
                   int32_t* dev_info) {
  const int mode = flags & (WR_RECODE_NEAREST | WR_RECODE_GPTQ | WR_RECODE_SEARCH);
  const bool search = flags == WR_RECODE_SEARCH;  // H and lambda unused
  if (!ctx || !dev_info || rows < 0 || n <= 0 || n > 65536 || group <= 0 || n % group != 0 || group % 8 != 0 ||
      (flags & ~(WR_RECODE_NEAREST | WR_RECODE_GPTQ | WR_RECODE_SEARCH)) || (mode & (mode - 1)) != 0)
    return WR_EINVAL;
  if (!search && (!H || ldh < n || !(lambda >= 0.0f))) return WR_EINVAL;
  if ((flags & WR_RECODE_GPTQ) && n % 4 != 0) return WR_EINVAL;
  if (rows > 65535) return WR_EINVAL;
  if (target && (!valid_dtype(t_dtype) || ldt < n)) return WR_EINVAL;
  if ((B != nullptr) != (A != nullptr)) return WR_EINVAL;
  if (B && (rank <= 0 || rank % 4 != 0 || !valid_dtype(ab_dtype))) return WR_EINVAL;
  if (rows > 0 && (!bits || !codes || !scales)) return WR_EINVAL;
  if ((!search && (!aligned(H, 16) || ldh % 4 != 0)) || !aligned(codes, 16)) return WR_EINVAL;
  DeviceScope ds(ctx->device);
  if (!ds.ok) return WR_EHIP;
  return wr_wring_solve_impl(ctx, target, t_dtype, ldt, B, A, rank, alpha, ab_dtype, H, ldh, rows, n, bits, group,
                             lambda, flags, codes, scales, dev_info);
}

int wr_pack(wr_ctx* ctx, const uint8_t* codes, const uint16_t* scales, int64_t rows, int64_t n, int32_t bits,
            int32_t group, uint8_t* out, size_t out_bytes) {
  if (!ctx || rows < 0 || n <= 0 || bits < 2 || bits > 4 || group <= 0 || n % group != 0 || n % 8 != 0) return WR_EINVAL;
  if (rows > 0 && (!codes || !scales || !out || !aligned(codes, 8))) return WR_EINVAL;
  const size_t need = (size_t)rows * n * bits / 8 + 2 * (size_t)rows * (n / group);
  if (out_bytes != need) return WR_EINVAL;
  DeviceScope ds(ctx->device);
  if (!ds.ok) return WR_EHIP;
  return wr_pack_impl(ctx, codes, scales, rows, n, bits, group, out);
}

int wr_unpack(wr_ctx* ctx, const uint8_t* in, size_t in_bytes, int64_t rows, int64_t n, int32_t bits, int32_t group,
              uint8_t* codes, uint16_t* scales, uint16_t* dequant_bf16) {
  if (!ctx || rows < 0 || n <= 0 || bits < 2 || bits > 4 || group <= 0 || n % group != 0 || n % 8 != 0) return WR_EINVAL;
  if (rows > 0 && !in) return WR_EINVAL;
  const size_t need = (size_t)rows * n * bits / 8 + 2 * (size_t)rows * (n / group);
  if (in_bytes != need) return WR_EINVAL;
  DeviceScope ds(ctx->device);
  if (!ds.ok) return WR_EHIP;
  return wr_unpack_impl(ctx, in, rows, n, bits, group, codes, scales, dequant_bf16);
}

int wr_materialize(wr_ctx* ctx, const uint8_t* in, size_t in_bytes, int64_t rows, int64_t n_store, int32_t bits,
                   int32_t group, int32_t had_block, const int8_t* signs, int64_t n_out, uint16_t* out, int64_t ldo) {
  if (!ctx || rows < 0 || n_store <= 0 || n_store > (1 << 24) || bits < 2 || bits > 4 || group <= 0 ||
      n_store % group != 0 || n_store % 8 != 0 || n_out <= 0 || n_out > n_store || ldo < n_out)
    return WR_EINVAL;
  if (rows > 65535) return WR_EINVAL;
  if (had_block != 0 && (!signs || !pow2(had_block) || had_block < 2 || had_block > 4096 || n_store % had_block != 0))
    return WR_EINVAL;
  if (rows > 0 && (!in || !out)) return WR_EINVAL;
  const size_t need = (size_t)rows * n_store * bits / 8 + 2 * (size_t)rows * (n_store / group);
  if (in_bytes != need) return WR_EINVAL;
  DeviceScope ds(ctx->device);
  if (!ds.ok) return WR_EHIP;
  return wr_materialize_impl(ctx, in, rows, n_store, bits, group, had_block, signs, n_out, out, ldo);
}

int wr_trellis_quantize(wr_ctx* ctx, const float* T, int64_t ldt, int64_t rows, int64_t n, int32_t log2_states,
                        int32_t coset_size, const float* values, int32_t start_state, uint8_t* codes, int64_t ldc,
                        float* recon, int64_t ldr, double* cost) {
  if (!ctx || rows < 0 || n <= 0 || n > (1 << 24) || log2_states < 1 || log2_states > 4 ||
      !(coset_size == 1 || coset_size == 2 || coset_size == 4) || start_state < 0 || start_state >= (1 << log2_states))
    return WR_EINVAL;
  if (rows > 0 && (!T || !values || !codes || ldt < n || ldt % 4 != 0 || !aligned(T, 16) || ldc < n ||
                   (recon && ldr < n)))
    return WR_EINVAL;
  if (rows > ((int64_t)1 << 31) / 16) return WR_EINVAL;
  DeviceScope ds(ctx->device);
  if (!ds.ok) return WR_EHIP;
  return wr_trellis_quantize_impl(ctx, T, ldt, rows, n, log2_states, coset_size, values, start_state, codes, ldc, recon,
                                  ldr, cost);
}

int wr_packed_gemv(wr_ctx* ctx, const uint8_t* in, size_t in_bytes, int64_t rows, int64_t n_store, int32_t bits,
                   int32_t group, int32_t had_block, const int8_t* signs, const float* x, int64_t n_in, int64_t ldx,
                   int32_t batch, float* y, int64_t ldy) {
  if (!ctx || rows < 0 || n_store <= 0 || n_store > (1 << 24) || n_store % 32 != 0 || bits < 2 || bits > 4 ||
      group <= 0 || group % 32 != 0 || n_store % group != 0 || batch < 1 || batch > 8 || n_in <= 0 || n_in > n_store ||
      ldx < n_in || !x || !y || ldy < rows)
    return WR_EINVAL;
  if (rows > 2147483647 / 16) return WR_EINVAL;
  if (had_block != 0 && (!signs || !pow2(had_block) || had_block < 2 || had_block > 4096 || n_store % had_block != 0))
    return WR_EINVAL;
  if (rows > 0 && (!in || !aligned(in, 16))) return WR_EINVAL;
  const size_t need = (size_t)rows * n_store * bits / 8 + 2 * (size_t)rows * (n_store / group);
  if (in_bytes != need) return WR_EINVAL;
  DeviceScope ds(ctx->device);
  if (!ds.ok) return WR_EHIP;
  return wr_packed_gemv_impl(ctx, in, rows, n_store, bits, group, had_block, signs, x, n_in, ldx, batch, y, ldy);
}

int wr_set_scale_trace(wr_ctx* ctx, float* raw, int64_t capacity) {
  if (!ctx || (raw && capacity <= 0) || (raw && !aligned(raw, 4))) return WR_EINVAL;
  ctx->scale_trace = raw;
  ctx->scale_trace_count = raw ? capacity : 0;
  return WR_OK;
}

int wr_wring_target(wr_ctx* ctx, const void* target, int t_dtype, int64_t ldt, const void* B, const void* A,
                    int32_t rank, float alpha, int ab_dtype, int64_t rows, int64_t n, const uint8_t* bits,
                    int32_t group, const uint8_t* codes, const uint16_t* scales, float* T_out, int32_t* dev_info) {
  if (!ctx || !dev_info || rows < 0 || rows > 65535 || n <= 0 || n > 65536 || group <= 0 || n % group != 0 ||
      group % 8 != 0)
    return WR_EINVAL;
  if (target && (!valid_dtype(t_dtype) || ldt < n)) return WR_EINVAL;
  if ((B != nullptr) != (A != nullptr)) return WR_EINVAL;
  if (B && (rank <= 0 || rank % 4 != 0 || !valid_dtype(ab_dtype))) return WR_EINVAL;
  if (rows > 0 && (!bits || !T_out || (!target && (!codes || !scales)))) return WR_EINVAL;
  if (codes && !aligned(codes, 16)) return WR_EINVAL;
  DeviceScope ds(ctx->device);
  if (!ds.ok) return WR_EHIP;
  return wr_wring_target_impl(ctx, target, t_dtype, ldt, B, A, rank, alpha, ab_dtype, rows, n, bits, group, codes,
                              scales, T_out, dev_info);
}

int wr_quant_stats(wr_ctx* ctx, const float* T, int64_t ldt, const uint8_t* codes, const uint16_t* scales,
                   const uint8_t* bits, int64_t rows, int64_t n, int32_t group, const uint8_t* codes_ref,
                   const float* scales_raw, double* out) {
  if (!ctx || !out || rows < 0 || rows > 2147483647 || n <= 0 || n > 65536 || group <= 0 || n % group != 0)
    return WR_EINVAL;
  if (rows > 0 && (!codes || !scales || !bits || (T && ldt < n))) return WR_EINVAL;
  DeviceScope ds(ctx->device);
  if (!ds.ok) return WR_EHIP;
  return wr_quant_stats_impl(ctx, T, ldt, codes, scales, bits, rows, n, group, codes_ref, scales_raw, out);
}

const char* wr_strerror(int status) {
  switch (status) {
    case WR_OK: return "success";
    case WR_EINVAL: return "invalid argument";
    case WR_EWORKSPACE: return "workspace missing or too small";
    case WR_EHIP: return "HIP runtime error";
    case WR_EUNSUPPORTED: return "unsupported configuration";
    case WR_ESCRATCH: return "request exceeds the static scratch of the allocation-free entry point";
    default: return "unknown status";
  }
}

}  // extern "C"
