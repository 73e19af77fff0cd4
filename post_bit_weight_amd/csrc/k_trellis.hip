// Trellis-coded quantization with a Viterbi search (Pingala-8 post, "Trick 3: trellis coding"):
// the state carried from one step to the next picks the coset of values the step may use; the
// bits written pick the value and the next state; the Viterbi algorithm keeps, for every
// state, the cheapest path ending there.  Scalar steps on a shift-register trellis of S = 2^m
// states: branch bit u leads from s to ((s << 1) | u) mod S, so the predecessors of s are
// s >> 1 and (s >> 1) + S/2 with branch bit s & 1; branch (p, u) carries a coset of C values,
// of which the nearest is taken.
//
// Layout of the work: S consecutive lanes per row, lane s holding the cost of the cheapest path
// that ends in state s.  A step computes the two branch metrics into s (the coset values of
// both incoming branches sit in the lane's registers), reads the two predecessors' costs across
// lanes and keeps the cheaper (the smaller predecessor on a tie); the decision bit goes into a
// word written every 32 steps to a step-major workspace (coalesced).  Costs are renormalised by
// the row's minimum every 16 steps, so fp32 keeps the differences that decide the path.  The
// traceback is a second kernel.
#include "common.hpp"

namespace wr {

typedef float f32x2 __attribute__((ext_vector_type(2)));

// Cost of the predecessor p0 = s >> 1 (J = 0) or p1 = p0 + S/2 (J = 1) of this lane's state:
// quad_perm patterns for S = 2 ([0,0,2,2], [1,1,3,3]) and S = 4 ([0,0,1,1], [2,2,3,3]), a lane
// permute for larger S.
template <int S, int J>
__device__ __forceinline__ float pred_cost(float x, int src_lane) {
  const int i = __float_as_int(x);
  if constexpr (S == 2) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(i, J ? 0xF5 : 0xA0, 0xF, 0xF, true));
  } else if constexpr (S == 4) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(i, J ? 0xFA : 0x50, 0xF, 0xF, true));
  } else {
    return __shfl(x, src_lane);
  }
}

// the 32 targets of chunk ch of a row (zeros past n)
__device__ __forceinline__ void load_chunk(const float* __restrict__ t, int ch, int n, float (&x)[32]) {
  const int k0 = ch * 32;
  if (k0 + 32 <= n) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(t + k0 + 4 * q);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[4 * q + e] = v[e];
    }
  } else {
#pragma unroll
    for (int j = 0; j < 32; ++j) x[j] = k0 + j < n ? t[k0 + j] : 0.0f;
  }
}

// the 32 targets of chunk ch of a row, which lies wholly before n
__device__ __forceinline__ void load_full(const float* __restrict__ t, int ch, float (&x)[32]) {
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(t + ch * 32 + 4 * q);
#pragma unroll
    for (int e = 0; e < 4; ++e) x[4 * q + e] = v[e];
  }
}

using full_chunk = std::integral_constant<bool, true>;
using tail_chunk = std::integral_constant<bool, false>;

template <int LOGS, int C>
__global__ __launch_bounds__(256) void trellis_viterbi_kernel(const float* __restrict__ T, int64_t ldt, int64_t rows,
                                                              int n, const float* __restrict__ values, int start,
                                                              uint32_t* __restrict__ bp, int32_t* __restrict__ end_state) {
  constexpr int S = 1 << LOGS;
  __shared__ float tab[S * 2 * C];
  for (int i = threadIdx.x; i < S * 2 * C; i += blockDim.x) tab[i] = values[i];
  __syncthreads();
  const int s = threadIdx.x & (S - 1);
  const int gbase = (threadIdx.x & 63) & ~(S - 1);
  const int64_t row0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> LOGS;
  const bool live = row0 < rows;
  const int64_t row = live ? row0 : rows - 1;  // every lane takes part in the exchanges
  const float* t = T + row * ldt;
  const int p0 = s >> 1, p1 = p0 + S / 2, u = s & 1;
  const int lane0 = gbase + p0, lane1 = gbase + p1;
  float v0[C], v1[C];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    v0[c] = tab[(p0 * 2 + u) * C + c];
    v1[c] = tab[(p1 * 2 + u) * C + c];
  }
  const int64_t stride = rows * S;  // words per 32-step chunk
  const int nchunk = (n + 31) >> 5;
  float cost = s == start ? 0.0f : INFINITY;
  float xs[32], nx[32];
  load_chunk(t, 0, n, xs);
  // the first chunk has arrived before the loop: otherwise the compiler, which cannot tell the
  // first iteration's registers from later ones, waits inside every chunk for the next
  // chunk's loads that were just issued
  __builtin_amdgcn_s_waitcnt(0);
  for (int ch = 0; ch < nchunk; ++ch) {
    if (ch + 1 < nchunk) load_chunk(t, ch + 1, n, nx);
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      if (ch * 32 + j < n) {
        const float x = xs[j];
        float b0 = INFINITY, b1 = INFINITY;
#pragma unroll
        for (int c = 0; c < C; ++c) {
          const float d0 = x - v0[c], d1 = x - v1[c];
          b0 = fminf(b0, d0 * d0);
          b1 = fminf(b1, d1 * d1);
        }
        const float c0 = pred_cost<S, 0>(cost, lane0) + b0;
        const float c1 = pred_cost<S, 1>(cost, lane1) + b1;
        const bool up = c1 < c0;  // a tie keeps the smaller predecessor
        cost = up ? c1 : c0;
        word |= (uint32_t)up << j;
        if ((j & 15) == 15) {
          float m = cost;
#pragma unroll
          for (int o = 1; o < S; o <<= 1) m = fminf(m, __shfl_xor(m, o));
          cost -= m;
        }
      }
    }
    if (live) bp[(int64_t)ch * stride + row * S + s] = word;
#pragma unroll
    for (int j = 0; j < 32; ++j) xs[j] = nx[j];
  }
  // cheapest end state (the smaller state on a tie)
  float bc = cost;
  int bs = s;
#pragma unroll
  for (int o = 1; o < S; o <<= 1) {
    const float oc = __shfl_xor(bc, o);
    const int os = __shfl_xor(bs, o);
    if (oc < bc || (oc == bc && os < bs)) {
      bc = oc;
      bs = os;
    }
  }
  if (live && s == 0) end_state[row] = bs;
}

// Traceback, one lane per row: from the cheapest end state back through the decision words
// (the S words of a 32-step chunk read together, the next chunk's words and targets requested
// before the current chunk is walked); writes codes u | v << 1, the decoded values and the
// path's fp64 cost.
template <int LOGS, int C>
__global__ __launch_bounds__(256) void trellis_traceback_kernel(const float* __restrict__ T, int64_t ldt, int64_t rows,
                                                                int n, const float* __restrict__ values,
                                                                const uint32_t* __restrict__ bp,
                                                                const int32_t* __restrict__ end_state,
                                                                uint8_t* __restrict__ codes, int64_t ldc,
                                                                float* __restrict__ recon, int64_t ldr,
                                                                double* __restrict__ cost_out) {
  constexpr int S = 1 << LOGS;
  __shared__ float tab[S * 2 * C];
  for (int i = threadIdx.x; i < S * 2 * C; i += blockDim.x) tab[i] = values[i];
  __syncthreads();
  const int64_t row = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (row >= rows) return;
  const float* t = T + row * ldt;
  const int64_t stride = rows * S;
  const int nchunk = (n + 31) >> 5;
  float xs[32], nx[32];
  int cur = end_state[row];
  double acc = 0.0;
  // codes and values of a 16-step block collect in registers and go out in one 16-byte (or four)
  // stores when the block is whole and the rows aligned
  const bool vec = ldc % 16 == 0 && (reinterpret_cast<uintptr_t>(codes) & 15) == 0 &&
                   (!recon || (ldr % 4 == 0 && (reinterpret_cast<uintptr_t>(recon) & 15) == 0));
  uint32_t cw[4] = {0u, 0u, 0u, 0u};
  float rv[16];
  uint32_t w[S], nw[S];
  const uint32_t* src = bp + (int64_t)(nchunk - 1) * stride + row * S;
#pragma unroll
  for (int j = 0; j < S; ++j) w[j] = src[j];
  load_chunk(t, nchunk - 1, n, xs);
  for (int ch = nchunk - 1; ch >= 0; --ch) {
    if (ch > 0) {
      const uint32_t* ps = bp + (int64_t)(ch - 1) * stride + row * S;
#pragma unroll
      for (int j = 0; j < S; ++j) nw[j] = ps[j];
      load_chunk(t, ch - 1, n, nx);
    }
#pragma unroll
    for (int j = 31; j >= 0; --j) {
      const int k = ch * 32 + j;
      if (k < n) {
        uint32_t wd = w[0];
#pragma unroll
        for (int q = 1; q < S; ++q) wd = cur == q ? w[q] : wd;
        const int upb = (wd >> j) & 1;
        const int p = (cur >> 1) + upb * (S / 2);
        const int uu = cur & 1;
        const float x = xs[j];
        const float* cs = tab + (p * 2 + uu) * C;
        int vb = 0;
        float rb = cs[0];
        float db = (x - rb) * (x - rb);
#pragma unroll
        for (int c = 1; c < C; ++c) {
          const float val = cs[c];
          const float d = (x - val) * (x - val);
          if (d < db) {  // a tie keeps the smaller index
            db = d;
            rb = val;
            vb = c;
          }
        }
        const double dd = (double)x - (double)rb;
        acc = fma(dd, dd, acc);
        cw[(j >> 2) & 3] |= (uint32_t)(uu | (vb << 1)) << (8 * (j & 3));
        rv[j & 15] = rb;
        cur = p;
      }
      if ((j & 15) == 0) {  // the block of steps [k, k + 16) is done
        uint8_t* cd = codes + row * ldc + k;
        float* rd = recon ? recon + row * ldr + k : nullptr;
        if (vec && k + 16 <= n) {
          *reinterpret_cast<u32x4*>(cd) = u32x4{cw[0], cw[1], cw[2], cw[3]};
          if (rd) {
#pragma unroll
            for (int q = 0; q < 4; ++q)
              *reinterpret_cast<f32x4*>(rd + 4 * q) = f32x4{rv[4 * q], rv[4 * q + 1], rv[4 * q + 2], rv[4 * q + 3]};
          }
        } else {
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if (k + e < n) {
              cd[e] = (uint8_t)(cw[e >> 2] >> (8 * (e & 3)));
              if (rd) rd[e] = rv[e];
            }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) cw[q] = 0u;
      }
    }
    if (ch > 0) {
#pragma unroll
      for (int j = 0; j < S; ++j) w[j] = nw[j];
#pragma unroll
      for (int j = 0; j < 32; ++j) xs[j] = nx[j];
    }
  }
  if (cost_out) cost_out[row] = acc;
}

// Two steps per exchange (S >= 4).  After two steps state s'' = (4 p + 2 u1 + u2) mod S comes
// from one of four states two steps back, p_j = (s'' >> 2) + j S/4, through the middle state
// mid_a = s'' >> 1 (from p_0 or p_2) or mid_b = mid_a + S/2 (from p_1 or p_3).  Taking the
// cheaper of each pair (the smaller state on a tie), then the cheaper middle state (mid_a on a
// tie), with the costs added in the same order, is the one-step algorithm's decisions and
// fp32 rounding exactly, with one round of lane exchanges per two steps.  Decision: 2 bits per
// state and pair of steps (bit 0: mid_b taken; bit 1: the chosen middle state came from its
// larger predecessor).  An odd last step is paired with a step of zero cost.
template <int LOGS, int C>
__global__ __launch_bounds__(256, 4) void trellis_viterbi2_kernel(const float* __restrict__ T, int64_t ldt, int64_t rows,
                                                               int n, const float* __restrict__ values, int start,
                                                               uint32_t* __restrict__ bp, int32_t* __restrict__ end_state) {
  constexpr int S = 1 << LOGS;
  static_assert(S >= 4, "two steps per exchange need four predecessors");
  __shared__ float tab[S * 2 * C];
  // costs exchanged through LDS: state p of a row at slot (p mod S/4) * 4 + p / (S/4) of the
  // row's S slots, so that the four predecessors p_j = q + j S/4 of a state sit at slots
  // 4q .. 4q + 3 and one 16-byte read fetches them in order.  A row's lanes are in one wave,
  // whose LDS operations complete in order: no barrier between the write and the reads.
  __shared__ __align__(16) float xcost[256];
  for (int i = threadIdx.x; i < S * 2 * C; i += blockDim.x) tab[i] = values[i];
  __syncthreads();
  const int s = threadIdx.x & (S - 1);
  const int64_t row0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> LOGS;
  const bool live = row0 < rows;
  const int64_t row = live ? row0 : rows - 1;  // every lane takes part in the exchanges
  const float* t = T + row * ldt;
  const int q = s >> 2, u1 = (s >> 1) & 1, u2 = s & 1;
  const int ma = s >> 1, mb = ma + S / 2;
  float* const wslot = xcost + (threadIdx.x & ~(S - 1)) + (s % (S / 4)) * 4 + s / (S / 4);
  const f32x4* const rslot = reinterpret_cast<const f32x4*>(xcost + (threadIdx.x & ~(S - 1)) + 4 * q);
  float va[4][C], vma[C], vmb[C];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int pj = q + j * (S / 4);
#pragma unroll
    for (int c = 0; c < C; ++c) va[j][c] = tab[(pj * 2 + u1) * C + c];
  }
#pragma unroll
  for (int c = 0; c < C; ++c) {
    vma[c] = tab[(ma * 2 + u2) * C + c];
    vmb[c] = tab[(mb * 2 + u2) * C + c];
  }
  const int64_t stride = rows * S;  // words per 32-step chunk
  const int nfull = n >> 5;
  float cost = s == start ? 0.0f : INFINITY;
  float xs[32], nx[32];
  // When every branch into this lane's state two steps on carries the same coset at the first
  // step, and both middle states' branches the same coset at the second (as for a coset chosen
  // by the state's low bit and the branch bit, with 8 or more states), each metric is computed
  // once: the same numbers, fewer operations.  Decided per wave from the table, so uniformly.
  bool same = S >= 8;
#pragma unroll
  for (int c = 0; c < C; ++c) {
#pragma unroll
    for (int j = 1; j < 4; ++j) same = same && va[j][c] == va[0][c];
    same = same && vmb[c] == vma[c];
  }
  const bool shared = __all(same);
  // one chunk of 32 steps on the targets in xc (FULL: all of them before n; SHARED: the
  // metrics above are shared)
  auto chunk = [&](auto full, auto shared_tag, int ch, const float (&xc)[32]) __attribute__((always_inline)) {
    constexpr bool FULL = decltype(full)::value;
    constexpr bool SHARED = decltype(shared_tag)::value;
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int k = ch * 32 + 2 * i;
      if (FULL || k < n) {
        const float x1 = xc[2 * i], x2 = xc[2 * i + 1];
        *wslot = cost;
        __builtin_amdgcn_wave_barrier();
        const f32x4 pcv = *rslot;
        __builtin_amdgcn_wave_barrier();
        const float pc[4] = {pcv[0], pcv[1], pcv[2], pcv[3]};
        // the smallest squared distance to a coset is the square of the smallest distance
        // (squaring and its rounding are monotone): one min with |.| operands per value
        float b1[4];
#pragma unroll
        for (int j = 0; j < (SHARED ? 1 : 4); ++j) {
          float m = fabsf(x1 - va[j][0]);
#pragma unroll
          for (int c = 1; c < C; ++c) m = fminf(m, fabsf(x1 - va[j][c]));
          b1[j] = m * m;
        }
        if constexpr (SHARED) b1[1] = b1[2] = b1[3] = b1[0];
        const float ca0 = pc[0] + b1[0], ca1 = pc[2] + b1[2];
        const float cb0 = pc[1] + b1[1], cb1 = pc[3] + b1[3];
        const bool upa = ca1 < ca0, upb = cb1 < cb0;  // a tie keeps the smaller state
        const float cA = upa ? ca1 : ca0, cB = upb ? cb1 : cb0;
        float ba = 0.0f, bb = 0.0f;  // an odd last step is paired with a step of zero cost
        if (FULL || k + 1 < n) {
          float ma2 = fabsf(x2 - vma[0]);
#pragma unroll
          for (int c = 1; c < C; ++c) ma2 = fminf(ma2, fabsf(x2 - vma[c]));
          ba = ma2 * ma2;
          if constexpr (SHARED) {
            bb = ba;
          } else {
            float mb2 = fabsf(x2 - vmb[0]);
#pragma unroll
            for (int c = 1; c < C; ++c) mb2 = fminf(mb2, fabsf(x2 - vmb[c]));
            bb = mb2 * mb2;
          }
        }
        const float fa = cA + ba, fb = cB + bb;
        const bool up2 = fb < fa;
        cost = up2 ? fb : fa;
        const uint32_t da = upa ? 2u : 0u, db = upb ? 3u : 1u;
        word |= (up2 ? db : da) << (2 * i);
        if ((i & 7) == 7) {
          float m = cost;
#pragma unroll
          for (int o = 1; o < S; o <<= 1) m = fminf(m, __shfl_xor(m, o));
          cost -= m;
        }
      }
    }
    // transpose the row's S words so that the traceback finds a state's decision with one
    // bit-field read: split each word into S fields of E = 32/S bits (P = 16/S steps pairs each);
    // afterwards word j holds field j of every state, state r's at bits E r.  One exchange per
    // bit of the lane index swaps that bit between the lane and field indices.
    constexpr int E = 32 / S;
#pragma unroll
    for (int o = 1; o < S; o <<= 1) {
      uint32_t mo = 0u;
#pragma unroll
      for (int e = 0; e < S; ++e)
        if (e & o) mo |= ((1u << E) - 1u) << (E * e);
      const uint32_t other = (uint32_t)__shfl_xor((int)word, o);
      word = (s & o) ? (word & mo) | ((other >> (E * o)) & ~mo) : (word & ~mo) | ((other << (E * o)) & mo);
    }
    if (live) bp[(int64_t)ch * stride + row * S + s] = word;
  };
  // Whole chunks two per iteration, the buffers trading roles (no copies), each chunk's
  // targets loaded one chunk ahead.  The loop holds only unconditional vector loads (the
  // index clamped at the last whole chunk) and the first chunk has arrived before it: with a
  // conditional or ragged load in the loop the compiler's wait counts, merged over both paths,
  // would wait inside every chunk for the loads just issued.  The ragged last chunk follows.
  auto run = [&](auto shared_tag) __attribute__((always_inline)) {
    if (nfull > 0) load_full(t, 0, xs);
    __builtin_amdgcn_s_waitcnt(0);
    int ch = 0;
    for (; ch + 1 < nfull; ch += 2) {
      load_full(t, ch + 1, nx);
      __builtin_amdgcn_sched_barrier(0);  // keep the loads a whole chunk ahead of their use
      chunk(full_chunk{}, shared_tag, ch, xs);
      load_full(t, ch + 2 < nfull ? ch + 2 : ch + 1, xs);
      __builtin_amdgcn_sched_barrier(0);
      chunk(full_chunk{}, shared_tag, ch + 1, nx);
    }
    if (ch < nfull) chunk(full_chunk{}, shared_tag, ch++, xs);
    if (ch * 32 < n) {
      load_chunk(t, ch, n, nx);
      chunk(tail_chunk{}, shared_tag, ch, nx);
    }
  };
  if (shared)
    run(std::integral_constant<bool, true>{});
  else
    run(std::integral_constant<bool, false>{});
  float bc = cost;
  int bs = s;
#pragma unroll
  for (int o = 1; o < S; o <<= 1) {
    const float oc = __shfl_xor(bc, o);
    const int os = __shfl_xor(bs, o);
    if (oc < bc || (oc == bc && os < bs)) {
      bc = oc;
      bs = os;
    }
  }
  if (live && s == 0) end_state[row] = bs;
}

// Traceback of trellis_viterbi2_kernel, two lanes per row: both walk the row's states through
// every chunk of 32 steps (one bit-field read of the transposed decision words per pair of
// steps), and lane h then decodes steps [16 h, 16 h + 16) of the chunk: the coset values of its
// 16 branches are read from LDS together, the nearest value of each taken (the smaller index on
// a tie), and its codes and values are written as whole 16-byte vectors.  The path's squared
// error is summed in fp64 per lane, the two halves added at the end.
template <int LOGS, int C>
__global__ __launch_bounds__(256) void trellis_traceback2_kernel(const float* __restrict__ T, int64_t ldt, int64_t rows,
                                                                 int n, const float* __restrict__ values,
                                                                 const uint32_t* __restrict__ bp,
                                                                 const int32_t* __restrict__ end_state,
                                                                 uint8_t* __restrict__ codes, int64_t ldc,
                                                                 float* __restrict__ recon, int64_t ldr,
                                                                 double* __restrict__ cost_out) {
  constexpr int S = 1 << LOGS;
  constexpr int E = 32 / S, P = 16 / S;  // bits per state field of a word, step pairs per field
  __shared__ __align__(16) float tab[S * 2 * C];
  for (int i = threadIdx.x; i < S * 2 * C; i += blockDim.x) tab[i] = values[i];
  __syncthreads();
  const int h = threadIdx.x & 1;
  const int64_t row0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 1;
  const bool live = row0 < rows;
  const int64_t row = live ? row0 : rows - 1;
  const float* t = T + row * ldt + 16 * h;
  const int64_t stride = rows * S;
  const int nfull = n >> 5;
  const bool vec = ldc % 16 == 0 && (reinterpret_cast<uintptr_t>(codes) & 15) == 0 &&
                   (!recon || (ldr % 4 == 0 && (reinterpret_cast<uintptr_t>(recon) & 15) == 0));
  // this lane's 16 targets of a whole chunk ch, and of the ragged last chunk (zeros past n)
  auto load_half = [&](int ch, float (&x)[16]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(t + ch * 32 + 4 * q);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[4 * q + e] = v[e];
    }
  };
  auto load_tail_half = [&](int ch, float (&x)[16]) {
    const int k0 = ch * 32 + 16 * h;
#pragma unroll
    for (int j = 0; j < 16; ++j) x[j] = k0 + j < n ? t[ch * 32 + j] : 0.0f;
  };
  float xs[16], nx[16];
  uint32_t w[S], nw[S];
  int cur = end_state[row];
  double acc = 0.0;
  auto load_words = [&](int ch, uint32_t (&wd)[S]) {
    const uint32_t* src = bp + (int64_t)ch * stride + row * S;
#pragma unroll
    for (int j = 0; j < S; ++j) wd[j] = src[j];
  };
  // chunk ch on the decision words wc and targets xc (FULL: all 32 steps before n)
  auto chunk = [&](auto full, int ch, const uint32_t (&wc)[S], const float (&xc)[16]) __attribute__((always_inline)) {
    constexpr bool FULL = decltype(full)::value;
    // walk the chunk's pairs of steps; br[2m + e] = the branch (2 p + u) taken into step
    // 16 h + 2 m + e: lane 1 keeps pairs 8..15, lane 0 pairs 0..7
    int br[16];
#pragma unroll
    for (int i = 15; i >= 0; --i) {
      if (FULL || ch * 32 + 2 * i < n) {
        const uint32_t d = __builtin_amdgcn_ubfe(wc[i / P], (uint32_t)(E * cur + 2 * (i % P)), 2u);
        const int mid = (cur >> 1) + (int)(d & 1u) * (S / 2);
        const int p = (mid >> 1) + (int)(d >> 1) * (S / 2);
        const int bhi = 2 * mid + (cur & 1), blo = 2 * p + (mid & 1);
        if (i >= 8) {
          br[2 * (i - 8)] = blo;
          br[2 * (i - 8) + 1] = bhi;
        } else {
          br[2 * i] = h ? br[2 * i] : blo;
          br[2 * i + 1] = h ? br[2 * i + 1] : bhi;
        }
        cur = p;
      } else if (i >= 8) {
        br[2 * (i - 8)] = 0;
        br[2 * (i - 8) + 1] = 0;
      } else if (!h) {
        br[2 * i] = 0;
        br[2 * i + 1] = 0;
      }
    }
    float cv[16][C];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float* cs = tab + br[e] * C;
      if constexpr (C == 4) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(cs);
#pragma unroll
        for (int c = 0; c < 4; ++c) cv[e][c] = v[c];
      } else if constexpr (C == 2) {
        const f32x2 v = *reinterpret_cast<const f32x2*>(cs);
        cv[e][0] = v[0];
        cv[e][1] = v[1];
      } else {
        cv[e][0] = cs[0];
      }
    }
    const int k0 = ch * 32 + 16 * h;
    uint32_t cw[4] = {0u, 0u, 0u, 0u};
    float rv[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float x = xc[e];
      int vb = 0;
      float rb = cv[e][0];
      float db = (x - rb) * (x - rb);
#pragma unroll
      for (int c = 1; c < C; ++c) {
        const float d = (x - cv[e][c]) * (x - cv[e][c]);
        if (d < db) {  // a tie keeps the smaller index
          db = d;
          rb = cv[e][c];
          vb = c;
        }
      }
      rv[e] = rb;
      cw[e >> 2] |= (uint32_t)((br[e] & 1) | (vb << 1)) << (8 * (e & 3));
      if (FULL || k0 + e < n) {
        const double dd = (double)x - (double)rb;
        acc = fma(dd, dd, acc);
      }
    }
    if (live && (FULL || k0 < n)) {
      uint8_t* cd = codes + row * ldc + k0;
      float* rd = recon ? recon + row * ldr + k0 : nullptr;
      if (vec && (FULL || k0 + 16 <= n)) {
        *reinterpret_cast<u32x4*>(cd) = u32x4{cw[0], cw[1], cw[2], cw[3]};
        if (rd) {
#pragma unroll
          for (int qq = 0; qq < 4; ++qq)
            *reinterpret_cast<f32x4*>(rd + 4 * qq) = f32x4{rv[4 * qq], rv[4 * qq + 1], rv[4 * qq + 2], rv[4 * qq + 3]};
        }
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (k0 + e < n) {
            cd[e] = (uint8_t)(cw[e >> 2] >> (8 * (e & 3)));
            if (rd) rd[e] = rv[e];
          }
      }
    }
  };
  // The ragged last chunk first, then whole chunks two per iteration with the buffers trading
  // roles, each chunk's words and targets loaded one chunk ahead by unconditional vector loads
  // (index clamped at 0), as in the forward kernel.
  const bool ragged = nfull * 32 < n;
  if (ragged) {
    load_words(nfull, nw);
    load_tail_half(nfull, nx);
  }
  if (nfull > 0) {
    load_words(nfull - 1, w);
    load_half(nfull - 1, xs);
  }
  __builtin_amdgcn_s_waitcnt(0);
  if (ragged) chunk(tail_chunk{}, nfull, nw, nx);
  int ch = nfull - 1;
  for (; ch >= 1; ch -= 2) {
    load_words(ch - 1, nw);
    load_half(ch - 1, nx);
    __builtin_amdgcn_sched_barrier(0);  // keep the loads a whole chunk ahead of their use
    chunk(full_chunk{}, ch, w, xs);
    const int c2 = ch >= 2 ? ch - 2 : 0;
    load_words(c2, w);
    load_half(c2, xs);
    __builtin_amdgcn_sched_barrier(0);
    chunk(full_chunk{}, ch - 1, nw, nx);
  }
  if (ch == 0) chunk(full_chunk{}, 0, w, xs);
  const int lo = __shfl_xor(__double2loint(acc), 1), hi = __shfl_xor(__double2hiint(acc), 1);
  const double other = __hiloint2double(hi, lo);
  if (live && h == 0 && cost_out) cost_out[row] = acc + other;
}

}  // namespace wr

using namespace wr;

size_t wr_trellis_ws_bytes(int64_t rows, int64_t n, int32_t states) {
  return (((size_t)((n + 31) / 32) * (size_t)rows * (size_t)states * 4 + 255) & ~(size_t)255) + (size_t)rows * 4;
}

int wr_trellis_quantize_impl(wr_ctx* ctx, const float* T, int64_t ldt, int64_t rows, int64_t n, int32_t log2_states,
                             int32_t coset_size, const float* values, int32_t start_state, uint8_t* codes, int64_t ldc,
                             float* recon, int64_t ldr, double* cost) {
  if (rows == 0) return WR_OK;
  const int S = 1 << log2_states;
  if (ctx->ws_bytes < wr_trellis_ws_bytes(rows, n, S)) return WR_EWORKSPACE;
  uint32_t* bp = static_cast<uint32_t*>(ctx->ws);
  int32_t* end_state = reinterpret_cast<int32_t*>(
      static_cast<char*>(ctx->ws) + (((size_t)((n + 31) / 32) * (size_t)rows * S * 4 + 255) & ~(size_t)255));
  const dim3 grid((unsigned)((rows * S + 255) / 256));
  const dim3 tgrid((unsigned)((rows + 255) / 256));
  const dim3 tgrid2((unsigned)((2 * rows + 255) / 256));
#define WR_TRL(LS, CC)                                                                                                \
  hipLaunchKernelGGL((trellis_viterbi_kernel<LS, CC>), grid, dim3(256), 0, ctx->stream, T, ldt, rows, (int)n, values,    \
                     start_state, bp, end_state);                                                                       \
  hipLaunchKernelGGL((trellis_traceback_kernel<LS, CC>), tgrid, dim3(256), 0, ctx->stream, T, ldt, rows, (int)n, values, \
                     bp, end_state, codes, ldc, recon, ldr, cost)
#define WR_TRL2(LS, CC)                                                                                               \
  hipLaunchKernelGGL((trellis_viterbi2_kernel<LS, CC>), grid, dim3(256), 0, ctx->stream, T, ldt, rows, (int)n, values,    \
                     start_state, bp, end_state);                                                                        \
  hipLaunchKernelGGL((trellis_traceback2_kernel<LS, CC>), tgrid2, dim3(256), 0, ctx->stream, T, ldt, rows, (int)n, values, \
                     bp, end_state, codes, ldc, recon, ldr, cost)
#define WR_TRL_C(M, LS)                \
  switch (coset_size) {                \
    case 1: M(LS, 1); break;           \
    case 2: M(LS, 2); break;           \
    default: M(LS, 4); break;          \
  }
  // one step per exchange for 2 states, two steps per exchange from 4 states on
  switch (log2_states) {
    case 1: WR_TRL_C(WR_TRL, 1); break;
    case 2: WR_TRL_C(WR_TRL2, 2); break;
    case 3: WR_TRL_C(WR_TRL2, 3); break;
    default: WR_TRL_C(WR_TRL2, 4); break;
  }
#undef WR_TRL_C
#undef WR_TRL2
#undef WR_TRL
  WR_CHECK_LAUNCH();
  return WR_OK;
}
