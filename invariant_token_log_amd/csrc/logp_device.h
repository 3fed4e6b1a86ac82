// Device arithmetic shared by every kernel of the logp contract.
//
// The tile statistic, the wave reductions, the exp/log primitives and the
// fixed-order merge live here once, so that the single-launch forward, the
// shard-partial kernel, the merge kernel, the backward and the fused LM-head
// epilogue all perform the same floating-point operations in the same order
// ("Batch-Invariant LogP", Tensor Parallel: every tile is reduced as the same
// contiguous shape on any rank and every rank merges in the same fixed
// order).  Built with -ffp-contract=off: every fused multiply-add below is an
// explicit fmaf, nothing else is contracted or reassociated.
#pragma once

#include <hip/hip_runtime.h>
#include <float.h>
#include <stdint.h>

namespace itl {

constexpr int kWave = 64;
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;

// e^(a - b) as 2^((a - b) * log2 e) on the hardware base-2 exponential
// (v_exp_f32).  The subtraction comes first, so the row maximum gives exactly
// 2^0 = 1: every tile that holds its own maximum has s >= 1, the merged sum is
// >= 1 and log(sum) >= 0, hence logp <= 0 on every active row.
__device__ __forceinline__ float exp_sub(float a, float b) {
  return __builtin_amdgcn_exp2f((a - b) * kLog2e);
}

// Natural log as log2 (v_log_f32) times ln 2.  Only called on sums >= 1.
__device__ __forceinline__ float log_nat(float a) {
  return __builtin_amdgcn_logf(a) * kLn2;
}

// Lane moves for the reductions below.  DPP within rows of 16 lanes: quad
// permutes, row rotations (rotating right by n hands lane i the value of lane
// i - n mod 16) and mirrors (lane i <- lane 15 - i; half mirror: lane i <-
// lane 7 - i within each 8).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}
constexpr int kDppXor1 = 0xB1;     // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;     // quad_perm [2, 3, 0, 1]
constexpr int kDppRowRor12 = 0x12C;  // lane i <- lane i + 4 (mod 16)
constexpr int kDppRowRor8 = 0x128;   // lane i <- lane i + 8 (mod 16)
constexpr int kDppRowMirror = 0x140;      // lane i <- lane 15 - i
constexpr int kDppRowHalfMirror = 0x141;  // lane i <- lane 7 - i (within 8)

// XOR butterfly over the 64 lanes of a wave, offsets 1, 2, 4, ..., 32: at
// level o every lane combines its value with that of lane i ^ o, and every
// lane ends with the same value (both partners combine the same two operands;
// addition and max commute exactly).  The partners come from lane moves
// without LDS: quad permutes give lanes i ^ 1 and i ^ 2 exactly; after those
// levels the four lanes of a quad hold one value, so the half mirror (lane
// 7 - i, in the other quad of the 8) supplies the value of lane i ^ 4; then
// the eight lanes of each half row agree and the row mirror (lane 15 - i, in
// the other half) supplies lane i ^ 8.  Offsets 16 and 32 use gfx950's
// permlane swaps of a value with itself: after v_permlane16_swap one operand
// holds rows (0, 0, 2, 2) and the other rows (1, 1, 3, 3), so combining the
// two gives every lane op(row r, row r ^ 1); v_permlane32_swap does the same
// for the two halves of the wave.
__device__ __forceinline__ float swap_combine16(float x, bool is_max) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  const float a = __uint_as_float(r[0]), b = __uint_as_float(r[1]);
  return is_max ? fmaxf(a, b) : a + b;
}
__device__ __forceinline__ float swap_combine32(float x, bool is_max) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  const float a = __uint_as_float(r[0]), b = __uint_as_float(r[1]);
  return is_max ? fmaxf(a, b) : a + b;
}

__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp_mov<kDppXor1>(x));
  x = fmaxf(x, dpp_mov<kDppXor2>(x));
  x = fmaxf(x, dpp_mov<kDppRowHalfMirror>(x));
  x = fmaxf(x, dpp_mov<kDppRowMirror>(x));
  x = swap_combine16(x, true);
  return swap_combine32(x, true);
}

__device__ __forceinline__ float wave_sum(float x) {
  x = x + dpp_mov<kDppXor1>(x);
  x = x + dpp_mov<kDppXor2>(x);
  x = x + dpp_mov<kDppRowHalfMirror>(x);
  x = x + dpp_mov<kDppRowMirror>(x);
  x = swap_combine16(x, false);
  return swap_combine32(x, false);
}

// The same butterfly with every partner fetched through the LDS crossbar
// (ds_bpermute): the same partners, so the same bits, but the moves use the
// LDS unit instead of vector ALU issue.  Wide tiles, whose per-lane work
// already keeps the ALU busy, reduce this way; narrow tiles, where the
// butterfly's latency dominates, use the lane moves above.
__device__ __forceinline__ float wave_max_lds(float x) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) x = fmaxf(x, __shfl_xor(x, o, kWave));
  return x;
}

__device__ __forceinline__ float wave_sum_lds(float x) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) x = x + __shfl_xor(x, o, kWave);
  return x;
}

// Reductions over the 16 lanes of a row (lanes 16r .. 16r+15) whose result is
// taken from the row's first lane.  That lane sees exactly the xor butterfly
// (offsets 1, 2, 4, 8): ((x0 + x1) + (x2 + x3)) + ((x4 + x5) + (x6 + x7)) ...
// in the same association as __shfl_xor steps, but the partners come from
// DPP lane moves instead of LDS-routed permutes: quad permutes for 1 and 2,
// then row rotations (a rotation right by n hands lane i the value of lane
// i - n mod 16), by 12 so that lane 0 reads lane 4, and by 8 so that it reads
// lane 8.  Other lanes of the row end with other, unused associations.
__device__ __forceinline__ float row16_sum_first(float x) {
  x = x + dpp_mov<kDppXor1>(x);
  x = x + dpp_mov<kDppXor2>(x);
  x = x + dpp_mov<kDppRowRor12>(x);
  x = x + dpp_mov<kDppRowRor8>(x);
  return x;
}

// The exact maximum of the LM-head statistics: IEEE maximum, which gfx950
// evaluates as v_maximum3_f32 on its operands as they are (fmaxf makes the
// compiler quiet each operand first, one more instruction per value).  On
// non-NaN values it equals fmaxf except that -0 orders below +0; the LM-head
// logits are never -0 (every accumulator starts at +0), and a tile maximum of
// either zero gives the same partial sums and merge anyway.  A NaN logit
// makes the tile maximum NaN, and with it the row's LSE, as its sum already
// would.
__device__ __forceinline__ float max_exact(float a, float b) {
  return __builtin_elementwise_maximum(a, b);
}

__device__ __forceinline__ float row16_max_first(float x) {
  x = max_exact(x, dpp_mov<kDppXor1>(x));
  x = max_exact(x, dpp_mov<kDppXor2>(x));
  x = max_exact(x, dpp_mov<kDppRowRor12>(x));
  x = max_exact(x, dpp_mov<kDppRowRor8>(x));
  return x;
}

// ---------------------------------------------------------------------------
// Element access.  bf16 is carried as its raw 16 bits; widening to fp32 is a
// 16-bit left shift and exact.
// ---------------------------------------------------------------------------

template <typename T> struct Elt;
template <> struct Elt<float> {
  static constexpr int kPerChunk = 4;  // 16 bytes
  __device__ static float load(const float* p, int64_t i) { return p[i]; }
};
template <> struct Elt<uint16_t> {  // bfloat16 bits
  static constexpr int kPerChunk = 8;  // 16 bytes
  __device__ static float load(const uint16_t* p, int64_t i) {
    return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
  }
};
template <> struct Elt<_Float16> {  // IEEE binary16, widened exactly (v_cvt_f32_f16)
  static constexpr int kPerChunk = 8;  // 16 bytes
  __device__ static float load(const _Float16* p, int64_t i) { return static_cast<float>(p[i]); }
};

// 16-byte streaming accesses with the non-temporal hint: the logits are read
// once per pass and the gradient is written once, so neither should displace
// other lines in L2; on gfx950 these loads also sustain a higher HBM read rate
// than plain ones.  They move the same bytes as plain accesses.
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream(const void* p) {
  const u32x4_t w = __builtin_nontemporal_load(static_cast<const u32x4_t*>(p));
  return make_uint4(w.x, w.y, w.z, w.w);
}
__device__ __forceinline__ void store_stream(void* p, uint4 v) {
  const u32x4_t w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, static_cast<u32x4_t*>(p));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float f16_lo(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w & 0xffffu)));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w >> 16)));
}

// Widen the elements of one 16-byte chunk to fp32 (exact for every type).
template <typename T>
__device__ __forceinline__ void widen_chunk(const uint4 q, float (&x)[Elt<T>::kPerChunk]) {
  if constexpr (Elt<T>::kPerChunk == 4) {
    x[0] = __uint_as_float(q.x); x[1] = __uint_as_float(q.y);
    x[2] = __uint_as_float(q.z); x[3] = __uint_as_float(q.w);
  } else if constexpr (sizeof(T) == 2 && __is_same(T, _Float16)) {
    x[0] = f16_lo(q.x); x[1] = f16_hi(q.x); x[2] = f16_lo(q.y); x[3] = f16_hi(q.y);
    x[4] = f16_lo(q.z); x[5] = f16_hi(q.z); x[6] = f16_lo(q.w); x[7] = f16_hi(q.w);
  } else {
    x[0] = bf16_lo(q.x); x[1] = bf16_hi(q.x); x[2] = bf16_lo(q.y); x[3] = bf16_hi(q.y);
    x[4] = bf16_lo(q.z); x[5] = bf16_hi(q.z); x[6] = bf16_lo(q.w); x[7] = bf16_hi(q.w);
  }
}

// Widen one 16-byte chunk that starts at element c of a row; elements at or
// beyond v become -inf and are not read.  VEC: the chunk start is 16-byte
// aligned, so a whole chunk is one 128-bit load.
template <typename T, bool VEC>
__device__ __forceinline__ void load_chunk(const T* row, int64_t c, int64_t v,
                                           float (&x)[Elt<T>::kPerChunk]) {
  constexpr int E = Elt<T>::kPerChunk;
  if (VEC && c + E <= v) {
    widen_chunk<T>(load_stream(row + c), x);
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e)
      x[e] = (c + e < v) ? Elt<T>::load(row, c + e) : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// Entropy moment.  Next to s = sum e_j, e_j = e^(x_j - m), a tile can carry
//   w = sum e_j * (x_j - m)
// folded in the same tree as s (one fma per term).  A term whose x_j is -inf
// (a padding column or a masked logit) has e_j = 0 and must add nothing: its
// difference is clamped to -FLT_MAX, so the product is an exact -0 instead of
// 0 * (-inf) = NaN.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float ent_term(float e, float d, float w) {
  return fmaf(e, fmaxf(d, -FLT_MAX), w);
}

// ---------------------------------------------------------------------------
// Tile statistic ("Batch-Invariant LogP", Tensor Parallel, step 2): one wave
// reduces the W = C * 64 * E columns [col0, col0 + W) of one row to
//   m = max x,   s = sum exp(x - m)   (fp32, two passes over registers),
// and, with ENT, the entropy moment w of the same terms.
// Layout: lane l holds chunks j = 0..C-1 covering the tile-local elements
// [(j * 64 + l) * E, +E), so every chunk load is one coalesced 1 KiB wave
// access.  Summation tree: each lane folds its C * E terms in ascending
// tile-local column order (chunk by chunk, element by element) starting from
// +0, then the xor butterfly adds across lanes.  The tree depends only on the
// column index inside the tile, on W and on the dtype.  Padding columns
// (>= v) contribute exp(-inf) = +0, which leaves every partial sum unchanged.
// ---------------------------------------------------------------------------
template <typename T, int C, bool VEC, bool ENT = false>
__device__ __forceinline__ void tile_stats(const T* row, int64_t col0, int64_t v,
                                           float& m_out, float& s_out, float* w_out = nullptr) {
  constexpr int E = Elt<T>::kPerChunk;
  const int lane = threadIdx.x & (kWave - 1);
  constexpr int W = C * kWave * E;
  float x[C][E];
  if (VEC && col0 + W <= v) {
    // Whole tile inside the row: unguarded 128-bit loads.
#pragma unroll
    for (int j = 0; j < C; ++j)
      load_chunk<T, true>(row, col0 + static_cast<int64_t>(j * kWave + lane) * E, INT64_MAX, x[j]);
  } else {
#pragma unroll
    for (int j = 0; j < C; ++j)
      load_chunk<T, VEC>(row, col0 + static_cast<int64_t>(j * kWave + lane) * E, v, x[j]);
  }
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < C; ++j)
#pragma unroll
    for (int e = 0; e < E; ++e) m = fmaxf(m, x[j][e]);
  // lane moves for tiles of at most 16 elements per lane, LDS crossbar above
  constexpr bool kLds = C * E > 16;
  m = kLds ? wave_max_lds(m) : wave_max(m);
  float s = 0.0f, w = 0.0f;
#pragma unroll
  for (int j = 0; j < C; ++j)
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if constexpr (ENT) {
        const float d = x[j][e] - m;  // exp_sub(x, m) evaluated in two steps
        const float ex = __builtin_amdgcn_exp2f(d * kLog2e);
        s = s + ex;
        w = ent_term(ex, d, w);
      } else {
        s = s + exp_sub(x[j][e], m);
      }
    }
  m_out = m;
  s_out = kLds ? wave_sum_lds(s) : wave_sum(s);
  if constexpr (ENT) *w_out = kLds ? wave_sum_lds(w) : wave_sum(w);
}

// ---------------------------------------------------------------------------
// Fixed-order merge ("Batch-Invariant LogP", Tensor Parallel, step 4):
//   M = max_k m_k;  acc = +0;  for k = 0 .. T-1:  acc = fma(s_k, e^(m_k - M), acc)
//   (tiles with m_k = -inf skipped: they hold no column);  LSE = M + log(acc).
// With ENT the same loop also folds b = fma(y_k, e^(m_k - M), b), y_k =
// fma(s_k, m_k - M, w_k) = sum over the tile of e^(x - M) (x - M) scaled back
// by e^(M - m_k), and the full-vocabulary entropy is
//   H = log(acc) - b / acc          (= LSE - sum_j p_j x_j).
// One wave evaluates one row.  The row's partials are loaded up front, PRE
// chunks of 64 tiles per lane at a time, so the loads of a row overlap instead
// of waiting one chunk after another.  The max is exact in any order; each
// exponential is the same function of the same two values, whichever lane
// takes it.  The ascending fma chains then run over the tiles in order, 64 at a
// time: each lane parks its (s_k, e_k[, y_k]) in a wave-private LDS stage and
// every lane folds the 64 entries by broadcast reads, so each step of the
// chain is one fma on exact copies of the operands.  Entries past the last
// tile are zeros: fma(0, 0, x) = x for every x but -0, and neither acc nor b
// is ever -0 (both start at +0 and an exact zero sum rounds to +0), so the
// fold may run on to a multiple of 8.  Partial k of the row is read at
// m[k * stride], s[k * stride] (w[k * stride]).  All 64 lanes must call; all
// return the LSE (and H).
// ---------------------------------------------------------------------------
struct MergeStage {
  float2 se[kWave];  // (s_k, e_k) of the 64 tiles being folded
  float y[kWave];    // y_k (entropy)
};

template <bool ENT, int PRE, typename P>
__device__ __forceinline__ float merge_lse_t(P m, P s, P w, int ntiles, int64_t stride,
                                             MergeStage& st, float* ent) {
  const int lane = threadIdx.x & (kWave - 1);
  constexpr int kGroup = PRE * kWave;  // tiles held in registers at once
  float mr[PRE], sr[PRE], wr[ENT ? PRE : 1];
  auto load = [&](int g0, bool with_sw) {
#pragma unroll
    for (int c = 0; c < PRE; ++c) {
      const int k = g0 + c * kWave + lane;
      const bool in = k < ntiles;
      mr[c] = in ? m[k * stride] : -INFINITY;
      if (with_sw) {
        sr[c] = in ? s[k * stride] : 0.0f;
        if constexpr (ENT) wr[c] = in ? w[k * stride] : 0.0f;
      }
    }
  };
  const bool one_group = ntiles <= kGroup;
  float mx = -INFINITY;
  for (int g0 = 0; g0 < ntiles; g0 += kGroup) {
    load(g0, one_group);
#pragma unroll
    for (int c = 0; c < PRE; ++c) mx = fmaxf(mx, mr[c]);
  }
  const float big_m = wave_max(mx);
  float acc = 0.0f, b = 0.0f;
  for (int g0 = 0; g0 < ntiles; g0 += kGroup) {
    if (!one_group) load(g0, true);
#pragma unroll
    for (int c = 0; c < PRE; ++c) {
      const int c0 = g0 + c * kWave;
      if (c0 < ntiles) {
        // A tile without columns (m_k = -inf) enters as s_k = e_k = y_k = 0,
        // the same fold as skipping it (see above).
        const bool live = mr[c] != -INFINITY;
        const float ek = live ? exp_sub(mr[c], big_m) : 0.0f;
        st.se[lane] = make_float2(live ? sr[c] : 0.0f, ek);
        if constexpr (ENT) st.y[lane] = live ? fmaf(sr[c], mr[c] - big_m, wr[c]) : 0.0f;
        __builtin_amdgcn_wave_barrier();
        const int cnt = ntiles - c0 < kWave ? ntiles - c0 : kWave;
        for (int j0 = 0; j0 < cnt; j0 += 8) {
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float2 p = st.se[j0 + j];
            acc = fmaf(p.x, p.y, acc);
            if constexpr (ENT) b = fmaf(st.y[j0 + j], p.y, b);
          }
        }
        __builtin_amdgcn_wave_barrier();
      }
    }
  }
  const float la = log_nat(acc);
  if constexpr (ENT) *ent = la - b / acc;
  return big_m + la;
}

// Final combine (step 6): logp = target_logit - LSE, or NaN for an active row
// whose target lies outside [0, v).
__device__ __forceinline__ float combine(float target_logit, float lse, bool valid) {
  return valid ? target_logit - lse : __uint_as_float(0x7fc00000u);
}

}  // namespace itl
