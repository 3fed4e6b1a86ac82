// Streaming kernels of the logp contract on gfx950: the single-launch
// forward, the shard-partial forward, the fixed-order merge and the
// tile-wise backward.  Host-side argument checks live in api.hip; the
// launchers here assume valid arguments.
#include "launch.h"
#include "logp_device.h"

namespace itl {

constexpr int kBlock = 256;               // 4 waves (merge kernel, backward)
constexpr int kWavesPerBlock = kBlock / kWave;
constexpr int kFwdBlock = 512;            // 8 waves per row in the forward kernels
constexpr int kFwdWaves = kFwdBlock / kWave;
constexpr int64_t kMaxRowBlocks = 1 << 20;  // grid-stride beyond this
constexpr int64_t kMaxGridY = 65535;        // backward grid rows (grid-stride beyond)
constexpr int kMergeChunks = 16;             // merge: 64-tile chunks a lane loads at once

// ---------------------------------------------------------------------------
// Single-launch forward ("Batch-Invariant LogP", Tensor Parallel with one
// shard).  One workgroup per row (grid-stride over rows); wave w of 8 reduces
// the tiles k = w, w + 8, ... and parks (m_k, s_k[, w_k]) in LDS; wave 0
// merges them in ascending order, copies the target logit and writes logp,
// lse (and the entropy with ENT).  Ignored rows are not read.  Which wave
// reduces a tile changes no bit: the tile statistic depends only on the tile.
// ---------------------------------------------------------------------------
template <typename T, int C, bool VEC, bool ENT>
__global__ __launch_bounds__(kFwdBlock) void logp_fwd_fused_kernel(
    const T* __restrict__ logits, int64_t ld, int64_t n, int64_t v,
    const void* __restrict__ tgt, int32_t tgt32, int64_t ignore_index, int ntiles,
    float* __restrict__ logp, float* __restrict__ lse, float* __restrict__ ent,
    int* __restrict__ status) {
  const Targets targets{tgt, tgt32};
  extern __shared__ float lds[];
  __shared__ MergeStage stage;  // wave 0's merge
  float* lm = lds;
  float* ls = lds + ntiles;
  float* lw = lds + 2 * ntiles;  // ENT only
  constexpr int W = C * kWave * Elt<T>::kPerChunk;
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  for (int64_t r = blockIdx.x; r < n; r += gridDim.x) {
    const int64_t t = targets[r];
    if (t == ignore_index) {
      if (threadIdx.x == 0) {
        logp[r] = 0.0f;
        if (lse) lse[r] = 0.0f;
        if (ENT) ent[r] = 0.0f;
      }
      continue;
    }
    const T* row = logits + r * ld;
    for (int k = wave; k < ntiles; k += kFwdWaves) {
      float mk, sk, wk;
      tile_stats<T, C, VEC, ENT>(row, static_cast<int64_t>(k) * W, v, mk, sk, &wk);
      if (lane == 0) {
        lm[k] = mk;
        ls[k] = sk;
        if (ENT) lw[k] = wk;
      }
    }
    __syncthreads();
    if (wave == 0) {
      float h = 0.0f;
      const float L = merge_lse_t<ENT, 1>(lm, ls, lw, ntiles, 1, stage, &h);
      if (lane == 0) {
        const bool valid = t >= 0 && t < v;
        const float xt = valid ? Elt<T>::load(row, t) : 0.0f;
        logp[r] = combine(xt, L, valid);
        if (lse) lse[r] = L;
        if (ENT) ent[r] = h;
        if (!valid && status) status[0] = 1;
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Shard partials: the same tile statistic over the tiles [k_begin, k_end) a
// shard owns, written to the tile-major [T, n] tables pm / ps (/ pw with ENT).
// The owner of the target's tile copies the target logit into pt[r].  Ignored
// rows are skipped (the merge never reads them).
// ---------------------------------------------------------------------------
template <typename T, int C, bool VEC, bool ENT>
__global__ __launch_bounds__(kFwdBlock) void logp_partials_kernel(
    const T* __restrict__ logits, int64_t ld, int64_t n, int64_t v,
    const void* __restrict__ tgt, int32_t tgt32, int64_t ignore_index, int k_begin,
    int k_end, float* __restrict__ pm, float* __restrict__ ps, float* __restrict__ pw,
    float* __restrict__ pt) {
  const Targets targets{tgt, tgt32};
  constexpr int W = C * kWave * Elt<T>::kPerChunk;
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  for (int64_t r = blockIdx.x; r < n; r += gridDim.x) {
    const int64_t t = targets[r];
    if (t == ignore_index) continue;
    const T* row = logits + r * ld;
    for (int k = k_begin + wave; k < k_end; k += kFwdWaves) {
      float mk, sk, wk;
      tile_stats<T, C, VEC, ENT>(row, static_cast<int64_t>(k) * W, v, mk, sk, &wk);
      if (lane == 0) {
        pm[static_cast<int64_t>(k) * n + r] = mk;
        ps[static_cast<int64_t>(k) * n + r] = sk;
        if (ENT) pw[static_cast<int64_t>(k) * n + r] = wk;
      }
    }
    if (threadIdx.x == 0 && t >= 0 && t < v &&
        t >= static_cast<int64_t>(k_begin) * W && t < static_cast<int64_t>(k_end) * W)
      pt[r] = Elt<T>::load(row, t);
  }
}

// ---------------------------------------------------------------------------
// Merge of gathered partials: one wave per row, the same merge and combine as
// the single-launch forward.  Partial (r, k) sits at
// p[r * row_stride + k * tile_stride] (tile-major [T, n] tables from the
// shard launches, row-major [n, T] tables from the fused LM head).
// ---------------------------------------------------------------------------
template <bool ENT>
__global__ __launch_bounds__(kBlock) void logp_merge_kernel(
    const float* __restrict__ pm, const float* __restrict__ ps, const float* __restrict__ pw,
    const float* __restrict__ pt, int64_t n, int ntiles, int64_t row_stride,
    int64_t tile_stride, int64_t v, const void* __restrict__ tgt, int32_t tgt32,
    int64_t ignore_index, float* __restrict__ logp, float* __restrict__ lse,
    float* __restrict__ ent, int* __restrict__ status) {
  const Targets targets{tgt, tgt32};
  __shared__ MergeStage stage[kWavesPerBlock];
  const int lane = threadIdx.x % kWave;
  const int64_t waves = static_cast<int64_t>(gridDim.x) * kWavesPerBlock;
  for (int64_t r = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + threadIdx.x / kWave; r < n;
       r += waves) {
    const int64_t t = targets[r];
    if (t == ignore_index) {
      if (lane == 0) {
        logp[r] = 0.0f;
        if (lse) lse[r] = 0.0f;
        if (ENT) ent[r] = 0.0f;
      }
      continue;
    }
    float h = 0.0f;
    const float L = merge_lse_t<ENT, kMergeChunks>(pm + r * row_stride, ps + r * row_stride,
                                                   pw + r * row_stride, ntiles, tile_stride,
                                                   stage[threadIdx.x / kWave], &h);
    if (lane == 0) {
      const bool valid = t >= 0 && t < v;
      logp[r] = combine(valid ? pt[r] : 0.0f, L, valid);
      if (lse) lse[r] = L;
      if (ENT) ent[r] = h;
      if (!valid && status) status[0] = 1;
    }
  }
}

// ---------------------------------------------------------------------------
// Backward ("Batch-Invariant LogP", Batch-Invariance: one program per row
// tile reusing the forward's lse, no cross-row reduction).
//   p = exp(x - lse);  u = 1 - p on the target column, -p elsewhere;
//   d = g * u rounded to the logits dtype (RNE).
// g * (-p) is computed as (-g) * p, which is the same IEEE product.
// Grid: x = 256-chunk segments of a row, y = rows; one 16-byte chunk per
// thread, non-temporal loads and stores.  Ignored rows are written +0 without
// reading the logits.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const __bf16 a = static_cast<__bf16>(lo);
  const __bf16 b = static_cast<__bf16>(hi);
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, a)) |
         (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b)) << 16);
}

__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
  const _Float16 a = static_cast<_Float16>(lo);  // v_cvt_f16_f32: round to nearest even
  const _Float16 b = static_cast<_Float16>(hi);
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, a)) |
         (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b)) << 16);
}

template <typename T> __device__ __forceinline__ void store_elem(T* p, int64_t i, float d);
template <> __device__ __forceinline__ void store_elem<float>(float* p, int64_t i, float d) {
  p[i] = d;
}
template <> __device__ __forceinline__ void store_elem<uint16_t>(uint16_t* p, int64_t i, float d) {
  p[i] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(d));
}
template <> __device__ __forceinline__ void store_elem<_Float16>(_Float16* p, int64_t i, float d) {
  p[i] = static_cast<_Float16>(d);
}

// Per-row constants of the gradient: lse, g, -g and, with the entropy term,
// the row entropy H and -gH.
struct GradRow {
  float L, g, ng, H, ngh;
};

// d = g (1 - p) on the target column, (-g) p elsewhere, p = e^(x - lse); with
// ENT the entropy gradient -gH p (log p + H) is added by one fma, log p taken
// as x - lse (the subtraction of exp_sub, kept).  A -inf logit has p = 0 and
// its entropy term is clamped to an exact -0.
template <bool ENT>
__device__ __forceinline__ float grad_val(float x, const GradRow& q, bool is_target) {
  if constexpr (ENT) {
    const float dl = x - q.L;  // exp_sub(x, L) in two steps
    const float p = __builtin_amdgcn_exp2f(dl * kLog2e);
    const float d = is_target ? q.g * (1.0f - p) : q.ng * p;
    return fmaf(q.ngh, p * fmaxf(dl + q.H, -FLT_MAX), d);
  } else {
    const float p = exp_sub(x, q.L);
    return is_target ? q.g * (1.0f - p) : q.ng * p;
  }
}

template <typename T, bool ENT>
__device__ __forceinline__ uint4 grad_chunk(const uint4 q, const GradRow& gr, int64_t c,
                                            int64_t t) {
  constexpr int E = Elt<T>::kPerChunk;
  float x[E];
  widen_chunk<T>(q, x);
  float d[E];
  if (t >= c && t < c + E) {
#pragma unroll
    for (int e = 0; e < E; ++e) d[e] = grad_val<ENT>(x[e], gr, c + e == t);
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) d[e] = grad_val<ENT>(x[e], gr, false);
  }
  uint4 o;
  if constexpr (E == 4) {
    o.x = __float_as_uint(d[0]); o.y = __float_as_uint(d[1]);
    o.z = __float_as_uint(d[2]); o.w = __float_as_uint(d[3]);
  } else if constexpr (__is_same(T, _Float16)) {
    o.x = pack_f16(d[0], d[1]); o.y = pack_f16(d[2], d[3]);
    o.z = pack_f16(d[4], d[5]); o.w = pack_f16(d[6], d[7]);
  } else {
    o.x = pack_bf16(d[0], d[1]); o.y = pack_bf16(d[2], d[3]);
    o.z = pack_bf16(d[4], d[5]); o.w = pack_bf16(d[6], d[7]);
  }
  return o;
}

template <typename T, bool VEC, bool ENT>
__global__ __launch_bounds__(kBlock) void logp_bwd_kernel(
    const T* logits, int64_t ld, int64_t n, int64_t v,
    const void* __restrict__ tgt, int32_t tgt32, int64_t ignore_index,
    const float* __restrict__ lse, const float* __restrict__ grad,
    const float* __restrict__ ent, const float* __restrict__ gent, T* dlogits,
    int64_t ld_out) {
  const Targets targets{tgt, tgt32};
  constexpr int E = Elt<T>::kPerChunk;
  // Thread (x, tid) owns the 16-byte chunk c = x * 256 + tid of every row it
  // visits: consecutive workgroups walk along a row, so the whole launch
  // streams the matrix row by row.  Rows go last to first, the reverse of the
  // forward, so the first rows read are those the forward read last and may
  // still sit in the last-level cache (measured: 0.6% off a fwd + bwd step).
  const int64_t j0 = (static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x) * E;
  if (j0 >= v) return;
  const bool full = VEC && j0 + E <= v;
  for (int64_t rr = blockIdx.y; rr < n; rr += gridDim.y) {
    const int64_t r = n - 1 - rr;
    const int64_t t = targets[r];
    T* orow = dlogits + r * ld_out;
    if (t == ignore_index) {
      if (full) {
        store_stream(orow + j0, make_uint4(0u, 0u, 0u, 0u));
      } else {
        for (int e = 0; e < E; ++e)
          if (j0 + e < v) store_elem<T>(orow, j0 + e, 0.0f);
      }
      continue;
    }
    const T* row = logits + r * ld;
    GradRow gr;
    gr.L = lse[r];
    gr.g = grad[r];
    gr.ng = -gr.g;
    gr.H = ENT ? ent[r] : 0.0f;
    gr.ngh = ENT ? -gent[r] : 0.0f;
    if (full) {
      store_stream(orow + j0, grad_chunk<T, ENT>(load_stream(row + j0), gr, j0, t));
    } else {
      for (int e = 0; e < E; ++e)
        if (j0 + e < v)
          store_elem<T>(orow, j0 + e, grad_val<ENT>(Elt<T>::load(row, j0 + e), gr, j0 + e == t));
    }
  }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
static unsigned row_grid(int64_t n) {
  return static_cast<unsigned>(n < kMaxRowBlocks ? n : kMaxRowBlocks);
}

template <typename T, bool VEC, bool ENT>
static void fused_dispatch(int chunks, const void* logits, int64_t ld, int64_t n, int64_t v,
                           Targets tg, int64_t ignore, int ntiles, float* logp, float* lse,
                           float* ent, int* status, hipStream_t s) {
  const size_t lds = static_cast<size_t>(ntiles) * (ENT ? 3 : 2) * sizeof(float);
  const T* x = static_cast<const T*>(logits);
#define ITL_FUSED(CC)                                                                        \
  case CC:                                                                                   \
    hipLaunchKernelGGL((logp_fwd_fused_kernel<T, CC, VEC, ENT>), dim3(row_grid(n)),          \
                       dim3(kFwdBlock), lds, s, x, ld, n, v, tg.p, tg.is32, ignore, ntiles, \
                       logp, lse, ent, status);                                              \
    break;
  switch (chunks) { ITL_FUSED(1) ITL_FUSED(2) ITL_FUSED(4) ITL_FUSED(8) ITL_FUSED(16) }
#undef ITL_FUSED
}

template <typename T, bool VEC, bool ENT>
static void partials_dispatch(int chunks, const void* logits, int64_t ld, int64_t n,
                              int64_t v, Targets tg, int64_t ignore, int kb, int ke, float* pm,
                              float* ps, float* pw, float* pt, hipStream_t s) {
  const T* x = static_cast<const T*>(logits);
#define ITL_PART(CC)                                                                           \
  case CC:                                                                                     \
    hipLaunchKernelGGL((logp_partials_kernel<T, CC, VEC, ENT>), dim3(row_grid(n)),             \
                       dim3(kFwdBlock), 0, s, x, ld, n, v, tg.p, tg.is32, ignore, kb, ke, pm, \
                       ps, pw, pt);                                                            \
    break;
  switch (chunks) { ITL_PART(1) ITL_PART(2) ITL_PART(4) ITL_PART(8) ITL_PART(16) }
#undef ITL_PART
}

// Instantiate a dispatcher for the dtype, the load path and the entropy flag.
#define ITL_TYPED(FN, DTYPE, VECF, ENTF, ...)                                        \
  do {                                                                               \
    if ((DTYPE) == kF32) {                                                           \
      if (VECF) { if (ENTF) FN<float, true, true>(__VA_ARGS__);                      \
                  else FN<float, true, false>(__VA_ARGS__); }                        \
      else { if (ENTF) FN<float, false, true>(__VA_ARGS__);                          \
             else FN<float, false, false>(__VA_ARGS__); }                            \
    } else if ((DTYPE) == kF16) {                                                    \
      if (VECF) { if (ENTF) FN<_Float16, true, true>(__VA_ARGS__);                   \
                  else FN<_Float16, true, false>(__VA_ARGS__); }                     \
      else { if (ENTF) FN<_Float16, false, true>(__VA_ARGS__);                       \
             else FN<_Float16, false, false>(__VA_ARGS__); }                         \
    } else {                                                                         \
      if (VECF) { if (ENTF) FN<uint16_t, true, true>(__VA_ARGS__);                   \
                  else FN<uint16_t, true, false>(__VA_ARGS__); }                     \
      else { if (ENTF) FN<uint16_t, false, true>(__VA_ARGS__);                       \
             else FN<uint16_t, false, false>(__VA_ARGS__); }                         \
    }                                                                                \
  } while (0)

void launch_fwd_fused(int dtype, bool vec, int chunks, const void* logits, int64_t ld,
                      int64_t n, int64_t v, Targets tg, int64_t ignore, int ntiles,
                      float* logp, float* lse, float* ent, int* status, hipStream_t s) {
  ITL_TYPED(fused_dispatch, dtype, vec, ent != nullptr, chunks, logits, ld, n, v, tg, ignore,
            ntiles, logp, lse, ent, status, s);
}

void launch_fwd_partials(int dtype, bool vec, int chunks, const void* logits, int64_t ld,
                         int64_t n, int64_t v, Targets tg, int64_t ignore, int k_begin,
                         int k_end, float* pm, float* ps, float* pw, float* pt, hipStream_t s) {
  ITL_TYPED(partials_dispatch, dtype, vec, pw != nullptr, chunks, logits, ld, n, v, tg, ignore,
            k_begin, k_end, pm, ps, pw, pt, s);
}

void launch_fwd_merge(const float* pm, const float* ps, const float* pw, const float* pt,
                      int64_t n, int ntiles, int64_t row_stride, int64_t tile_stride, int64_t v,
                      Targets tg, int64_t ignore, float* logp, float* lse, float* ent,
                      int* status, hipStream_t s) {
  int64_t blocks = (n + kWavesPerBlock - 1) / kWavesPerBlock;
  if (blocks > kMaxRowBlocks) blocks = kMaxRowBlocks;
  if (ent)
    hipLaunchKernelGGL(logp_merge_kernel<true>, dim3(static_cast<unsigned>(blocks)),
                       dim3(kBlock), 0, s, pm, ps, pw, pt, n, ntiles, row_stride, tile_stride,
                       v, tg.p, tg.is32, ignore, logp, lse, ent, status);
  else
    hipLaunchKernelGGL(logp_merge_kernel<false>, dim3(static_cast<unsigned>(blocks)),
                       dim3(kBlock), 0, s, pm, ps, ps, pt, n, ntiles, row_stride, tile_stride,
                       v, tg.p, tg.is32, ignore, logp, lse, ent, status);
}

template <typename T, bool VEC, bool ENT>
static void bwd_dispatch(dim3 grid, const void* logits, int64_t ld, int64_t n, int64_t v,
                         Targets tg, int64_t ignore, const float* lse, const float* grad,
                         const float* ent, const float* gent, void* dlogits, int64_t ld_out,
                         hipStream_t s) {
  hipLaunchKernelGGL((logp_bwd_kernel<T, VEC, ENT>), grid, dim3(kBlock), 0, s,
                     static_cast<const T*>(logits), ld, n, v, tg.p, tg.is32, ignore, lse, grad,
                     ent, gent, static_cast<T*>(dlogits), ld_out);
}

void launch_bwd(int dtype, bool vec, const void* logits, int64_t ld, int64_t n, int64_t v,
                Targets tg, int64_t ignore, const float* lse, const float* grad,
                const float* ent, const float* gent, void* dlogits, int64_t ld_out,
                hipStream_t s) {
  const int64_t per = dtype == kF32 ? 4 : 8;  // elements per 16-byte chunk
  const int64_t chunks = (v + per - 1) / per;
  const dim3 grid(static_cast<unsigned>((chunks + kBlock - 1) / kBlock),
                  static_cast<unsigned>(n < kMaxGridY ? n : kMaxGridY));
  ITL_TYPED(bwd_dispatch, dtype, vec, ent != nullptr, grid, logits, ld, n, v, tg, ignore, lse,
            grad, ent, gent, dlogits, ld_out, s);
}

#undef ITL_TYPED

}  // namespace itl
