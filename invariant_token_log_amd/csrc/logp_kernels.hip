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

// ---------------------------------------------------------------------------
// Single-launch forward ("Batch-Invariant LogP", Tensor Parallel with one
// shard).  One workgroup per row (grid-stride over rows); wave w of 8 reduces
// the tiles k = w, w + 8, ... and parks (m_k, s_k) in LDS; wave 0 merges them
// in ascending order, copies the target logit and writes logp and lse.
// Ignored rows are not read.  Which wave reduces a tile changes no bit: the
// tile statistic depends only on the tile.
// ---------------------------------------------------------------------------
template <typename T, int C, bool VEC>
__global__ __launch_bounds__(kFwdBlock) void logp_fwd_fused_kernel(
    const T* __restrict__ logits, int64_t ld, int64_t n, int64_t v,
    const void* __restrict__ tgt, int32_t tgt32, int64_t ignore_index, int ntiles,
    float* __restrict__ logp, float* __restrict__ lse, int* __restrict__ status) {
  const Targets targets{tgt, tgt32};
  extern __shared__ float lds[];
  float* lm = lds;
  float* ls = lds + ntiles;
  constexpr int W = C * kWave * Elt<T>::kPerChunk;
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  for (int64_t r = blockIdx.x; r < n; r += gridDim.x) {
    const int64_t t = targets[r];
    if (t == ignore_index) {
      if (threadIdx.x == 0) {
        logp[r] = 0.0f;
        if (lse) lse[r] = 0.0f;
      }
      continue;
    }
    const T* row = logits + r * ld;
    for (int k = wave; k < ntiles; k += kFwdWaves) {
      float mk, sk;
      tile_stats<T, C, VEC>(row, static_cast<int64_t>(k) * W, v, mk, sk);
      if (lane == 0) {
        lm[k] = mk;
        ls[k] = sk;
      }
    }
    __syncthreads();
    if (wave == 0) {
      const float L = merge_lse(lm, ls, ntiles, 1);
      if (lane == 0) {
        const bool valid = t >= 0 && t < v;
        const float xt = valid ? Elt<T>::load(row, t) : 0.0f;
        logp[r] = combine(xt, L, valid);
        if (lse) lse[r] = L;
        if (!valid && status) status[0] = 1;
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Shard partials: the same tile statistic over the tiles [k_begin, k_end) a
// shard owns, written to the tile-major [T, n] tables pm / ps.  The owner of
// the target's tile copies the target logit into pt[r].  Ignored rows are
// skipped (the merge never reads them).
// ---------------------------------------------------------------------------
template <typename T, int C, bool VEC>
__global__ __launch_bounds__(kFwdBlock) void logp_partials_kernel(
    const T* __restrict__ logits, int64_t ld, int64_t n, int64_t v,
    const void* __restrict__ tgt, int32_t tgt32, int64_t ignore_index, int k_begin,
    int k_end, float* __restrict__ pm, float* __restrict__ ps,
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
      float mk, sk;
      tile_stats<T, C, VEC>(row, static_cast<int64_t>(k) * W, v, mk, sk);
      if (lane == 0) {
        pm[static_cast<int64_t>(k) * n + r] = mk;
        ps[static_cast<int64_t>(k) * n + r] = sk;
      }
    }
    if (threadIdx.x == 0 && t >= 0 && t < v &&
        t >= static_cast<int64_t>(k_begin) * W && t < static_cast<int64_t>(k_end) * W)
      pt[r] = Elt<T>::load(row, t);
  }
}

// ---------------------------------------------------------------------------
// Merge of gathered partials: one wave per row, the same merge_lse and
// combine as the single-launch forward.  Partial (r, k) sits at
// p[r * row_stride + k * tile_stride] (tile-major [T, n] tables from the
// shard launches, row-major [n, T] tables from the fused LM head).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kBlock) void logp_merge_kernel(
    const float* __restrict__ pm, const float* __restrict__ ps, const float* __restrict__ pt,
    int64_t n, int ntiles, int64_t row_stride, int64_t tile_stride, int64_t v,
    const void* __restrict__ tgt, int32_t tgt32, int64_t ignore_index, float* __restrict__ logp,
    float* __restrict__ lse, int* __restrict__ status) {
  const Targets targets{tgt, tgt32};
  const int lane = threadIdx.x % kWave;
  const int64_t waves = static_cast<int64_t>(gridDim.x) * kWavesPerBlock;
  for (int64_t r = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + threadIdx.x / kWave; r < n;
       r += waves) {
    const int64_t t = targets[r];
    if (t == ignore_index) {
      if (lane == 0) {
        logp[r] = 0.0f;
        if (lse) lse[r] = 0.0f;
      }
      continue;
    }
    const float L = merge_lse(pm + r * row_stride, ps + r * row_stride, ntiles, tile_stride);
    if (lane == 0) {
      const bool valid = t >= 0 && t < v;
      logp[r] = combine(valid ? pt[r] : 0.0f, L, valid);
      if (lse) lse[r] = L;
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

__device__ __forceinline__ float grad_elem(float x, float L, float g, float ng, bool is_target) {
  const float p = exp_sub(x, L);
  return is_target ? g * (1.0f - p) : ng * p;
}

template <typename T>
__device__ __forceinline__ uint4 grad_chunk(const uint4 q, float L, float g, float ng,
                                            int64_t c, int64_t t) {
  constexpr int E = Elt<T>::kPerChunk;
  float x[E];
  widen_chunk<T>(q, x);
  float d[E];
  if (t >= c && t < c + E) {
#pragma unroll
    for (int e = 0; e < E; ++e) d[e] = grad_elem(x[e], L, g, ng, c + e == t);
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) d[e] = ng * exp_sub(x[e], L);
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

template <typename T, bool VEC>
__global__ __launch_bounds__(kBlock) void logp_bwd_kernel(
    const T* logits, int64_t ld, int64_t n, int64_t v,
    const void* __restrict__ tgt, int32_t tgt32, int64_t ignore_index,
    const float* __restrict__ lse, const float* __restrict__ grad, T* dlogits,
    int64_t ld_out) {
  const Targets targets{tgt, tgt32};
  constexpr int E = Elt<T>::kPerChunk;
  // Thread (x, tid) owns the 16-byte chunk c = x * 256 + tid of every row it
  // visits: consecutive workgroups walk along a row, so the whole launch
  // streams the matrix in address order.
  const int64_t j0 = (static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x) * E;
  if (j0 >= v) return;
  const bool full = VEC && j0 + E <= v;
  for (int64_t r = blockIdx.y; r < n; r += gridDim.y) {
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
    const float L = lse[r];
    const float g = grad[r];
    const float ng = -g;
    if (full) {
      store_stream(orow + j0, grad_chunk<T>(load_stream(row + j0), L, g, ng, j0, t));
    } else {
      for (int e = 0; e < E; ++e)
        if (j0 + e < v)
          store_elem<T>(orow, j0 + e, grad_elem(Elt<T>::load(row, j0 + e), L, g, ng, j0 + e == t));
    }
  }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
static unsigned row_grid(int64_t n) {
  return static_cast<unsigned>(n < kMaxRowBlocks ? n : kMaxRowBlocks);
}

template <typename T, bool VEC>
static void fused_dispatch(int chunks, const void* logits, int64_t ld, int64_t n, int64_t v,
                           Targets tg, int64_t ignore, int ntiles, float* logp, float* lse,
                           int* status, hipStream_t s) {
  const size_t lds = static_cast<size_t>(ntiles) * 2 * sizeof(float);
  const T* x = static_cast<const T*>(logits);
#define ITL_FUSED(CC)                                                                        \
  case CC:                                                                                   \
    hipLaunchKernelGGL((logp_fwd_fused_kernel<T, CC, VEC>), dim3(row_grid(n)),               \
                       dim3(kFwdBlock), lds, s, x, ld, n, v, tg.p, tg.is32, ignore, ntiles, \
                       logp, lse, status);                                                   \
    break;
  switch (chunks) { ITL_FUSED(1) ITL_FUSED(2) ITL_FUSED(4) ITL_FUSED(8) ITL_FUSED(16) }
#undef ITL_FUSED
}

template <typename T, bool VEC>
static void partials_dispatch(int chunks, const void* logits, int64_t ld, int64_t n,
                              int64_t v, Targets tg, int64_t ignore, int kb, int ke, float* pm,
                              float* ps, float* pt, hipStream_t s) {
  const T* x = static_cast<const T*>(logits);
#define ITL_PART(CC)                                                                           \
  case CC:                                                                                     \
    hipLaunchKernelGGL((logp_partials_kernel<T, CC, VEC>), dim3(row_grid(n)),                  \
                       dim3(kFwdBlock), 0, s, x, ld, n, v, tg.p, tg.is32, ignore, kb, ke, pm, \
                       ps, pt);                                                                \
    break;
  switch (chunks) { ITL_PART(1) ITL_PART(2) ITL_PART(4) ITL_PART(8) ITL_PART(16) }
#undef ITL_PART
}

void launch_fwd_fused(int dtype, bool vec, int chunks, const void* logits, int64_t ld,
                      int64_t n, int64_t v, Targets tg, int64_t ignore, int ntiles,
                      float* logp, float* lse, int* status, hipStream_t s) {
#define ITL_F(TT, VV) \
  fused_dispatch<TT, VV>(chunks, logits, ld, n, v, tg, ignore, ntiles, logp, lse, status, s)
  if (dtype == kF32) {
    if (vec) ITL_F(float, true); else ITL_F(float, false);
  } else if (dtype == kF16) {
    if (vec) ITL_F(_Float16, true); else ITL_F(_Float16, false);
  } else {
    if (vec) ITL_F(uint16_t, true); else ITL_F(uint16_t, false);
  }
#undef ITL_F
}

void launch_fwd_partials(int dtype, bool vec, int chunks, const void* logits, int64_t ld,
                         int64_t n, int64_t v, Targets tg, int64_t ignore, int k_begin,
                         int k_end, float* pm, float* ps, float* pt, hipStream_t s) {
#define ITL_P(TT, VV) \
  partials_dispatch<TT, VV>(chunks, logits, ld, n, v, tg, ignore, k_begin, k_end, pm, ps, pt, s)
  if (dtype == kF32) {
    if (vec) ITL_P(float, true); else ITL_P(float, false);
  } else if (dtype == kF16) {
    if (vec) ITL_P(_Float16, true); else ITL_P(_Float16, false);
  } else {
    if (vec) ITL_P(uint16_t, true); else ITL_P(uint16_t, false);
  }
#undef ITL_P
}

void launch_fwd_merge(const float* pm, const float* ps, const float* pt, int64_t n,
                      int ntiles, int64_t row_stride, int64_t tile_stride, int64_t v,
                      Targets tg, int64_t ignore, float* logp, float* lse, int* status,
                      hipStream_t s) {
  int64_t blocks = (n + kWavesPerBlock - 1) / kWavesPerBlock;
  if (blocks > kMaxRowBlocks) blocks = kMaxRowBlocks;
  hipLaunchKernelGGL(logp_merge_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kBlock), 0,
                     s, pm, ps, pt, n, ntiles, row_stride, tile_stride, v, tg.p, tg.is32, ignore,
                     logp, lse, status);
}

template <typename T>
static void bwd_dispatch(bool vec, dim3 grid, const void* logits, int64_t ld, int64_t n,
                         int64_t v, Targets tg, int64_t ignore, const float* lse,
                         const float* grad, void* dlogits, int64_t ld_out, hipStream_t s) {
  const T* x = static_cast<const T*>(logits);
  T* d = static_cast<T*>(dlogits);
  if (vec)
    hipLaunchKernelGGL((logp_bwd_kernel<T, true>), grid, dim3(kBlock), 0, s, x, ld, n, v, tg.p,
                       tg.is32, ignore, lse, grad, d, ld_out);
  else
    hipLaunchKernelGGL((logp_bwd_kernel<T, false>), grid, dim3(kBlock), 0, s, x, ld, n, v, tg.p,
                       tg.is32, ignore, lse, grad, d, ld_out);
}

void launch_bwd(int dtype, bool vec, const void* logits, int64_t ld, int64_t n, int64_t v,
                Targets tg, int64_t ignore, const float* lse, const float* grad, void* dlogits,
                int64_t ld_out, hipStream_t s) {
  const int64_t per = dtype == kF32 ? 4 : 8;  // elements per 16-byte chunk
  const int64_t chunks = (v + per - 1) / per;
  const dim3 grid(static_cast<unsigned>((chunks + kBlock - 1) / kBlock),
                  static_cast<unsigned>(n < kMaxGridY ? n : kMaxGridY));
  if (dtype == kF32)
    bwd_dispatch<float>(vec, grid, logits, ld, n, v, tg, ignore, lse, grad, dlogits, ld_out, s);
  else if (dtype == kF16)
    bwd_dispatch<_Float16>(vec, grid, logits, ld, n, v, tg, ignore, lse, grad, dlogits, ld_out,
                           s);
  else
    bwd_dispatch<uint16_t>(vec, grid, logits, ld, n, v, tg, ignore, lse, grad, dlogits, ld_out,
                           s);
}

}  // namespace itl
