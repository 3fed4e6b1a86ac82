// Fused LM-head + logp statistics on gfx950 ("[RFC][ROCm] End-to-end
// optimization of bitwise VIME R/R beyond native P/P", Workstream 3: stream
// LM-head tiles through the matrix cores, take the local (max, sumexp,
// target) statistics and never store the [tokens, vocab] logits).
//
//   z[r, j] = sum_k hidden[r, k] * weight[j, k]
//
// Each workgroup computes a 128 (rows) x 256 (vocabulary) block of z in fp32
// with v_mfma_f32_16x16x32_bf16, walking K in ascending steps of 32, one
// accumulator per output and no split-K, so every z[r, j] is the same bits
// for any N, any row position and any grid.  The epilogue reduces each row's
// 256 columns to the tile pair (m, s) of the logp contract with the shared
// exp primitive, copies z at the target column, and writes them to the
// [T, n] partial tables that the fixed-order merge consumes.
#include "launch.h"
#include "logp_device.h"

namespace itl {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 128;             // rows of hidden per workgroup
constexpr int BN = kLinearTile;     // vocabulary columns per workgroup (= statistic tile)
constexpr int BK = 32;              // K per MFMA step
constexpr int kThreads = 256;       // 4 waves: 2 (rows) x 2 (columns)
constexpr int kLdsStride = BK + 8;  // bf16 elements per LDS row (80 B: breaks bank aliasing)
constexpr int kAChunks = BM * BK / 8 / kThreads;  // 16-byte chunks per thread per step
constexpr int kBChunks = BN * BK / 8 / kThreads;

struct Smem {
  uint16_t a[2][BM * kLdsStride];
  uint16_t b[2][BN * kLdsStride];
  float red[2][BM];       // per column-half row statistics
  int64_t target[BM];
};

// Blocks are dealt round-robin to the 8 XCDs; give each XCD one contiguous
// range of logical tiles so that a vocabulary block's weight rows are read
// into one XCD's L2 only.
__device__ __forceinline__ int xcd_logical(int b, int g) {
  const int x = b % 8, y = b / 8, per = g / 8, rem = g % 8;
  return x < rem ? x * (per + 1) + y : rem * (per + 1) + (x - rem) * per + y;
}

}  // namespace

__global__ __launch_bounds__(kThreads) void linear_logp_stats_kernel(
    const uint16_t* __restrict__ hidden, int64_t ld_h, const uint16_t* __restrict__ weight,
    int64_t ld_w, int64_t n, int64_t hdim, int64_t v, int mblocks, int vblocks,
    const int64_t* __restrict__ targets, int64_t ignore_index, float* __restrict__ pm,
    float* __restrict__ ps, float* __restrict__ pt) {
  __shared__ __align__(16) Smem sm;
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = tid / kWave;
  const int wm = wave / 2, wn = wave % 2;
  const int li = lane % 16, g = lane / 16;

  const int logical = xcd_logical(blockIdx.x, mblocks * vblocks);
  const int mb = logical % mblocks;
  const int vb = logical / mblocks;
  const int64_t m0 = static_cast<int64_t>(mb) * BM;
  const int64_t v0 = static_cast<int64_t>(vb) * BN;

  if (tid < BM) sm.target[tid] = (m0 + tid < n) ? targets[m0 + tid] : ignore_index;

  // Global -> register staging of one K step.
  uint4 ra[kAChunks], rb[kBChunks];
  auto fetch = [&](int64_t k0) {
#pragma unroll
    for (int p = 0; p < kAChunks; ++p) {
      const int c = tid + p * kThreads, row = c / 4, kc = c % 4;
      ra[p] = (m0 + row < n)
                  ? *reinterpret_cast<const uint4*>(hidden + (m0 + row) * ld_h + k0 + kc * 8)
                  : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int p = 0; p < kBChunks; ++p) {
      const int c = tid + p * kThreads, row = c / 4, kc = c % 4;
      rb[p] = (v0 + row < v)
                  ? *reinterpret_cast<const uint4*>(weight + (v0 + row) * ld_w + k0 + kc * 8)
                  : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int p = 0; p < kAChunks; ++p) {
      const int c = tid + p * kThreads, row = c / 4, kc = c % 4;
      *reinterpret_cast<uint4*>(&sm.a[buf][row * kLdsStride + kc * 8]) = ra[p];
    }
#pragma unroll
    for (int p = 0; p < kBChunks; ++p) {
      const int c = tid + p * kThreads, row = c / 4, kc = c % 4;
      *reinterpret_cast<uint4*>(&sm.b[buf][row * kLdsStride + kc * 8]) = rb[p];
    }
  };

  f32x4 acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  const int ksteps = static_cast<int>(hdim / BK);
  fetch(0);
  stash(0);
  __syncthreads();
  for (int kt = 0; kt < ksteps; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < ksteps) fetch(static_cast<int64_t>(kt + 1) * BK);
    bf16x8 a[4], b[8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      a[i] = *reinterpret_cast<const bf16x8*>(&sm.a[buf][(wm * 64 + i * 16 + li) * kLdsStride + g * 8]);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      b[j] = *reinterpret_cast<const bf16x8*>(&sm.b[buf][(wn * 128 + j * 16 + li) * kLdsStride + g * 8]);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    if (kt + 1 < ksteps) stash(buf ^ 1);
    __syncthreads();
  }

  // Epilogue.  acc[i][j][q] = z[m0 + wm*64 + i*16 + 4g + q][v0 + wn*128 + j*16 + li].
  // Tile statistic over the 256 columns of each row, two passes:
  //   max: lane max over j, xor butterfly over the 16 lanes of a row group
  //        (offsets 1, 2, 4, 8), then max of the two column halves;
  //   sum: each lane folds exp(z - m) over j = 0..7 ascending from +0, xor
  //        butterfly over the 16 lanes, then (half 0) + (half 1).
  // Columns >= v are -inf (they add +0).
  float rowmax[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float m = -INFINITY;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int64_t col = v0 + wn * 128 + j * 16 + li;
        m = fmaxf(m, col < v ? acc[i][j][q] : -INFINITY);
      }
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
      rowmax[i][q] = m;
    }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (li == 0) sm.red[wn][wm * 64 + i * 16 + 4 * g + q] = rowmax[i][q];
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int lr = wm * 64 + i * 16 + 4 * g + q;
      rowmax[i][q] = fmaxf(sm.red[0][lr], sm.red[1][lr]);
    }
  __syncthreads();
  float rowsum[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float m = rowmax[i][q];
      float s = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int64_t col = v0 + wn * 128 + j * 16 + li;
        s = s + exp_sub(col < v ? acc[i][j][q] : -INFINITY, m);
      }
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) s = s + __shfl_xor(s, o, kWave);
      rowsum[i][q] = s;
    }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (li == 0) sm.red[wn][wm * 64 + i * 16 + 4 * g + q] = rowsum[i][q];
  __syncthreads();
  if (wn == 0 && li == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int lr = wm * 64 + i * 16 + 4 * g + q;
        const int64_t r = m0 + lr;
        if (r < n && sm.target[lr] != ignore_index) {
          pm[static_cast<int64_t>(vb) * n + r] = rowmax[i][q];
          ps[static_cast<int64_t>(vb) * n + r] = sm.red[0][lr] + sm.red[1][lr];
        }
      }
  }
  // Target copy: the lane holding column t of row r writes z[r, t].
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int lr = wm * 64 + i * 16 + 4 * g + q;
      const int64_t r = m0 + lr;
      const int64_t t = sm.target[lr];
      if (r < n && t != ignore_index && t >= 0 && t < v && t >= v0 + wn * 128 &&
          t < v0 + wn * 128 + 128) {
        const int off = static_cast<int>(t - v0 - wn * 128);
        if (off % 16 == li) {
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (off / 16 == j) pt[r] = acc[i][j][q];
        }
      }
    }
}

void launch_linear_partials(const uint16_t* hidden, int64_t ld_h, const uint16_t* weight,
                            int64_t ld_w, int64_t n, int64_t h, int64_t v,
                            const int64_t* targets, int64_t ignore, float* pm, float* ps,
                            float* pt, hipStream_t s) {
  const int mblocks = static_cast<int>((n + BM - 1) / BM);
  const int vblocks = static_cast<int>((v + BN - 1) / BN);
  hipLaunchKernelGGL(linear_logp_stats_kernel, dim3(mblocks * vblocks), dim3(kThreads), 0, s,
                     hidden, ld_h, weight, ld_w, n, h, v, mblocks, vblocks, targets, ignore,
                     pm, ps, pt);
}

}  // namespace itl
