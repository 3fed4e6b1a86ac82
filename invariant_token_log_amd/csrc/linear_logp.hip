// Fused LM-head + logp statistics on gfx950 ("[RFC][ROCm] End-to-end
// optimization of bitwise VIME R/R beyond native P/P", Workstream 3: stream
// LM-head tiles through the matrix cores, take the local (max, sumexp,
// target) statistics and never store the [tokens, vocab] logits).
//
//   z[r, j] = sum_k hidden[r, k] * weight[j, k]
//
// Arithmetic (identical in both kernels below, so they give the same bits):
//   * every z[r, j] is one fp32 accumulator fed by v_mfma_f32_16x16x32_bf16
//     over K in ascending steps of 32, no split-K;
//   * the 256-column statistic tile of a row is cut into four quarters of 64
//     columns; column c of the tile is column group G = c / 16, lane li =
//     c % 16, quarter Q = G / 4.
//     max: exact (order-free);
//     sum: per lane, exp(z - m) folded over the quarter's 4 groups in
//          ascending order from +0; the xor-butterfly association over the 16
//          lanes (1, 2, 4, 8) gives the quarter sum q_Q; s = (q0 + q1) + (q2 + q3);
//     columns >= v are -inf and add +0;
//   * the target logit is the accumulator itself, copied by the lane that
//     holds it.
// A row's z, m, s and target logit therefore depend only on that row of
// hidden, the weight and K: not on N, the row's position, the block shape or
// the grid.
//
// Two kernels share this contract:
//   * linear_stats_dma (N > 128): the 256 x 256 MFMA tile of mfma_gemm.h,
//     eight waves of 128 x 64 (two per SIMD, so each hides the other's LDS
//     and barrier latency), operands streamed global -> LDS by direct 16-byte
//     LDS loads through a four-stage ring;
//   * linear_stats_narrow<64 / 128> (N <= 64 / N <= 128): the narrow tiles
//     of mfma_gemm.h, eight waves of 16 / 32 x 128, the same direct loads
//     (few rows give little arithmetic per weight byte, so these tiles are
//     bound by the bytes they keep in flight).
#include <atomic>
#include <type_traits>

#include "launch.h"
#include "logp_device.h"
#include "mfma_gemm.h"

namespace itl {

namespace {

using gemm::f32x4;
using gemm::tile_coords;
using gemm::xcd_logical;

constexpr int BN = kLinearTile;  // vocabulary columns per workgroup (= statistic tile)
constexpr int BK = gemm::kK;     // K per MFMA step

template <int BM>
struct Reduce {
  float red[BM][4];  // per-row quarter maxima
  float sum[BM][4];  // per-row quarter sums
  float wsum[BM][4]; // per-row quarter entropy moments (when requested)
  float tmax[BM];    // per-row tile maximum
  float tval[BM];    // target logit, when the target column is in this block
  int code[BM];      // row_code() of each row
};

// Per-row code for the epilogue: -2 = no statistics (row past n, or its
// target is ignore_index), -1 = target column outside this vocabulary block,
// else the target column minus v0.
__device__ __forceinline__ int row_code(int64_t r, int64_t n, Targets targets,
                                        int64_t ignore_index, int64_t v0, int64_t v) {
  if (r >= n) return -2;
  const int64_t t = targets[r];
  if (t == ignore_index) return -2;
  return (t >= v0 && t < v0 + BN && t < v) ? static_cast<int>(t - v0) : -1;
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS
// operations, not for its outstanding global loads or stores.
__device__ __forceinline__ void block_sync_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Statistic epilogue.  The wave holds acc[i][j][q] =
//   z[m0 + row0 + i*16 + 4g + q][v0 + col0 + j*16 + li],  j < NJ,
// where its NJ column groups form NJ / 4 whole quarters starting at quarter
// col0 / 64.  NT = threads of the workgroup.  rd.code must be filled, and
// accumulators of columns >= v must already hold -inf.
template <int MI, int NJ, int BM, int NT, bool ENT>
__device__ __forceinline__ void stats_epilogue_body(const f32x4 (&acc)[MI][NJ], Reduce<BM>& rd,
                                                    int row0, int col0, int li, int g, int tid,
                                                    int64_t m0, int64_t v0, int vb, int vblocks,
                                                    int64_t v, float* pm, float* ps, float* pw,
                                                    float* pt) {
  constexpr int NQ = NJ / 4;  // quarters held by this wave
  const int q0 = col0 / 64;
  auto z = [&](int i, int j, int q) { return acc[i][j][q]; };

  // Pass 1: quarter maxima (exact, order-free).
  float part[MI][4][NQ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int h = 0; h < NQ; ++h) {
        float m = z(i, 4 * h, q);
#pragma unroll
        for (int j = 4 * h + 1; j < 4 * h + 4; ++j) m = max_exact(m, z(i, j, q));
        part[i][q][h] = row16_max_first(m);
      }
  if (li == 0) {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int h = 0; h < NQ; ++h) rd.red[row0 + i * 16 + 4 * g + q][q0 + h] = part[i][q][h];
  }
  block_sync_lds();
  for (int lr = tid; lr < BM; lr += NT) {
    const float4 r4 = *reinterpret_cast<const float4*>(rd.red[lr]);
    rd.tmax[lr] = max_exact(max_exact(r4.x, r4.y), max_exact(r4.z, r4.w));
  }
  block_sync_lds();

  // Pass 2.  The lane's rows are 4 consecutive rows per row group i, so their
  // codes and tile maxima come in as one 16-byte LDS read per group, all
  // issued before any use.  First the target copies: the one lane holding
  // the target column of a row parks z[r, t] in LDS.  A wave's 64 columns
  // hold a target only now and then, so the hit tests run branch-free and
  // one wave-uniform branch enters the copy only when some lane has a hit.
  // Then the quarter sums against the tile maximum (and, with ENT, the
  // entropy moments sum e (z - m), same tree) as one branch-free block, so
  // that the exponentials of all row groups interleave.
  int4 code4[MI];
  float4 m4[MI];
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    const int lr = row0 + i * 16 + 4 * g;
    code4[i] = *reinterpret_cast<const int4*>(&rd.code[lr]);
    m4[i] = *reinterpret_cast<const float4*>(&rd.tmax[lr]);
  }
  // 1 when this lane holds the target column of a row with this code (the
  // code is -1 or -2 for rows whose target is elsewhere or absent)
  auto holds_target = [&](int code) {
    const unsigned off = static_cast<unsigned>(code - col0);
    return static_cast<int>(off < static_cast<unsigned>(NJ * 16)) &
           static_cast<int>((off & 15u) == static_cast<unsigned>(li));
  };
  int any_hit = 0;
#pragma unroll
  for (int i = 0; i < MI; ++i)
    any_hit |= holds_target(code4[i].x) | holds_target(code4[i].y) | holds_target(code4[i].z) |
               holds_target(code4[i].w);
  if (__builtin_amdgcn_ballot_w64(any_hit != 0)) {
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int c4[4] = {code4[i].x, code4[i].y, code4[i].z, code4[i].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (holds_target(c4[q])) {
          const int off = c4[q] - col0;
          float zt = acc[i][0][q];
#pragma unroll
          for (int j = 1; j < NJ; ++j)
            if ((off >> 4) == j) zt = acc[i][j][q];
          rd.tval[row0 + i * 16 + 4 * g + q] = zt;
        }
      }
    }
  }
  float wpart[ENT ? MI : 1][4][NQ];
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    const float mq[4] = {m4[i].x, m4[i].y, m4[i].z, m4[i].w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float m = mq[q];
#pragma unroll
      for (int h = 0; h < NQ; ++h) {
        if constexpr (ENT) {
          float s = 0.0f, w = 0.0f;
#pragma unroll
          for (int j = 4 * h; j < 4 * h + 4; ++j) {
            const float d = z(i, j, q) - m;  // exp_sub(z, m) in two steps
            const float e = __builtin_amdgcn_exp2f(d * kLog2e);
            s = j == 4 * h ? e : s + e;
            w = ent_term(e, d, w);
          }
          part[i][q][h] = row16_sum_first(s);
          wpart[i][q][h] = row16_sum_first(w);
        } else {
          float s = exp_sub(z(i, 4 * h, q), m);
#pragma unroll
          for (int j = 4 * h + 1; j < 4 * h + 4; ++j) s = s + exp_sub(z(i, j, q), m);
          part[i][q][h] = row16_sum_first(s);
        }
      }
    }
  }
  if (li == 0) {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int h = 0; h < NQ; ++h) {
          rd.sum[row0 + i * 16 + 4 * g + q][q0 + h] = part[i][q][h];
          if constexpr (ENT) rd.wsum[row0 + i * 16 + 4 * g + q][q0 + h] = wpart[i][q][h];
        }
  }
  block_sync_lds();

  for (int lr = tid; lr < BM; lr += NT) {
    const int code = rd.code[lr];
    if (code != -2) {
      const int64_t r = m0 + lr;
      const float4 s4 = *reinterpret_cast<const float4*>(rd.sum[lr]);
      pm[r * vblocks + vb] = rd.tmax[lr];
      ps[r * vblocks + vb] = (s4.x + s4.y) + (s4.z + s4.w);
      if constexpr (ENT) {
        const float4 w4 = *reinterpret_cast<const float4*>(rd.wsum[lr]);
        pw[r * vblocks + vb] = (w4.x + w4.y) + (w4.z + w4.w);
      }
      if (code >= 0) pt[r] = rd.tval[lr];
    }
  }
}

// Options of the forward statistic kernels: the logits' rounding point, the
// temperature's reciprocal (logits are multiplied by it before any
// statistic), the entropy moment table and the unscaled logits.
struct LinearExtras {
  float inv_t;      // 1 = no temperature
  int32_t round_bf16;  // 1 = z is RNE_bf16 of the accumulator
  float* pw;        // [n, T] entropy moments, or null
  void* z;          // [n, ld_z] unscaled logits (fp32 or bf16), or null
  int32_t z_bf16;
  int64_t ld_z;
  int32_t z_vec;    // z and its rows are 16-byte aligned: staged 16-byte stores
};

// Logits output through LDS: the tile's accumulators go to `scratch` (the
// main loop's stages, free by now) a row chunk at a time, then leave as
// whole 16-byte pieces along the rows (the accumulator layout would store
// 4 or 2 bytes per lane).  RPC rows per chunk: the largest power-of-two part
// of the tile that fits.
template <typename E, int MI, int NJ, int BM, int NT, int SCRATCH>
__device__ __forceinline__ void store_logits_staged(const f32x4 (&acc)[MI][NJ], void* scratch,
                                                    int row0, int col0, int li, int g, int tid,
                                                    int64_t m0, int64_t v0, int64_t n,
                                                    int64_t v, E* z, int64_t ld_z) {
  constexpr int kPer = 16 / static_cast<int>(sizeof(E));  // elements per 16-byte piece
  constexpr int kStride = BN + kPer;                       // padded LDS row
  constexpr int kRowBytes = kStride * static_cast<int>(sizeof(E));
  constexpr int RPC = BM * kRowBytes <= SCRATCH       ? BM
                      : BM / 2 * kRowBytes <= SCRATCH ? BM / 2
                      : BM / 4 * kRowBytes <= SCRATCH ? BM / 4
                                                      : BM / 8;
  static_assert(RPC * kRowBytes <= SCRATCH && RPC % 16 == 0, "logits chunk does not fit");
  E* tile = static_cast<E*>(scratch);
  for (int c = 0; c < BM / RPC; ++c) {
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int lr0 = row0 + i * 16 - c * RPC;  // uniform
      if (lr0 < 0 || lr0 >= RPC) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const float x = acc[i][j][q];
          E e;
          if constexpr (sizeof(E) == 2)
            e = __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
          else
            e = x;
          tile[(lr0 + 4 * g + q) * kStride + col0 + j * 16 + li] = e;
        }
    }
    __syncthreads();
    constexpr int kCpr = BN / kPer;  // pieces per row
    for (int idx = tid; idx < RPC * kCpr; idx += NT) {
      const int lr = idx / kCpr, pc = (idx % kCpr) * kPer;
      const int64_t r = m0 + c * RPC + lr, col = v0 + pc;
      if (r >= n) continue;
      E* dst = z + r * ld_z + col;
      const E* src = tile + lr * kStride + pc;
      if (col + kPer <= v) {
        *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
      } else {
        for (int u = 0; u < kPer; ++u)
          if (col + u < v) dst[u] = src[u];
      }
    }
    __syncthreads();
  }
}

template <int MI, int NJ, int BM, int NT, int SCRATCH>
__device__ __forceinline__ void stats_epilogue(f32x4 (&acc)[MI][NJ], Reduce<BM>& rd, void* scratch,
                                               int row0, int col0, int li, int g, int tid,
                                               int64_t m0, int64_t v0, int vb, int vblocks,
                                               int64_t n, int64_t v, float* pm, float* ps,
                                               float* pt, const LinearExtras& ex) {
  // The bf16-rounded variant: z becomes RNE_bf16(accumulator), widened
  // exactly, before anything reads it (logits output, temperature, every
  // statistic and the target copy).
  if (ex.round_bf16) {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          acc[i][j][q] = static_cast<float>(static_cast<__bf16>(acc[i][j][q]));
  }
  // The unscaled logits, when asked for: they are the accumulators as they
  // are (the statistics below do not change them).
  if (ex.z && ex.z_vec) {
    if (ex.z_bf16)
      store_logits_staged<uint16_t, MI, NJ, BM, NT, SCRATCH>(acc, scratch, row0, col0, li, g, tid,
                                                             m0, v0, n, v,
                                                             static_cast<uint16_t*>(ex.z), ex.ld_z);
    else
      store_logits_staged<float, MI, NJ, BM, NT, SCRATCH>(acc, scratch, row0, col0, li, g, tid, m0,
                                                          v0, n, v, static_cast<float*>(ex.z),
                                                          ex.ld_z);
  } else if (ex.z) {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t r = m0 + row0 + i * 16 + 4 * g + q;
        if (r >= n) continue;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int64_t c = v0 + col0 + j * 16 + li;
          if (c >= v) continue;
          if (ex.z_bf16)
            static_cast<uint16_t*>(ex.z)[r * ex.ld_z + c] =
                __builtin_bit_cast(uint16_t, static_cast<__bf16>(acc[i][j][q]));
          else
            static_cast<float*>(ex.z)[r * ex.ld_z + c] = acc[i][j][q];
        }
      }
  }
  // Temperature: x = z * (1 / T) on every accumulator before any statistic.
  if (ex.inv_t != 1.0f) {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[i][j] = acc[i][j] * ex.inv_t;
  }
  // Columns >= v exist only in the last vocabulary block.  Their -inf takes
  // no part in a maximum and adds an exact 0 to a sum; no target lies there.
  if (v0 + BN > v) {
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      if (v0 + col0 + j * 16 + li >= v)
#pragma unroll
        for (int i = 0; i < MI; ++i) acc[i][j] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  }
  if (ex.pw)
    stats_epilogue_body<MI, NJ, BM, NT, true>(acc, rd, row0, col0, li, g, tid, m0, v0, vb,
                                              vblocks, v, pm, ps, ex.pw, pt);
  else
    stats_epilogue_body<MI, NJ, BM, NT, false>(acc, rd, row0, col0, li, g, tid, m0, v0, vb,
                                               vblocks, v, pm, ps, ex.pw, pt);
}

// ---------------------------------------------------------------------------
// linear_stats_dma: BM = 256, the mfma_gemm.h tile (hidden rows x weight rows),
// statistic epilogue on its accumulators.
// ---------------------------------------------------------------------------
constexpr int kDmaThreads = gemm::kThreads;

// One LDS object per kernel, the stage ring first: a second __shared__
// variable moves the ring off the start of LDS, which measured 23% slower.
struct SmemDma {
  gemm::Stages st;  // 128 KiB
  Reduce<256> rd;
  int slot;         // tile-queue broadcast
};

// hidden K32-blocked (mblocks * 256 rows); weight row-major, or K32-blocked
// with round_up(v, 256) rows when WBLK (a prepared weight).  The grid covers
// vocabulary blocks [0, vtiles) of the vblocks that index the partial
// tables.  Tiles come from the mfma_gemm.h tile queue (counters `queue`, zero
// at launch; `queued` and the grid from queue_plan).
template <bool WBLK>
__global__ __launch_bounds__(kDmaThreads) void linear_stats_dma(
    const uint16_t* __restrict__ hidden, int64_t ld_h, const uint16_t* __restrict__ weight,
    int64_t ld_w, int64_t n, int64_t hdim, int64_t v, int mblocks, int vblocks, int vtiles,
    const void* __restrict__ tgt, int32_t tgt32, int64_t ignore_index, float* __restrict__ pm,
    float* __restrict__ ps, float* __restrict__ pt, LinearExtras ex, int* queue, int queued) {
  const Targets targets{tgt, tgt32};
  __shared__ __align__(16) SmemDma sm;
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wave / 4, wn = wave % 4;
  const int li = lane % 16, g = lane / 16;

  const int logical = gemm::queue_tile(queue, mblocks * vtiles, queued, &sm.slot);
  if (logical < 0) return;
  int mb, vb;
  tile_coords(logical, mblocks, vtiles, mb, vb);
  const int64_t m0 = static_cast<int64_t>(mb) * 256;
  const int64_t v0 = static_cast<int64_t>(vb) * BN;
  if (tid < 256) sm.rd.code[tid] = row_code(m0 + tid, n, targets, ignore_index, v0, v);

  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  const int ksteps = static_cast<int>(hdim / BK);
  const int64_t kblk = static_cast<int64_t>(ksteps) * 512;  // blocked: 16-row block stride
  gemm::mainloop<true, WBLK>(sm.st, hidden, kblk, m0, static_cast<int64_t>(mblocks) * 256, weight,
                             WBLK ? kblk : ld_w, v0, WBLK ? static_cast<int64_t>(vblocks) * BN : v,
                             ksteps, acc);
  __syncthreads();
  stats_epilogue<8, 4, 256, kDmaThreads, sizeof(sm.st)>(acc, sm.rd, &sm.st, wm * 128, wn * 64, li,
                                                        g, tid, m0, v0, vb,
                                         vblocks, n, v, pm, ps, pt, ex);
}

// ---------------------------------------------------------------------------
// linear_stats_narrow<ROWS>: the narrow mfma_gemm.h tiles for few hidden rows
// (N <= 64: ROWS = 64, two workgroups per CU; N <= 128: ROWS = 128), and for
// the last vocabulary blocks of a larger N (below); same K walk and epilogue
// tree as linear_stats_dma, so a row gets the same bits on every path.  hidden
// row-major [n, ld_h], mblocks = ceil(n / ROWS) row blocks; the grid covers
// vocabulary blocks [vb0, vb0 + vtiles).
// ---------------------------------------------------------------------------
// WBLK: the stage ring of mainloop_narrow; row-major weight: the NPS pair
// slots of mainloop_narrow_pairs.
template <int ROWS, bool WBLK, int NPS, int S>
struct SmemNarrow {
  typename std::conditional<WBLK, gemm::StagesNarrow<ROWS, S>,
                            gemm::StagesNarrowPairs<ROWS, NPS>>::type st;
  Reduce<ROWS> rd;
};

// Row-major weight pair slots of the narrow tiles: 4 for 64 rows (144 KiB,
// the whole LDS of a CU: three pairs in flight), 2 for 128 rows.  A
// prepared weight's ring: NarrowCfg's stages, or with DEEP (64 rows only,
// for launches of at most one workgroup per CU) seven (140 KiB, six in
// flight).
template <int ROWS>
constexpr int kNarrowPairs = ROWS == 64 ? 4 : 2;
template <int ROWS, bool DEEP>
constexpr int kNarrowStages = DEEP ? 7 : gemm::NarrowCfg<ROWS>::kStages;

template <int ROWS, bool WBLK, bool NTB = false, bool DEEP = false>
__global__ __launch_bounds__(kDmaThreads) void linear_stats_narrow(
    const uint16_t* __restrict__ hidden, int64_t ld_h, const uint16_t* __restrict__ weight,
    int64_t ld_w, int64_t n, int64_t hdim, int64_t v, int mblocks, int vblocks, int vb0,
    int vtiles,
    const void* __restrict__ tgt, int32_t tgt32, int64_t ignore_index, float* __restrict__ pm,
    float* __restrict__ ps, float* __restrict__ pt, LinearExtras ex) {
  constexpr int MI = gemm::NarrowCfg<ROWS>::kMI;
  const Targets targets{tgt, tgt32};
  __shared__ __align__(16) SmemNarrow<ROWS, WBLK, kNarrowPairs<ROWS>, kNarrowStages<ROWS, DEEP>> sm;
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wave / 4, wn = wave % 4;
  const int li = lane % 16, g = lane / 16;

  const int logical = xcd_logical(blockIdx.x, mblocks * vtiles);
  const int mb = logical % mblocks;
  const int vb = vb0 + logical / mblocks;
  const int64_t m0 = static_cast<int64_t>(mb) * ROWS;
  const int64_t v0 = static_cast<int64_t>(vb) * BN;
  if (tid < ROWS) sm.rd.code[tid] = row_code(m0 + tid, n, targets, ignore_index, v0, v);

  f32x4 acc[MI][4];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  const int ksteps = static_cast<int>(hdim / BK);
  if constexpr (WBLK)
    gemm::mainloop_narrow<ROWS, true, NTB, kNarrowStages<ROWS, DEEP>>(sm.st, hidden, ld_h, m0, n, weight,
                                           static_cast<int64_t>(ksteps) * 512, v0,
                                           static_cast<int64_t>(vblocks) * BN, ksteps, acc);
  else
    gemm::mainloop_narrow_pairs<ROWS, NTB, kNarrowPairs<ROWS>>(sm.st, hidden, ld_h, m0, n, weight, ld_w, v0, v,
                                           ksteps, acc);
  __syncthreads();
  stats_epilogue<MI, 4, ROWS, kDmaThreads, sizeof(sm.st)>(acc, sm.rd, &sm.st, wm * (ROWS / 2),
                                                          wn * 64, li, g, tid,
                                           m0, v0, vb, vblocks, n, v, pm, ps, pt, ex);
}

}  // namespace

void launch_linear_partials(const uint16_t* hidden, int64_t ld_h, const uint16_t* weight,
                            int64_t ld_w, int64_t n, int64_t h, int64_t v, Targets targets,
                            int64_t ignore, float* pm, float* ps, float* pt, float inv_t,
                            int32_t round_bf16, float* pw, void* z, int32_t z_bf16, int64_t ld_z,
                            const uint16_t* wblk, uint16_t* hb, hipStream_t s) {
  const int vblocks = static_cast<int>((v + BN - 1) / BN);
  const int32_t z_vec = z && reinterpret_cast<uintptr_t>(z) % 16 == 0 &&
                        (ld_z * (z_bf16 ? 2 : 4)) % 16 == 0;
  const LinearExtras ex{inv_t, round_bf16, pw, z, z_bf16, ld_z, z_vec};
  // the narrow tiles read a prepared (K32-blocked) weight when there is one
  const uint16_t* wn = wblk ? wblk : weight;
  const int64_t ldn = wblk ? 0 : ld_w;
  // once: every weight row is read by one workgroup only (a single row
  // block), so the weight streams with non-temporal loads
  auto narrow = [&](int rows, int mb, int vb0, int vt, bool once, bool deep) {
    auto kern = rows == 64
                    ? (wblk ? (once ? linear_stats_narrow<64, true, true>
                               : deep ? linear_stats_narrow<64, true, false, true>
                                    : linear_stats_narrow<64, true, false>)
                            : (once ? linear_stats_narrow<64, false, true>
                                    : linear_stats_narrow<64, false, false>))
                    : (wblk ? (once ? linear_stats_narrow<128, true, true>
                                    : linear_stats_narrow<128, true, false>)
                            : (once ? linear_stats_narrow<128, false, true>
                                    : linear_stats_narrow<128, false, false>));
    hipLaunchKernelGGL(kern, dim3(mb * vt), dim3(kDmaThreads), 0, s, hidden, ld_h, wn, ldn, n, h,
                       v, mb, vblocks, vb0, vt, targets.p, targets.is32, ignore, pm, ps, pt, ex);
  };
  if (n <= 128) {
    narrow(n <= 64 ? 64 : 128, 1, 0, vblocks, true, false);
  } else {
    const int mblocks = static_cast<int>((n + 255) / 256);
    const int64_t np = static_cast<int64_t>(mblocks) * 256;
    // Last round: when the 256 x 256 tiles leave the final round at most a
    // quarter full, the last `tail` vocabulary blocks go to the 64-row tile
    // instead (four times as many, four times smaller, the same bits), so
    // that round spreads over the GPU.
    const int cus = xcd_cus() * 8, tiles = mblocks * vblocks, rem = tiles % cus;
    int tail = 0;
    if (rem != 0 && rem <= cus / 4 && tiles > cus) tail = (rem + mblocks - 1) / mblocks;
    const int vmain = vblocks - tail;
    // the tile-queue counters follow the blocked hidden; block_rows clears them
    int* queue = reinterpret_cast<int*>(hb + np * h);
    launch_block_rows(hidden, ld_h, n, np, h, hb, s, queue, gemm::kQueueBytes / 4);
    const gemm::QueuePlan qp = gemm::queue_plan(mblocks * vmain, xcd_cus());
    const dim3 grid(static_cast<unsigned>(qp.grid));
    if (wblk)
      hipLaunchKernelGGL(linear_stats_dma<true>, grid, dim3(kDmaThreads), 0, s, hb, ld_h, wblk,
                         int64_t{0}, n, h, v, mblocks, vblocks, vmain, targets.p, targets.is32,
                         ignore, pm, ps, pt, ex, queue, qp.queued);
    else
      hipLaunchKernelGGL(linear_stats_dma<false>, grid, dim3(kDmaThreads), 0, s, hb, ld_h, weight,
                         ld_w, n, h, v, mblocks, vblocks, vmain, targets.p, targets.is32, ignore,
                         pm, ps, pt, ex, queue, qp.queued);
    // a tail of at most one workgroup per CU takes the deep ring
    const int tmb = static_cast<int>((n + 63) / 64);
    if (tail) narrow(64, tmb, vmain, tail, false, static_cast<int64_t>(tmb) * tail <= cus);
  }
}

int xcd_cus() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices];  // 0 = not looked up yet
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 32;
  int c = cache[dev].load(std::memory_order_relaxed);
  if (c == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus < 8)
      cus = 256;
    c = cus / 8;
    cache[dev].store(c, std::memory_order_relaxed);
  }
  return c;
}

int64_t linear_fwd_blocked_bytes(int64_t n, int64_t h) {
  return n > 128 ? (n + 255) / 256 * 256 * h * 2 + gemm::kQueueBytes : 0;
}

}  // namespace itl
