// 256 x 256 bf16 MFMA tile of C = A * B^T (operands K-contiguous, or read
// K-outer through transposed LDS reads), the product engine of the fused LM
// head and of its backward.
//
// Arithmetic (part of the fused-LM-head contract): every output is one fp32
// accumulator fed by v_mfma_f32_16x16x32_bf16 over K in ascending steps of
// 32, no split-K.  The accumulator may start from a caller-supplied value;
// continuing a K walk from a stored accumulator gives the same bits as one
// uninterrupted walk.
//
// Layout: 8 waves; wave w covers rows (w / 4) * 128 + [0, 128) and columns
// (w % 4) * 64 + [0, 64) of the tile as acc[i][j][q] =
//   C[row0 + i*16 + 4*g + q][col0 + j*16 + li],   li = lane % 16, g = lane / 16.
// Operands stream global -> LDS by direct 16-byte loads through a four-stage
// ring (three K steps in flight).  LDS stage layout: [A | B], each 256 rows x
// 32 bf16 (64 B per row, 16 KiB); 16-byte chunk kc of row r sits in slot
// kc ^ swz(r), swz(r) = ((r >> 1) ^ (r >> 2)) & 3, so the 16 rows of a
// fragment read (one 16-byte chunk per row) spread over all banks.  One
// direct load instruction fills 1 KiB = 16 rows: lane L writes row L / 4,
// slot L % 4, so it fetches chunk (L % 4) ^ swz(L / 4) of its row.  Waves
// 0-3 fill the stages: wave w loads A and B blocks w, w + 4, w + 8, w + 12.
//
// Operand layouts.  Row-major: element (r, k) at r * ld + k.  K32-blocked
// (kblocked_index): the 16 rows x 32 K piece that one direct load
// instruction fills is one contiguous KiB, element (r, k) at
// ((r / 16) * ksteps + k / 32) * 512 + (r % 16) * 32 + k % 32, rows padded to
// a multiple of 16 with zeros; a product may read the K range [k0, k0 + K)
// of a wider blocked operand by starting at its piece k0 / 32 and passing
// ksteps * 512 (the operand's full width) as the distance between 16-row
// blocks.  A blocked operand makes every load
// instruction read eight whole 128-byte lines instead of sixteen half lines
// (measured: 9% more MFMA throughput with both operands blocked).  The layout
// moves bytes only, so the products have the same bits.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace itl {
namespace gemm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kTile = 256;     // rows and columns of a workgroup tile
constexpr int kK = 32;         // K per MFMA step
constexpr int kThreads = 512;  // 8 waves
constexpr int kStages = 4;
constexpr int kStageElems = kTile * kK;  // bf16 per operand per stage

struct Stages {
  uint16_t s[kStages][2][kStageElems];  // 128 KiB
};

// Workgroups are dealt round-robin to the 8 XCDs; give each XCD one
// contiguous range of logical tiles so that an operand slice is read into one
// XCD's L2 only.
__device__ __forceinline__ int xcd_logical(int b, int g) {
  const int x = b % 8, y = b / 8, per = g / 8, rem = g % 8;
  return x < rem ? x * (per + 1) + y : rem * (per + 1) + (x - rem) * per + y;
}

// Logical tile -> (row block, column block).  Tiles are grouped 8 row blocks
// x 4 column blocks, so the ~32 workgroups an XCD runs at once share each A
// slice 4 ways and each B slice 8 ways in its L2.
__device__ __forceinline__ void tile_coords(int logical, int mblocks, int nblocks, int& mb,
                                            int& nb) {
  const int nbg = logical / (mblocks * 4);
  const int gn = min(4, nblocks - nbg * 4);
  const int rem = logical - nbg * mblocks * 4;
  const int mbg = rem / (8 * gn);
  const int gm = min(8, mblocks - mbg * 8);
  const int r2 = rem - mbg * 8 * gn;
  mb = mbg * 8 + r2 % gm;
  nb = nbg * 4 + r2 / gm;
}

// Logical tiles [first, last) of XCD x under xcd_logical's split of g tiles.
__host__ __device__ __forceinline__ void xcd_range(int g, int x, int& first, int& last) {
  const int per = g / 8, rem = g % 8;
  first = x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per;
  last = first + per + (x < rem ? 1 : 0);
}

// ---------------------------------------------------------------------------
// Tile queue.  The XCDs of one GPU do not run at the same speed (clocks and
// memory paths differ), so with a static split the fastest XCD idles while
// the slowest finishes its range.  Instead, the last `queued` tiles of each
// XCD range are claimed at run time: workgroup b (XCD b % 8, slot b / 8)
// takes the slot-th tile of its range while slot < range - queued, as
// xcd_logical does; every later workgroup claims the next queued tile of its
// own range from that range's counter, and once those are gone the next
// queued tile of another range.  The grid carries `extra` workgroups per XCD
// beyond the tiles, so that a fast XCD has workgroups to take over a slow
// one's tail; a workgroup that finds every queue empty exits.  Each tile is
// computed exactly once, by one workgroup, with the same arithmetic: the
// schedule changes no bit of any output, whatever queued and extra are.
//
// The 8 counters sit 64 bytes apart (kQueueBytes) and must be zero when the
// kernel starts; kernels that use them are preceded, on the same stream, by
// a launch that clears them.  Claims are vector atomics.
// ---------------------------------------------------------------------------
constexpr int kQueued = 128;       // most queued tiles per XCD range
constexpr int kQueueExtra = 64;    // most extra workgroups per XCD
constexpr int kQueueStride = 16;   // ints between counters
constexpr int kQueueBytes = 8 * kQueueStride * 4;

struct QueuePlan {
  int queued;  // queued tiles per XCD range
  int extra;   // extra workgroups per XCD
  int grid;    // tiles + 8 * extra
};

// The first round of every XCD (xcd_cus workgroups, one per CU) stays
// static, since a single round has no tail to balance; of the rest, up to
// kQueued tiles per range are queued.
inline QueuePlan queue_plan(int tiles, int xcd_cus) {
  const int per = tiles / 8;
  int queued = per - xcd_cus;
  queued = queued < 0 ? 0 : queued > kQueued ? kQueued : queued;
  int extra = queued ? per / 8 : 0;
  extra = extra > kQueueExtra ? kQueueExtra : extra;
  return QueuePlan{queued, extra, tiles + 8 * extra};
}

__device__ __forceinline__ int queue_skip(int first, int last, int queued) {
  return last - first > queued ? last - first - queued : 0;
}

// Next queued tile for a workgroup of XCD x, or -1 (one lane calls it).
__device__ __forceinline__ int queue_claim(int* ctr, int x, int tiles, int queued) {
  for (int d = 0; d < 8; ++d) {
    const int y = (x + d) & 7;
    int first, last;
    xcd_range(tiles, y, first, last);
    const int s = queue_skip(first, last, queued);
    if (first + s >= last) continue;
    const int t = atomicAdd(ctr + y * kQueueStride, 1);
    if (first + s + t < last) return first + s + t;
  }
  return -1;
}

// This workgroup's logical tile, or -1 when it has none (the whole
// workgroup then returns).  slot: an int of the kernel's LDS for the
// broadcast.  All threads must call.
__device__ __forceinline__ int queue_tile(int* ctr, int tiles, int queued, int* slot) {
  const int x = blockIdx.x % 8, y = blockIdx.x / 8;
  int first, last;
  xcd_range(tiles, x, first, last);
  if (y < queue_skip(first, last, queued)) return first + y;
  if (threadIdx.x == 0) *slot = queue_claim(ctr, x, tiles, queued);
  __syncthreads();
  return *slot;
}

__device__ __forceinline__ int swz(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }

// Element (r, k) of a K32-blocked operand with ksteps = K / 32.
__host__ __device__ constexpr int64_t kblocked_index(int64_t r, int64_t k, int64_t ksteps) {
  return ((r >> 4) * ksteps + (k >> 5)) * 512 + (r & 15) * 32 + (k & 31);
}

// This lane's chunk of 16-row block `blk` (counted from row0, a multiple of
// 16) of an operand at K step 0.  ld: elements between rows (row-major) or
// between 16-row blocks (K32-blocked).  Rows at or past `rows` are read from
// the last valid row (row-major) or the last 16-row block (K32-blocked, whose
// rows are padded to a multiple of 16): every load stays in bounds, and those
// rows only feed outputs the caller masks.
template <bool BLOCKED>
__device__ __forceinline__ const uint16_t* lane_chunk(const uint16_t* X, int64_t ld,
                                                      int64_t row0, int64_t rows, int blk,
                                                      int lrow, int lk) {
  if constexpr (BLOCKED)
    return X + min(row0 / 16 + blk, (rows + 15) / 16 - 1) * ld + lrow * 32 + lk;
  else
    return X + min(row0 + blk * 16 + lrow, rows - 1) * ld + lk;
}

// s_waitcnt vmcnt(N) with N a template constant.
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(N) : "memory");
}

// Direct loads of one operand by a loader wave: blocks wave + 4u (u < 4) of
// its 16-row blocks.  K32-blocked: the blocks' element offsets are uniform
// (scalar registers) and the lane adds its place in the 1 KiB piece;
// row-major: one lane pointer per block (lane_chunk).  `at` gives the lane's
// source at K step 0 plus k elements.
template <bool BLOCKED>
struct LoaderSrc {
  const uint16_t* p[4];
  int lofs;
  __device__ __forceinline__ void init(const uint16_t* X, int64_t ld, int64_t row0, int64_t rows,
                                       int wave, int lrow, int lk) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if constexpr (BLOCKED)
        p[u] = X + min(row0 / 16 + wave + 4 * u, (rows + 15) / 16 - 1) * ld;
      else
        p[u] = lane_chunk<false>(X, ld, row0, rows, wave + 4 * u, lrow, lk);
    }
    lofs = lrow * 32 + lk;
  }
  __device__ __forceinline__ const uint16_t* at(int u, int64_t k) const {
    return BLOCKED ? p[u] + k + lofs : p[u] + k;
  }
};

// Waves 0-3 (one per SIMD) issue all 32 direct loads of a K step (16 A and
// 16 B blocks, 8 per wave) at the start of the step; waves 4-7 issue none,
// so they never wait behind the memory pipeline and on every SIMD one wave
// keeps the matrix core fed while the other queues its loads (measured on
// the bare 256 x 256 product: 6% more throughput than 4 loads from every
// wave spread over the step).
constexpr int kLoaderWaves = 4;
constexpr int kLoaderLoads = 8;  // per loader wave per K step

// A loader wave's 8 direct loads of K step `step` into LDS stage `s`; SA,
// SB: elements between consecutive K steps of one lane's A / B chunk (32
// row-major, 512 K32-blocked).
template <int SA, int SB, bool ABLK, bool BBLK>
__device__ __forceinline__ void issue_loads(Stages& sm, const LoaderSrc<ABLK>& sa,
                                            const LoaderSrc<BBLK>& sb, int wave, int s, int step) {
  constexpr int kBlk = 16 * kK;  // elements per 16-row block
  const int64_t ka = static_cast<int64_t>(step) * SA, kb = static_cast<int64_t>(step) * SB;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    __builtin_amdgcn_global_load_lds(sa.at(u, ka), sm.s[s][0] + (wave + 4 * u) * kBlk, 16, 0, 0);
    __builtin_amdgcn_global_load_lds(sb.at(u, kb), sm.s[s][1] + (wave + 4 * u) * kBlk, 16, 0, 0);
  }
}

// The main loop as run by one role: LOADER for waves 0-3, which issue the
// direct loads, else waves 4-7.  The two roles run different instruction
// orders: a loader issues its 8 loads right after the step's barrier and
// then interleaves fragment reads with MFMAs; the others are free to start
// on MFMAs the moment the barrier opens.  Every wave must call with its own
// role (mainloop does that); acc, the arguments and the result are as for
// mainloop.
// Row-major B in pairs of K steps.  A row-major B's 16-row x 32-K block
// spans half of sixteen 128-byte lines, so each direct load would fetch half
// lines; here B is staged two K steps at a time instead: 256 rows x 64 K (a
// "pair slot", row = 128 bytes, chunk c of row r in slot c ^ swzp(r), which
// keeps the 16 rows of a fragment read on distinct banks), each direct load
// filling 8 rows x 128 bytes, whole lines.  The 128 KiB of Stages hold A in
// four K32 slots (elements [0, 32768)) and B in two pair slots ([32768,
// 65536)).  Loader wave w issues A blocks w + 4u of every step (4 loads) and,
// on odd steps, rows (w + 4u) * 8 + [0, 8), u < 8, of the B pair two steps
// ahead (8 loads); the waits below count exactly those.  Same fragments, so
// the same bits (measured on the bare product: 1.45 -> 1.49 PFLOP/s).
__device__ __forceinline__ int swzp(int r) { return (r >> 1) & 7; }

template <bool ABLK, bool LOADER>
__device__ __forceinline__ void mainloop_pairs(Stages& sm, const uint16_t* __restrict__ A,
                                               int64_t lda, int64_t a_row0, int64_t a_rows,
                                               const uint16_t* __restrict__ B, int64_t ldb,
                                               int64_t b_row0, int64_t b_rows, int ksteps,
                                               f32x4 (&acc)[8][4]) {
  constexpr int SA = ABLK ? 512 : kK;
  constexpr int kPairElems = kTile * 2 * kK;   // one pair slot
  constexpr int kBBase = kStages * kStageElems;  // first pair slot
  uint16_t* const base = &sm.s[0][0][0];
  const int tid = threadIdx.x;
  const int lane = tid % 64;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int wm = wave / 4, wn = wave % 4;
  const int li = lane % 16, g = lane / 16;
  const int lrow = lane / 4;
  const int lk = ((lane % 4) ^ swz(lrow)) * 8;
  LoaderSrc<ABLK> sa;
  const uint16_t* bp[8];
  if constexpr (LOADER) {
    sa.init(A, lda, a_row0, a_rows, wave, lrow, lk);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int r = (wave + 4 * u) * 8 + lane / 8;  // tile row this lane fills
      bp[u] = B + min(b_row0 + r, b_rows - 1) * ldb + ((lane % 8) ^ swzp(r)) * 8;
    }
  }
  constexpr int kBlk = 16 * kK;  // elements per 1 KiB direct load
#define ITL_ISSUE_A(SLOT, STEP)                                                                 \
  if constexpr (LOADER) {                                                                       \
    const int64_t ka_ = static_cast<int64_t>(STEP) * SA;                                        \
    _Pragma("unroll") for (int u = 0; u < 4; ++u) __builtin_amdgcn_global_load_lds(             \
        sa.at(u, ka_), base + (SLOT) * kStageElems + (wave + 4 * u) * kBlk, 16, 0, 0);          \
  }
#define ITL_ISSUE_B(PSLOT, PAIR)                                                                \
  if constexpr (LOADER) {                                                                       \
    const int64_t kb_ = static_cast<int64_t>(PAIR) * 2 * kK;                                    \
    _Pragma("unroll") for (int u = 0; u < 8; ++u) __builtin_amdgcn_global_load_lds(             \
        bp[u] + kb_, base + kBBase + (PSLOT) * kPairElems + (wave + 4 * u) * kBlk, 16, 0, 0);   \
  }
  const int npairs = ksteps / 2;
  const int aoff = (wm * 128 + li) * kK + ((g ^ swz(li)) * 8);
  const int brow = wn * 64 + li;  // + 16 j; swzp(brow + 16 j) == swzp(li)
  const int bsw = swzp(li);
  constexpr int NA = LOADER ? 4 : 0, NB = LOADER ? 8 : 0;
  // Prologue = iterations -4 .. -1: each issues A of step it + 4, the odd ones
  // also the B pair (it + 3, it + 4).
  ITL_ISSUE_A(0, 0);
  ITL_ISSUE_A(1, 1 < ksteps ? 1 : ksteps - 1);
  ITL_ISSUE_B(0, 0);
  ITL_ISSUE_A(2, 2 < ksteps ? 2 : ksteps - 1);
  ITL_ISSUE_A(3, 3 < ksteps ? 3 : ksteps - 1);
  ITL_ISSUE_B(1, 1 < npairs ? 1 : npairs - 1);
  wait_vm<2 * NA + NB>();
  __builtin_amdgcn_s_barrier();
  bf16x8 xa[8], xb[4], ya[8], yb[4];
#define ITL_READ(FA, FB, STEP)                                                                  \
  {                                                                                             \
    const uint16_t* fa_ = base + ((STEP) % kStages) * kStageElems;                              \
    const uint16_t* fb_ = base + kBBase + (((STEP) / 2) % 2) * kPairElems;                      \
    const int ch_ = ((4 * ((STEP) % 2) + g) ^ bsw) * 8;                                         \
    _Pragma("unroll") for (int j = 0; j < 4; ++j)                                               \
      FB[j] = *reinterpret_cast<const bf16x8*>(fb_ + (brow + 16 * j) * 2 * kK + ch_);           \
    _Pragma("unroll") for (int i = 0; i < 8; ++i)                                               \
      FA[i] = *reinterpret_cast<const bf16x8*>(fa_ + aoff + i * 16 * kK);                       \
  }
  ITL_READ(xa, xb, 0)
  // Even iteration KT: A(KT+1) and the B pair (KT, KT+1), issued at KT-3,
  // have landed once at most A(KT-2), A(KT-1) and B(KT-1) are in flight; odd
  // KT: the B pair (KT+1, KT+2), issued at KT-2, once at most A(KT-1) is.
#define ITL_PSTEP(CA, CB, NXA, NXB, KT, ODD)                                                    \
  {                                                                                             \
    if constexpr (ODD)                                                                          \
      wait_vm_lgkm0<NA>();                                                                      \
    else                                                                                        \
      wait_vm_lgkm0<2 * NA + NB>();                                                             \
    __builtin_amdgcn_s_barrier();                                                               \
    ITL_ISSUE_A((KT) % kStages, (KT) + kStages < ksteps ? (KT) + kStages : ksteps - 1);         \
    if constexpr (ODD) {                                                                        \
      const int p_ = ((KT) + 3) / 2;                                                            \
      ITL_ISSUE_B(p_ % 2, p_ < npairs ? p_ : npairs - 1);                                       \
    }                                                                                           \
    ITL_READ(NXA, NXB, (KT) + 1)                                                                \
    _Pragma("unroll") for (int i = 0; i < 8; ++i)                                               \
      _Pragma("unroll") for (int j = 0; j < 4; ++j)                                             \
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(CA[i], CB[j], acc[i][j], 0, 0, 0);  \
    if constexpr (LOADER) __builtin_amdgcn_sched_group_barrier(0x020, ODD ? NA + NB : NA, 0);   \
    _Pragma("unroll") for (int u = 0; u < 12; ++u) {                                            \
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);                                        \
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                                        \
    }                                                                                           \
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);                                          \
  }
  for (int kt = 0; kt < ksteps; kt += 2) {
    ITL_PSTEP(xa, xb, ya, yb, kt, false)
    ITL_PSTEP(ya, yb, xa, xb, kt + 1, true)
  }
#undef ITL_PSTEP
#undef ITL_READ
#undef ITL_ISSUE_B
#undef ITL_ISSUE_A
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

template <bool ABLK, bool BBLK, bool LOADER>
__device__ __forceinline__ void mainloop_role(Stages& sm, const uint16_t* __restrict__ A,
                                              int64_t lda, int64_t a_row0, int64_t a_rows,
                                              const uint16_t* __restrict__ B, int64_t ldb,
                                              int64_t b_row0, int64_t b_rows, int ksteps,
                                              f32x4 (&acc)[8][4]) {
  if constexpr (!BBLK) {
    mainloop_pairs<ABLK, LOADER>(sm, A, lda, a_row0, a_rows, B, ldb, b_row0, b_rows, ksteps,
                                 acc);
    return;
  }
  constexpr int SA = ABLK ? 512 : kK, SB = BBLK ? 512 : kK;
  constexpr int NL = LOADER ? kLoaderLoads : 0;  // this wave's loads per step
  const int tid = threadIdx.x;
  const int lane = tid % 64;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int wm = wave / 4, wn = wave % 4;
  const int li = lane % 16, g = lane / 16;
  const int lrow = lane / 4;
  const int lk = ((lane % 4) ^ swz(lrow)) * 8;
  LoaderSrc<ABLK> sa;
  LoaderSrc<BBLK> sb;
  if constexpr (LOADER) {
    sa.init(A, lda, a_row0, a_rows, wave, lrow, lk);
    sb.init(B, ldb, b_row0, b_rows, wave, lrow, lk);
  }
#define ITL_ISSUE(S_, STEP_) \
  if constexpr (LOADER) issue_loads<SA, SB>(sm, sa, sb, wave, (S_), (STEP_))

  // Fragment offsets (elements) inside a stage: row wm*128 + li (+16 i) of A,
  // row wn*64 + li (+16 j) of B, chunk g.
  const int aoff = (wm * 128 + li) * kK + ((g ^ swz(li)) * 8);
  const int boff = (wn * 64 + li) * kK + ((g ^ swz(li)) * 8);

  // Pipeline.  Iteration kt runs the MFMAs of step kt on fragments already in
  // registers while the fragments of step kt+1 are read from LDS and the
  // direct loads of step kt+4 go out (steps kt+2, kt+3 are in flight).  Every
  // iteration issues the same loads per wave and 12 fragment reads, so the
  // wait counts are constant: past the end the loads re-fetch the last K step
  // into the stage that is no longer read, and the extra fragment reads land
  // in registers that are not used.
  for (int st = 0; st < kStages; ++st) ITL_ISSUE(st, st < ksteps ? st : ksteps - 1);
  wait_vm<(kStages - 1) * NL>();
  __builtin_amdgcn_s_barrier();
  bf16x8 xa[8], xb[4], ya[8], yb[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    xb[j] = *reinterpret_cast<const bf16x8*>(sm.s[0][1] + boff + j * 16 * kK);
#pragma unroll
  for (int i = 0; i < 8; ++i)
    xa[i] = *reinterpret_cast<const bf16x8*>(sm.s[0][0] + aoff + i * 16 * kK);
  // One step: this wave's reads of stage KT % 4 and (loader) its loads of
  // step KT+1 have landed (KT+2, KT+3 may still be in flight); after the
  // barrier step KT+1 is in LDS for every wave and stage KT % 4 is free.  A
  // bare s_barrier: the fence of __syncthreads would also wait for KT+2,
  // KT+3.  Order: the loads first (loader), then 12 x (2 MFMAs, 1 fragment
  // read), 8 MFMAs.
#define ITL_STEP(CA, CB, NA, NB, KT)                                                         \
  {                                                                                          \
    wait_vm_lgkm0<(kStages - 2) * NL>();                                                     \
    __builtin_amdgcn_s_barrier();                                                            \
    ITL_ISSUE((KT) % kStages, (KT) + kStages < ksteps ? (KT) + kStages : ksteps - 1);        \
    {                                                                                        \
      const uint16_t* fa = sm.s[((KT) + 1) % kStages][0];                                    \
      const uint16_t* fb = sm.s[((KT) + 1) % kStages][1];                                    \
      _Pragma("unroll") for (int j = 0; j < 4; ++j)                                          \
        NB[j] = *reinterpret_cast<const bf16x8*>(fb + boff + j * 16 * kK);                   \
      _Pragma("unroll") for (int i = 0; i < 8; ++i)                                          \
        NA[i] = *reinterpret_cast<const bf16x8*>(fa + aoff + i * 16 * kK);                   \
    }                                                                                        \
    _Pragma("unroll") for (int i = 0; i < 8; ++i)                                            \
      _Pragma("unroll") for (int j = 0; j < 4; ++j)                                          \
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(CA[i], CB[j], acc[i][j], 0, 0, 0); \
    if constexpr (LOADER) __builtin_amdgcn_sched_group_barrier(0x020, NL, 0);                \
    _Pragma("unroll") for (int u = 0; u < 12; ++u) {                                         \
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);                                     \
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                                     \
    }                                                                                        \
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);                                       \
  }
  for (int kt = 0; kt < ksteps; kt += 2) {
    ITL_STEP(xa, xb, ya, yb, kt)
    ITL_STEP(ya, yb, xa, xb, kt + 1)
  }
#undef ITL_STEP
#undef ITL_ISSUE
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// True for the waves that issue the direct loads (mainloop_role's LOADER).
__device__ __forceinline__ bool loader_wave() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x / 64) < kLoaderWaves;
}

// acc += A[a_row0 + 0..255, 0..K) * B[b_row0 + 0..255, 0..K)^T with K =
// ksteps * 32 (ksteps even, >= 2); ABLK / BBLK: the operand is K32-blocked
// and its lda / ldb is the distance between 16-row blocks in elements (512
// times the operand's K steps).  All 512 threads must call; on return every
// direct load has landed and the stages may be reused after a barrier.
template <bool ABLK = false, bool BBLK = false>
__device__ __forceinline__ void mainloop(Stages& sm, const uint16_t* __restrict__ A, int64_t lda,
                                         int64_t a_row0, int64_t a_rows,
                                         const uint16_t* __restrict__ B, int64_t ldb,
                                         int64_t b_row0, int64_t b_rows, int ksteps,
                                         f32x4 (&acc)[8][4]) {
  if (loader_wave())
    mainloop_role<ABLK, BBLK, true>(sm, A, lda, a_row0, a_rows, B, ldb, b_row0, b_rows, ksteps,
                                    acc);
  else
    mainloop_role<ABLK, BBLK, false>(sm, A, lda, a_row0, a_rows, B, ldb, b_row0, b_rows, ksteps,
                                     acc);
}

// ---------------------------------------------------------------------------
// K-outer operands: the K index is the outer one.  Two forms:
//   kKOuter: element (r, k) at X[k * ld + r], as the weight [V, H] is for a
//     product over the vocabulary and the hidden rows [N, H] for a product
//     over tokens;
//   kKOuterBlocked: a K32-blocked matrix read along its other axis, element
//     (r, k) at X[kblocked_index(k, r, ld)] (ld = that matrix's K steps), as
//     dz_c [tokens, chunk columns] is for the product over tokens.
// A K step takes 32 lines (K values) of 256 elements (the tile's rows).
// Fragments come from ds_read_b64_tr_b16: within each group of 16 lanes that
// instruction gives lane i element i % 4 of the 8-byte pieces read by lanes
// i / 4 + 4s, s = 0..3.  Lane (li, g) of a 16-row fragment reads rows
// 4 (li % 4) .. + 3 of line 8g + li / 4, then of line 8g + 4 + li / 4, so it
// receives row li at K 8g .. 8g + 7: the fragment a K-contiguous read gives,
// hence the same products and bits.
//   kKOuter stage: the 32 lines in order, 512 B each, the 32-byte unit p
//     (rows 16p .. 16p + 15) of line k at unit p ^ ksw(k), ksw(k) = (k & 3) |
//     ((k >> 1) & 4), so the eight lines one half-wave of a read touches fall
//     on different banks; one direct load fills two lines (lane L: line
//     L / 32, 16-byte unit L % 32), eight whole 128-byte lines.  Lines at or
//     past kvalid read a zero line (the zero rows of a padded K32-blocked
//     operand), rows at or past rvalid read rows from rvalid - 8 on (they
//     feed only outputs the caller masks; rvalid a multiple of 8, >= 8).
//   kKOuterBlocked stage: the source's own 1 KiB pieces (16 lines x 32 rows,
//     64 B per line), piece (line / 16) * 8 + row / 32, so one direct load
//     copies one whole piece; inside a piece the two 32-byte halves of line k
//     swap when bit 3 of k is set, which puts the eight lines of a half-wave
//     read on different banks.  Every line and row must hold data (the source
//     is padded with zeros to whole 256-row tiles and 32-line steps).
// ---------------------------------------------------------------------------
enum { kKContig = 0, kKOuter = 1, kKOuterBlocked = 2 };

static __device__ uint16_t kZeroLine[kTile];  // never written: zero from load time

__device__ __forceinline__ int ksw(int k) { return (k & 3) | ((k >> 1) & 4); }

// A loader wave's sources for one K-outer operand: load u (< 4) of a K step
// fills 1 KiB of the stage at (wave + 4u) KiB: lines 2 (wave + 4u) and
// 2 (wave + 4u) + 1 (kKOuter), or piece wave + 4u (kKOuterBlocked).
struct KOuterSrc {
  const uint16_t* p[4];  // this lane's source of load u at K step 0
  int line[4];           // its line within a K step
  int zofs;              // its 16-byte piece of the zero line
  int64_t sstride;       // elements between K steps
  template <int FORM>
  __device__ __forceinline__ void init(const uint16_t* X, int64_t ld, int64_t row0,
                                       int64_t rvalid, int wave, int lane) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int piece = wave + 4 * u;
      if constexpr (FORM == kKOuterBlocked) {
        const int l = (piece >> 3) * 16 + lane / 4;
        const int half = ((lane % 4) >> 1) ^ ((l >> 3) & 1);
        p[u] = X + kblocked_index(l, row0 + (piece & 7) * 32 + half * 16 + (lane & 1) * 8, ld);
        line[u] = l;
      } else {
        const int up = lane % 32;  // physical 16-byte unit of the line
        const int l = 2 * piece + lane / 32;
        const int64_t r = min(row0 + 16 * ((up / 2) ^ ksw(l)) + 8 * (up % 2), rvalid - 8);
        p[u] = X + l * ld + r;
        line[u] = l;
      }
    }
    zofs = 8 * (lane % 32);
    sstride = FORM == kKOuterBlocked ? 2 * ld * 512 : kK * ld;
  }
  __device__ __forceinline__ const uint16_t* at(int u, int step, int kvalid) const {
    return step * kK + line[u] < kvalid ? p[u] + step * sstride : kZeroLine + zofs;
  }
};

// A loader wave's 4 direct loads of one operand for K step `step` into the
// 16 KiB at dst: K32-blocked (blocks wave + 4u) or K-outer (the line pairs
// or pieces wave + 4u of KOuterSrc).
__device__ __forceinline__ void load_blocked(const LoaderSrc<true>& s, uint16_t* dst, int wave,
                                             int step) {
  const int64_t k = static_cast<int64_t>(step) * 512;
#pragma unroll
  for (int u = 0; u < 4; ++u)
    __builtin_amdgcn_global_load_lds(s.at(u, k), dst + (wave + 4 * u) * 16 * kK, 16, 0, 0);
}
__device__ __forceinline__ void load_kouter(const KOuterSrc& s, int kvalid, uint16_t* dst,
                                            int wave, int step) {
#pragma unroll
  for (int u = 0; u < 4; ++u)
    __builtin_amdgcn_global_load_lds(s.at(u, step, kvalid), dst + (wave + 4 * u) * 16 * kK, 16,
                                     0, 0);
}

// The fragment of a K-outer stage whose first transposed read is at p and
// second at p + SECOND (four lines on).
template <int SECOND>
__device__ __forceinline__ bf16x8 read_kouter_frag(const uint16_t* p) {
  typedef short i16x4 __attribute__((ext_vector_type(4)));
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + SECOND));
  const i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// Element offset, inside a K-outer stage of form FORM, of lane (li, g)'s
// first transposed read for the fragment of rows r0 .. r0 + 15 (r0 a
// multiple of 16), and the second read's distance.
template <int FORM>
__device__ __forceinline__ int kouter_off(int r0, int li, int g) {
  const int l = 8 * g + li / 4;
  if constexpr (FORM == kKOuterBlocked)
    return ((l >> 4) * 8 + (r0 >> 5)) * 512 + (l & 15) * 32 +
           ((((r0 >> 4) & 1) ^ ((l >> 3) & 1)) * 16) + 4 * (li % 4);
  else
    return l * kTile + (((r0 >> 4) ^ ksw(l)) * 16) + 4 * (li % 4);
}
template <int FORM>
constexpr int kouter_second() {
  return FORM == kKOuterBlocked ? 4 * 32 : 4 * kTile;
}

// The 256 x 256 tile's main loop (mainloop_role's pipeline, barriers, wait
// counts and loader waves) with each operand in one of the forms above (AF /
// BF; kKContig = K32-blocked with ld between 16-row blocks; a K-outer operand
// takes its ld and kvalid = its lines that hold data, counted from the
// first).  Waves of 128 x 64 as in mainloop_role.  Per K step a wave reads 8
// A and 4 B fragments, two transposed reads each for a K-outer operand,
// spread over its first 24 MFMAs.  (Waves of 64 x 128, which halve a K-outer
// A's transposed reads, measured slower.)
template <int AF, int BF, bool LOADER>
__device__ __forceinline__ void mainloop_ko(Stages& sm, const uint16_t* __restrict__ A,
                                            int64_t lda, int64_t a_row0, int64_t a_rows,
                                            int a_kvalid, const uint16_t* __restrict__ B,
                                            int64_t ldb, int64_t b_row0, int64_t b_rows,
                                            int b_kvalid, int ksteps, f32x4 (&acc)[8][4]) {
  constexpr int MI = 8, NJ = 4, WM = 128, WN = 64;
  constexpr bool AKO = AF != kKContig, BKO = BF != kKContig;
  constexpr int NL = LOADER ? kLoaderLoads : 0;
  constexpr int NR = MI * (AKO ? 2 : 1) + NJ * (BKO ? 2 : 1);  // LDS reads per K step
  static_assert(NR >= 12 && NR <= 24, "read interleave assumes 12 to 24 reads per step");
  const int tid = threadIdx.x;
  const int lane = tid % 64;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int wm = wave / 4, wn = wave % 4;
  const int li = lane % 16, g = lane / 16;
  const int lrow = lane / 4;
  const int lk = ((lane % 4) ^ swz(lrow)) * 8;
  LoaderSrc<true> ab, bb;
  KOuterSrc ak, bk;
  if constexpr (LOADER) {
    if constexpr (AKO) ak.init<AF>(A, lda, a_row0, a_rows, wave, lane);
    else ab.init(A, lda, a_row0, a_rows, wave, lrow, lk);
    if constexpr (BKO) bk.init<BF>(B, ldb, b_row0, b_rows, wave, lane);
    else bb.init(B, ldb, b_row0, b_rows, wave, lrow, lk);
  }
#define ITL_KO_ISSUE(S_, STEP_)                                                                 \
  if constexpr (LOADER) {                                                                       \
    if constexpr (AKO) load_kouter(ak, a_kvalid, sm.s[S_][0], wave, (STEP_));                   \
    else load_blocked(ab, sm.s[S_][0], wave, (STEP_));                                          \
    if constexpr (BKO) load_kouter(bk, b_kvalid, sm.s[S_][1], wave, (STEP_));                   \
    else load_blocked(bb, sm.s[S_][1], wave, (STEP_));                                          \
  }
  // Fragment offsets (elements) inside a stage.  K-contiguous: row wm*WM +
  // li (+16 i) of A, row wn*WN + li (+16 j) of B, chunk g.  K-outer: as
  // kouter_off gives them.
  const int aoff = (wm * WM + li) * kK + ((g ^ swz(li)) * 8);
  const int boff = (wn * WN + li) * kK + ((g ^ swz(li)) * 8);
#define ITL_KO_READ(FA, FB, ST)                                                                 \
  {                                                                                             \
    const uint16_t* fa = sm.s[ST][0];                                                           \
    const uint16_t* fb = sm.s[ST][1];                                                           \
    _Pragma("unroll") for (int j = 0; j < NJ; ++j) {                                            \
      if constexpr (BKO)                                                                        \
        FB[j] = read_kouter_frag<kouter_second<BF>()>(                                          \
            fb + kouter_off<BF>(wn * WN + 16 * j, li, g));                                      \
      else                                                                                      \
        FB[j] = *reinterpret_cast<const bf16x8*>(fb + boff + j * 16 * kK);                      \
    }                                                                                           \
    _Pragma("unroll") for (int i = 0; i < MI; ++i) {                                            \
      if constexpr (AKO)                                                                        \
        FA[i] = read_kouter_frag<kouter_second<AF>()>(                                          \
            fa + kouter_off<AF>(wm * WM + 16 * i, li, g));                                      \
      else                                                                                      \
        FA[i] = *reinterpret_cast<const bf16x8*>(fa + aoff + i * 16 * kK);                      \
    }                                                                                           \
  }
  for (int st = 0; st < kStages; ++st) ITL_KO_ISSUE(st, st < ksteps ? st : ksteps - 1);
  wait_vm<(kStages - 1) * NL>();
  __builtin_amdgcn_s_barrier();
  bf16x8 xa[MI], xb[NJ], ya[MI], yb[NJ];
  ITL_KO_READ(xa, xb, 0)
#define ITL_KO_STEP(CA, CB, NA, NB, KT)                                                         \
  {                                                                                             \
    wait_vm_lgkm0<(kStages - 2) * NL>();                                                        \
    __builtin_amdgcn_s_barrier();                                                               \
    ITL_KO_ISSUE((KT) % kStages, (KT) + kStages < ksteps ? (KT) + kStages : ksteps - 1);        \
    ITL_KO_READ(NA, NB, ((KT) + 1) % kStages)                                                   \
    _Pragma("unroll") for (int i = 0; i < MI; ++i)                                              \
      _Pragma("unroll") for (int j = 0; j < NJ; ++j)                                            \
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(CA[i], CB[j], acc[i][j], 0, 0, 0);  \
    if constexpr (LOADER) __builtin_amdgcn_sched_group_barrier(0x020, NL, 0);                   \
    _Pragma("unroll") for (int u = 0; u < 2 * NR - 24; ++u) {                                   \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                        \
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                                        \
    }                                                                                           \
    _Pragma("unroll") for (int u = 0; u < 24 - NR; ++u) {                                       \
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);                                        \
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                                        \
    }                                                                                           \
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);                                          \
  }
  for (int kt = 0; kt < ksteps; kt += 2) {
    ITL_KO_STEP(xa, xb, ya, yb, kt)
    ITL_KO_STEP(ya, yb, xa, xb, kt + 1)
  }
#undef ITL_KO_STEP
#undef ITL_KO_READ
#undef ITL_KO_ISSUE
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// ---------------------------------------------------------------------------
// Narrow tiles for few hidden rows: ROWS (64 or 128) A rows x 256 B rows,
// the same MFMA form, K walk and LDS chunk layout as the 256 x 256 tile, so
// every output gets the same bits.  8 waves; wave w covers rows
// (w / 4) * (ROWS / 2) + [0, ROWS / 2) and columns (w % 4) * 64 + [0, 64)
// as acc[i][j][q] = C[row0 + i*16 + 4*g + q][col0 + j*16 + li], i < ROWS /
// 32, j < 4 (the 256-row tile's arrangement with fewer rows; fewer registers
// than waves of 128 columns, the same time).  With so little arithmetic per weight byte the tile is bound by the
// bytes it keeps in flight: ROWS = 128 runs five stages (96 KiB in flight,
// one workgroup per CU); ROWS = 64 runs three stages of 20 KiB so that two
// workgroups share a CU (594 vocabulary tiles then take two rounds of 512
// instead of three of 256).  Wave w fills B blocks w, w + 8 and, for w <
// ROWS / 16, A block w of every stage.
// ---------------------------------------------------------------------------
template <int ROWS>
struct NarrowCfg {
  static constexpr int kStages = ROWS == 128 ? 5 : 3;
  static constexpr int kMI = ROWS / 32;
};

template <int ROWS, int S = NarrowCfg<ROWS>::kStages>
struct StagesNarrow {
  uint16_t a[S][ROWS * kK];
  uint16_t b[S][kTile * kK];  // 16 KiB each
};

// The narrow tile with a row-major B staged in pairs of K steps, as
// mainloop_pairs does for the 256-row tile: four A slots of ROWS x 32 and NPS
// B pair slots of 256 x 64 (NPS = 2: 80 KiB for ROWS = 64; NPS = 4: 144 KiB,
// NPS - 1 pairs in flight; one workgroup per CU either way), every B direct
// load 8 rows x 128 bytes.  Wave w issues, on odd steps, rows (w + 8u) * 8 +
// [0, 8), u < 4, of the B pair 2 NPS - 2 steps ahead and, for w < ROWS / 16,
// A block w of every step.  NTB: the B loads carry the non-temporal hint (B
// read by this workgroup only).
template <int ROWS, int NPS = 2>
struct StagesNarrowPairs {
  uint16_t a[4][ROWS * kK];
  uint16_t b[NPS][kTile * 2 * kK];  // 32 KiB each
};

template <int ROWS, bool NTB, int NPS = 2>
__device__ __forceinline__ void mainloop_narrow_pairs(StagesNarrowPairs<ROWS, NPS>& sm,
                                                      const uint16_t* __restrict__ A, int64_t lda,
                                                      int64_t a_row0, int64_t a_rows,
                                                      const uint16_t* __restrict__ B, int64_t ldb,
                                                      int64_t b_row0, int64_t b_rows, int ksteps,
                                                      f32x4 (&acc)[ROWS / 32][4]) {
  constexpr int MI = ROWS / 32;
  constexpr int kAux = NTB ? 2 : 0;  // cache policy: 2 = non-temporal
  const int tid = threadIdx.x;
  const int lane = tid % 64;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int wm = wave / 4, wn = wave % 4;
  const int li = lane % 16, g = lane / 16;
  const int lrow = lane / 4;
  const int lk = ((lane % 4) ^ swz(lrow)) * 8;
  const bool has_a = wave < ROWS / 16;  // uniform
  const uint16_t* a0 = A + min(a_row0 + (has_a ? wave : 0) * 16 + lrow, a_rows - 1) * lda + lk;
  const uint16_t* bp[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int r = (wave + 8 * u) * 8 + lane / 8;  // tile row this lane fills
    bp[u] = B + min(b_row0 + r, b_rows - 1) * ldb + ((lane % 8) ^ swzp(r)) * 8;
  }
  constexpr int kBlk = 16 * kK;  // elements per 1 KiB direct load
  auto issue_a = [&](int slot, int step) {
    if (has_a)
      __builtin_amdgcn_global_load_lds(a0 + static_cast<int64_t>(step) * kK,
                                       sm.a[slot] + wave * kBlk, 16, 0, 0);
  };
  auto issue_b = [&](int pslot, int pair) {
    const int64_t kb = static_cast<int64_t>(pair) * 2 * kK;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      __builtin_amdgcn_global_load_lds(bp[u] + kb, sm.b[pslot] + (wave + 8 * u) * kBlk, 16, 0,
                                       kAux);
  };
  const int npairs = ksteps / 2;
  const int aoff = (wm * (ROWS / 2) + li) * kK + ((g ^ swz(li)) * 8);
  const int brow = wn * 64 + li;
  const int bsw = swzp(li);
  // Iteration it issues A of step it + 4 and, when it is odd, the B pair
  // (it + 2 NPS - 1) / 2 (steps it + 2 NPS - 1, it + 2 NPS) into slot pair %
  // NPS, whose previous pair was last read for step it.  Prologue =
  // iterations -max(4, 2 NPS - 1) .. -1.
  constexpr int P0 = 2 * NPS - 1 > 4 ? 2 * NPS - 1 : 4;
#pragma unroll
  for (int it = -P0; it < 0; ++it) {
    if (it >= -4) issue_a(it + 4, it + 4 < ksteps ? it + 4 : ksteps - 1);
    if (it & 1) {
      const int p = (it + 2 * NPS - 1) / 2;
      issue_b(p, p < npairs ? p : npairs - 1);
    }
  }
  // Waits (NA = this wave's A loads per step, NB = its B loads per pair):
  // before step 0, A(0) and pair 0 have landed once the loads issued after
  // the later of the two are all that is in flight.
  constexpr int NB = 4;
  if (has_a) {
    if constexpr (NPS == 2) wait_vm<2 + NB>(); else wait_vm<3 + 2 * NB>();
  } else {
    if constexpr (NPS == 2) wait_vm<NB>(); else wait_vm<2 * NB>();
  }
  __builtin_amdgcn_s_barrier();
  bf16x8 xa[MI], xb[4], ya[MI], yb[4];
  auto read_frags = [&](bf16x8 (&fa)[MI], bf16x8 (&fb)[4], int step) {
    const uint16_t* fa_ = sm.a[step % 4];
    const uint16_t* fb_ = sm.b[(step / 2) % NPS];
    const int ch = ((4 * (step % 2) + g) ^ bsw) * 8;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      fb[j] = *reinterpret_cast<const bf16x8*>(fb_ + (brow + 16 * j) * 2 * kK + ch);
#pragma unroll
    for (int i = 0; i < MI; ++i)
      fa[i] = *reinterpret_cast<const bf16x8*>(fa_ + aoff + i * 16 * kK);
  };
  read_frags(xa, xb, 0);
  // Before iteration KT, A(KT+1) (issued at KT-3) and the pair of step
  // KT+1 must have landed: with NPS = 2 (that pair issued at KT-3 after the
  // A load for even KT, at KT-2 for odd KT) 2 NA + NB loads may still be in
  // flight for even KT and NA for odd KT; with NPS >= 3 (the pair older than
  // A(KT+1)) 2 NA + 2 NB for even KT and 2 NA + NB for odd KT.
#define ITL_NPSTEP(CA, CB, NXA, NXB, KT, ODD)                                                   \
  {                                                                                             \
    if (has_a) {                                                                                \
      if constexpr (NPS == 2) {                                                                 \
        if constexpr (ODD) wait_vm_lgkm0<1>(); else wait_vm_lgkm0<2 + NB>();                    \
      } else {                                                                                  \
        if constexpr (ODD) wait_vm_lgkm0<2 + NB>(); else wait_vm_lgkm0<2 + 2 * NB>();           \
      }                                                                                         \
    } else {                                                                                    \
      if constexpr (NPS == 2) {                                                                 \
        if constexpr (ODD) wait_vm_lgkm0<0>(); else wait_vm_lgkm0<NB>();                        \
      } else {                                                                                  \
        if constexpr (ODD) wait_vm_lgkm0<NB>(); else wait_vm_lgkm0<2 * NB>();                   \
      }                                                                                         \
    }                                                                                           \
    __builtin_amdgcn_s_barrier();                                                               \
    issue_a((KT) % 4, (KT) + 4 < ksteps ? (KT) + 4 : ksteps - 1);                               \
    if constexpr (ODD) {                                                                        \
      const int p_ = ((KT) + 2 * NPS - 1) / 2;                                                  \
      issue_b(p_ % NPS, p_ < npairs ? p_ : npairs - 1);                                         \
    }                                                                                           \
    read_frags(NXA, NXB, (KT) + 1);                                                             \
    _Pragma("unroll") for (int i = 0; i < MI; ++i)                                              \
      _Pragma("unroll") for (int j = 0; j < 4; ++j)                                             \
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(CA[i], CB[j], acc[i][j], 0, 0, 0);  \
  }
  for (int kt = 0; kt < ksteps; kt += 2) {
    ITL_NPSTEP(xa, xb, ya, yb, kt, false)
    ITL_NPSTEP(ya, yb, xa, xb, kt + 1, true)
  }
#undef ITL_NPSTEP
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// acc += A[a_row0 + 0..ROWS-1, 0..K) * B[b_row0 + 0..255, 0..K)^T, K =
// ksteps * 32 (ksteps even, >= 2); A row-major, B row-major or K32-blocked
// (BBLK, ldb = distance between 16-row blocks); rows at or past a_rows /
// b_rows are read from the last valid row (block).  NTB: B is read once per
// launch (no other workgroup reads the same rows) and K32-blocked, so its
// direct loads carry the non-temporal hint (measured: the decode-sized
// forward with a prepared weight 0.250 -> 0.227 ms; on row-major B, whose
// loads take half lines, the hint made it 43% slower).  All 512 threads must
// call; on return every direct load has landed and the stages may be reused
// after a barrier.
template <int ROWS, bool BBLK = false, bool NTB = false, int S = NarrowCfg<ROWS>::kStages>
__device__ __forceinline__ void mainloop_narrow(StagesNarrow<ROWS, S>& sm,
                                                const uint16_t* __restrict__ A, int64_t lda,
                                                int64_t a_row0, int64_t a_rows,
                                                const uint16_t* __restrict__ B, int64_t ldb,
                                                int64_t b_row0, int64_t b_rows, int ksteps,
                                                f32x4 (&acc)[NarrowCfg<ROWS>::kMI][4]) {
  constexpr int MI = NarrowCfg<ROWS>::kMI;
  const int tid = threadIdx.x;
  const int lane = tid % 64;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int wm = wave / 4, wn = wave % 4;
  const int li = lane % 16, g = lane / 16;
  const int lrow = lane / 4;
  const int lk = ((lane % 4) ^ swz(lrow)) * 8;
  const bool has_a = wave < ROWS / 16;  // uniform
  const uint16_t* a0 = A + min(a_row0 + (has_a ? wave : 0) * 16 + lrow, a_rows - 1) * lda + lk;
  const uint16_t* b0 = lane_chunk<BBLK>(B, ldb, b_row0, b_rows, wave, lrow, lk);
  const uint16_t* b1 = lane_chunk<BBLK>(B, ldb, b_row0, b_rows, wave + 8, lrow, lk);
  constexpr int SB = BBLK ? 512 : kK;
  const int aoff = (wm * (ROWS / 2) + li) * kK + ((g ^ swz(li)) * 8);
  const int boff = (wn * 64 + li) * kK + ((g ^ swz(li)) * 8);
  constexpr int kBlk = 16 * kK;
  auto issue_step = [&](int s, int step) {
    const int64_t k0 = static_cast<int64_t>(step) * kK, kb = static_cast<int64_t>(step) * SB;
    if (has_a) __builtin_amdgcn_global_load_lds(a0 + k0, sm.a[s] + wave * kBlk, 16, 0, 0);
    constexpr int kAux = NTB ? 2 : 0;  // cache policy: 2 = non-temporal
    __builtin_amdgcn_global_load_lds(b0 + kb, sm.b[s] + wave * kBlk, 16, 0, kAux);
    __builtin_amdgcn_global_load_lds(b1 + kb, sm.b[s] + (wave + 8) * kBlk, 16, 0, kAux);
  };
  // Iteration kt: MFMAs of step kt on fragments in registers, fragment reads
  // of step kt+1, direct loads of step kt+S (kt+2 .. kt+S-1 in flight).
  // Every iteration issues the same loads per wave (3 with an A block, else
  // 2), so the wait counts are constant per wave; past the end the loads
  // re-fetch the last K step into a stage no longer read.
  for (int st = 0; st < S; ++st) issue_step(st, st < ksteps ? st : ksteps - 1);
  if (has_a)
    wait_vm<(S - 1) * 3>();
  else
    wait_vm<(S - 1) * 2>();
  __builtin_amdgcn_s_barrier();
  bf16x8 xa[MI], xb[4], ya[MI], yb[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) xb[j] = *reinterpret_cast<const bf16x8*>(sm.b[0] + boff + j * 16 * kK);
#pragma unroll
  for (int i = 0; i < MI; ++i) xa[i] = *reinterpret_cast<const bf16x8*>(sm.a[0] + aoff + i * 16 * kK);
  int cur = 0;  // stage of step kt
#define ITL_NSTEP(CA, CB, NA, NB, KT)                                                        \
  {                                                                                          \
    if (has_a)                                                                               \
      wait_vm_lgkm0<(S - 2) * 3>();                                                          \
    else                                                                                     \
      wait_vm_lgkm0<(S - 2) * 2>();                                                          \
    __builtin_amdgcn_s_barrier();                                                            \
    const int nxt = cur + 1 == S ? 0 : cur + 1;                                              \
    issue_step(cur, (KT) + S < ksteps ? (KT) + S : ksteps - 1);                              \
    _Pragma("unroll") for (int j = 0; j < 4; ++j)                                            \
      NB[j] = *reinterpret_cast<const bf16x8*>(sm.b[nxt] + boff + j * 16 * kK);              \
    _Pragma("unroll") for (int i = 0; i < MI; ++i)                                           \
      NA[i] = *reinterpret_cast<const bf16x8*>(sm.a[nxt] + aoff + i * 16 * kK);              \
    cur = nxt;                                                                               \
    _Pragma("unroll") for (int i = 0; i < MI; ++i)                                           \
      _Pragma("unroll") for (int j = 0; j < 4; ++j)                                          \
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(CA[i], CB[j], acc[i][j], 0, 0, 0); \
  }
  for (int kt = 0; kt < ksteps; kt += 2) {
    ITL_NSTEP(xa, xb, ya, yb, kt)
    ITL_NSTEP(ya, yb, xa, xb, kt + 1)
  }
#undef ITL_NSTEP
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

}  // namespace gemm
}  // namespace itl
