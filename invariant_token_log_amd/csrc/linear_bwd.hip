// Backward of the fused LM head + logp on gfx950 ("[RFC][ROCm] End-to-end
// optimization of bitwise VIME R/R beyond native P/P", Workstream 3: the
// backward recomputes the fixed logit tiles from the saved LSE; "Batch-
// Invariant LogP", Batch-Invariance: the logit gradient is g * (onehot - p)).
//
//   z  = h W^T                (recomputed: the forward's MFMA tile and K walk,
//                              so z has the forward's bits; or read from the
//                              forward's saved logits, the same values)
//   dz = RNE_bf16(g * (onehot(t) - exp(z - lse)))   (0 on ignored and padded rows)
//   dh = dz W                 (fp32 accumulators, K = vocabulary, ascending)
//   dW = dz^T h               (fp32 accumulators, K = tokens, ascending)
//
// dz is rounded to bf16 once (the only rounding point besides the fp32
// accumulators) because both products run on bf16 MFMA.  Every product is a
// single ascending K walk with no split, so dh[r] depends only on row r (batch
// invariant) and dW is deterministic for a given token order.
//
// The vocabulary is walked in chunks of whole 256-column tiles (the
// caller's vocab_chunk, default kDefaultChunk columns); per chunk [c0, c1):
//   dz_c         = the chunk's columns of dz (recomputed tiles, or the saved
//                  logits);
//   dW[c0:c1]    = dz_c^T h        (K = all tokens, ascending: final rows);
//   dh          += dz_c W[c0:c1]   (K = the chunk's vocabulary, ascending,
//                                   continuing the fp32 accumulators the
//                                   previous chunk stored).
// Continuing a K walk from stored fp32 accumulators gives the same bits as
// one walk, so the chunk width changes the memory the backward needs, not a
// bit of dh or dW.
//
// Kernels (the products on the 256 x 256 tile of mfma_gemm.h):
//   block_rows_bf16   : h [N, H] -> the K32-blocked copy the recomputed
//                       product reads;
//   linear_dz_kernel  : h x W^T tile of one chunk -> dz in registers -> LDS
//                       tile -> dz_c;
//   linear_dz_saved_kernel: the same dz_c from saved logits, 32 x 256 tiles
//                       through LDS;
//   transpose_blocked : h -> h^T [H, Np] (32 x 256 tiles through LDS);
//   gemm_out_kernel   : C = A B^T (+ stored C) with fp32 or RNE-bf16 output.
// The operands the backward writes for a product (dz_c, h^T and the blocked
// h) are in the K32-blocked layout of mfma_gemm.h; the two operands whose K
// index is the outer one are read as they are, through mfma_gemm.h's
// K-outer staging (transposed LDS reads, same fragments, same bits): the
// weight rows W[c0:c1] for dh, and dz_c along its token axis for dW.  Np, Vp
// are N and V rounded up to multiples of 256; padded rows and columns hold
// zeros and add exact zeros to the K walks (a K-outer operand's lines past
// its data read a zero line).
#include "launch.h"
#include "logp_device.h"
#include "mfma_gemm.h"

namespace itl {

namespace {

using gemm::f32x4;

constexpr int kT = gemm::kTile;
constexpr int kDzStride = kT + 8;  // bf16 per LDS tile row (528 B, 16-byte aligned)

__device__ __forceinline__ uint16_t bf16_bits(float d) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(d));
}

// 32 x 256 tiles of bf16 staged in LDS for the transposing kernels (rows
// padded to 264 elements: 16-byte aligned, and the 8-row gathers of the
// transposed reads fall on different banks).
constexpr int kTR = 32, kTC = 256, kTS = kTC + 8;

// The 16-byte piece of the transposed tile that starts at tile row rq (a
// multiple of 8) in column c: tile[rq + 0..7][c] packed low to high.
__device__ __forceinline__ uint4 gather_column8(const uint16_t (*tile)[kTS], int rq, int c) {
  uint32_t w[4];
#pragma unroll
  for (int e = 0; e < 4; ++e)
    w[e] = static_cast<uint32_t>(tile[rq + 2 * e][c]) |
           (static_cast<uint32_t>(tile[rq + 2 * e + 1][c]) << 16);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// Writes the tile transposed: column c (< cols_here) becomes destination row
// c_dst0 + c of the K32-blocked dst (K steps per 16-row block: ksteps), its
// 32 tile rows the K range [k0, k0 + 32).  16 pieces of 1 KiB, one 16-byte
// chunk per thread and step.
__device__ __forceinline__ void store_transposed(const uint16_t (*tile)[kTS], uint16_t* dst,
                                                 int64_t c_dst0, int cols_here, int64_t k0,
                                                 int64_t ksteps, int tid) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int q = tid + 256 * u;
    const int p = q >> 6, e = q & 63;
    const int c = p * 16 + (e >> 2), rq = (e & 3) * 8;
    if (c < cols_here)
      store_stream(dst + gemm::kblocked_index(c_dst0 + c, k0 + rq, ksteps),
                   gather_column8(tile, rq, c));
  }
}

// dst = the K32-blocked [cols, K = rows_p] operand with element (c, r) =
// r < rows ? src[r * ld + c] : 0 (cols a multiple of 16, rows_p of 32).
// Tiles of 32 source rows x 256 source columns: every thread loads 16-byte
// chunks of whole 512-byte row segments, the tile leaves as 1 KiB pieces.
// Grid: x = column tiles, y = row tiles (grid-stride beyond gridDim.y).
__global__ __launch_bounds__(256) void transpose_blocked(const uint16_t* __restrict__ src,
                                                         int64_t ld, int64_t rows,
                                                         int64_t rows_p, int64_t cols,
                                                         uint16_t* __restrict__ dst) {
  __shared__ __align__(16) uint16_t tile[kTR][kTS];
  const int tid = threadIdx.x;
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * kTC;
  const int cols_here = static_cast<int>(cols - c0 < kTC ? cols - c0 : kTC);
  const int64_t ksteps = rows_p / gemm::kK;
  for (int64_t r0 = static_cast<int64_t>(blockIdx.y) * kTR; r0 < rows_p;
       r0 += static_cast<int64_t>(gridDim.y) * kTR) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int r = (tid >> 5) + 8 * u, ch = (tid & 31) * 8;
      uint4 x = make_uint4(0u, 0u, 0u, 0u);
      if (r0 + r < rows && ch < cols_here) x = load_stream(src + (r0 + r) * ld + c0 + ch);
      *reinterpret_cast<uint4*>(&tile[r][ch]) = x;
    }
    __syncthreads();
    store_transposed(tile, dst, c0, cols_here, r0, ksteps, tid);
    __syncthreads();
  }
}

// dst = the K32-blocked [rows_p, K = k] copy of src [rows, k] (rows past
// rows zero); one 16-byte chunk per thread in destination order.  Block 0
// also clears the nzero ints at zero (tile-queue counters of the launches
// that follow).
__global__ __launch_bounds__(256) void block_rows_bf16(const uint16_t* __restrict__ src,
                                                       int64_t ld, int64_t rows, int64_t rows_p,
                                                       int64_t k, uint16_t* __restrict__ dst,
                                                       int* __restrict__ zero, int nzero) {
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < nzero; i += 256) zero[i] = 0;
  const int64_t ksteps = k / gemm::kK, chunks = rows_p * (k / 8);
  for (int64_t c = blockIdx.x * 256ll + threadIdx.x; c < chunks;
       c += static_cast<int64_t>(gridDim.x) * 256) {
    // chunk c: 16-row block rb, K step ks, row r16 of the block, quarter q
    const int64_t q = c & 3, r16 = (c >> 2) & 15, t = c >> 6;
    const int64_t ks = t % ksteps, row = (t / ksteps) * 16 + r16;
    uint4 x = make_uint4(0u, 0u, 0u, 0u);
    if (row < rows) x = *reinterpret_cast<const uint4*>(src + row * ld + ks * gemm::kK + q * 8);
    *reinterpret_cast<uint4*>(dst + c * 8) = x;
  }
}

// One element of the logit gradient.  z = the logit (RNE_bf16 of it in the
// bf16-rounded variant, whose gradient passes the rounding unchanged);
// x = z (* 1/T); p = exp(x - lse) with the forward's primitive; d = g (1 - p)
// on the target column, (-g) p elsewhere, plus -gH p (x - lse + H) with the
// entropy term (one fma, the -inf clamp of ent_term); d (* 1/T) for dz.
// PLAIN: the caller knows that no option is on (no rounding, T = 1, no
// entropy term), so the options cost nothing; the operations left are the
// same, so the bits are too.
template <bool PLAIN = false>
__device__ __forceinline__ float dz_value(float zacc, float L, float G, float H, float NGH,
                                          bool is_target, float inv_t, bool scaled,
                                          bool with_ent, int32_t round_bf16) {
  const float z = !PLAIN && round_bf16 ? static_cast<float>(static_cast<__bf16>(zacc)) : zacc;
  const float x = !PLAIN && scaled ? z * inv_t : z;
  const float dl = x - L;  // exp_sub(x, L) in two steps
  const float p = __builtin_amdgcn_exp2f(dl * kLog2e);
  float d = is_target ? G * (1.0f - p) : (-G) * p;
  if (!PLAIN && with_ent) d = fmaf(NGH, p * fmaxf(dl + H, -FLT_MAX), d);
  if (!PLAIN && scaled) d = d * inv_t;
  return d;
}

struct SmemDz {
  union {
    gemm::Stages st;                // main loop
    uint16_t tile[kT][kDzStride];  // dz tile, one layout at a time
  } u;
  float lse[kT];
  float g[kT];
  float ent[kT];  // row entropy (entropy term only)
  float ngh[kT];  // -gH (entropy term only)
  // -2: no gradient (row past n or ignored); -1: target outside the block;
  // else t - v0
  int code[kT];
};

// dz of the vocabulary chunk of vcb 256-column blocks starting at block vb0:
// dz_c [Np, K = vcb * 256], K32-blocked with the chunk's own columns (the
// product over tokens reads it along its other axis).  hidden
// K32-blocked (mblocks * 256 rows); weight row-major, or K32-blocked with
// vblocks * 256 rows when WBLK (a prepared weight).  PLAIN: launched only
// when no option is on (no rounding, T = 1, no entropy term), so the
// epilogue skips their operations instead of selecting around them.
template <bool WBLK, bool PLAIN>
__global__ __launch_bounds__(gemm::kThreads) void linear_dz_kernel(
    const uint16_t* __restrict__ hidden, int64_t ld_h, const uint16_t* __restrict__ weight,
    int64_t ld_w, int64_t n, int64_t hdim, int64_t v, int mblocks, int vblocks, int vb0,
    int vcb, const void* __restrict__ tgt, int32_t tgt32, int64_t ignore_index,
    const float* __restrict__ lse,
    const float* __restrict__ grad, float inv_t, int32_t round_bf16,
    const float* __restrict__ ent, const float* __restrict__ gent, uint16_t* __restrict__ dz) {
  const Targets targets{tgt, tgt32};
  __shared__ __align__(16) SmemDz sm;
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wave / 4, wn = wave % 4;
  const int li = lane % 16, g = lane / 16;

  int mb, vb;
  gemm::tile_coords(gemm::xcd_logical(blockIdx.x, mblocks * vcb), mblocks, vcb, mb, vb);
  const int64_t m0 = static_cast<int64_t>(mb) * kT;
  const int64_t vl0 = static_cast<int64_t>(vb) * kT;          // column inside the chunk
  const int64_t v0 = static_cast<int64_t>(vb0) * kT + vl0;    // vocabulary column
  if (tid < kT) {
    const int64_t r = m0 + tid;
    int code = -2;
    float L = 0.0f, G = 0.0f, H = 0.0f, NGH = 0.0f;
    if (r < n) {
      const int64_t t = targets[r];
      if (t != ignore_index) {
        L = lse[r];
        G = grad[r];
        if (ent) {
          H = ent[r];
          NGH = -gent[r];
        }
        code = (t >= v0 && t < v0 + kT && t < v) ? static_cast<int>(t - v0) : -1;
      }
    }
    sm.code[tid] = code;
    sm.lse[tid] = L;
    sm.g[tid] = G;
    sm.ent[tid] = H;
    sm.ngh[tid] = NGH;
  }

  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  const int ksteps = static_cast<int>(hdim / gemm::kK);
  const int64_t kblk = static_cast<int64_t>(ksteps) * 512;  // blocked: 16-row block stride
  gemm::mainloop<true, WBLK>(sm.u.st, hidden, kblk, m0, static_cast<int64_t>(mblocks) * kT, weight,
                             WBLK ? kblk : ld_w, v0, WBLK ? static_cast<int64_t>(vblocks) * kT : v,
                             ksteps, acc);
  __syncthreads();

  // dz of every element (dz_value; 0 on ignored / padded rows and columns),
  // rounded to bf16; lane (li, g) holds rows 4g .. 4g+3 of column li of each
  // 16 x 16 block, packed in pairs.
  const bool scaled = inv_t != 1.0f;
  const bool with_ent = ent != nullptr;
  uint32_t dv[8][4][2];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float L[4], G[4], H[4], NGH[4];
    int code[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int lr = wm * 128 + i * 16 + 4 * g + q;
      code[q] = sm.code[lr];
      L[q] = sm.lse[lr];
      G[q] = sm.g[lr];
      H[q] = sm.ent[lr];
      NGH[q] = sm.ngh[lr];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int lc = wn * 64 + j * 16 + li;
      uint16_t b[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float d = code[q] != -2 && v0 + lc < v
                            ? dz_value<PLAIN>(acc[i][j][q], L[q], G[q], H[q], NGH[q],
                                              lc == code[q], inv_t, scaled, with_ent,
                                              round_bf16)
                            : 0.0f;
        b[q] = bf16_bits(d);
      }
      dv[i][j][0] = static_cast<uint32_t>(b[0]) | (static_cast<uint32_t>(b[1]) << 16);
      dv[i][j][1] = static_cast<uint32_t>(b[2]) | (static_cast<uint32_t>(b[3]) << 16);
    }
  }
  const int64_t vc_steps = static_cast<int64_t>(vcb) * (kT / gemm::kK);
  // tile[r][c] (row-major), then out in K32-blocked order.
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int lc = wn * 64 + j * 16 + li;
      const int lr = wm * 128 + i * 16 + 4 * g;
      sm.u.tile[lr][lc] = static_cast<uint16_t>(dv[i][j][0] & 0xffffu);
      sm.u.tile[lr + 1][lc] = static_cast<uint16_t>(dv[i][j][0] >> 16);
      sm.u.tile[lr + 2][lc] = static_cast<uint16_t>(dv[i][j][1] & 0xffffu);
      sm.u.tile[lr + 3][lc] = static_cast<uint16_t>(dv[i][j][1] >> 16);
    }
  __syncthreads();
  for (int idx = tid; idx < kT * 32; idx += gemm::kThreads) {
    const int piece = idx >> 6, e = idx & 63;
    const int r = (piece >> 3) * 16 + (e >> 2), c = (piece & 7) * 32 + (e & 3) * 8;
    store_stream(dz + gemm::kblocked_index(m0 + r, vl0 + c, vc_steps),
                 *reinterpret_cast<const uint4*>(&sm.u.tile[r][c]));
  }
}

// dz_c of the vocabulary chunk [c0, c0 + cols_p) from the forward's saved
// unscaled logits (fp32, or bf16 with ZBF16; [n, ld_z], 16-byte aligned
// rows) instead of the recomputed product: the same values through the same
// dz_value, so the same bits.  Tiles of 32 rows x 256 chunk columns: the
// logits of a row segment come in as 16-byte non-temporal loads of whole
// 512-byte (bf16) or 1 KiB (fp32) pieces, the bf16 dz goes to an LDS tile and
// leaves as 1 KiB K32-blocked pieces of dz_c [Np, K = cols_p].  Rows past n
// or ignored, and columns past v, get 0 without reading the logits.  Grid:
// x = column tiles, y = row tiles of the np_rows (grid-stride beyond
// gridDim.y): neighbouring workgroups read neighbouring KiB of the same rows
// and write neighbouring pieces of dz_c.
template <bool ZBF16>
__global__ __launch_bounds__(256) void linear_dz_saved_kernel(
    const void* __restrict__ zsaved, int64_t ld_z, int64_t n, int64_t v, int64_t np_rows,
    const void* __restrict__ tgt, int32_t tgt32, int64_t ignore_index,
    const float* __restrict__ lse, const float* __restrict__ grad, float inv_t,
    int32_t round_bf16, const float* __restrict__ ent, const float* __restrict__ gent,
    int64_t c0, int64_t cols_p, uint16_t* __restrict__ dz) {
  const Targets targets{tgt, tgt32};
  __shared__ __align__(16) uint16_t tile[kTR][kTS];
  __shared__ float rowc[kTR][4];  // lse, g, entropy, -gH of each tile row
  __shared__ int64_t rowt[kTR];   // target (ignore_index: no gradient)
  const int tid = threadIdx.x;
  const int64_t cl0 = static_cast<int64_t>(blockIdx.x) * kTC;
  const int64_t col0 = c0 + cl0;  // vocabulary column of the tile
  const bool scaled = inv_t != 1.0f;
  const bool with_ent = ent != nullptr;
  constexpr int E = ZBF16 ? 8 : 4;         // elements per 16-byte chunk
  constexpr int CPR = kTC / E;             // chunks per tile row
  constexpr int RPS = 256 / CPR;           // tile rows per step of the block
  const int64_t vc_steps = cols_p / gemm::kK;
  for (int64_t r0 = static_cast<int64_t>(blockIdx.y) * kTR; r0 < np_rows;
       r0 += static_cast<int64_t>(gridDim.y) * kTR) {
    if (tid < kTR) {
      const int64_t row = r0 + tid;
      int64_t t = ignore_index;
      float L = 0.0f, G = 0.0f, H = 0.0f, NGH = 0.0f;
      if (row < n) {
        t = targets[row];
        if (t != ignore_index) {
          L = lse[row];
          G = grad[row];
          if (with_ent) {
            H = ent[row];
            NGH = -gent[row];
          }
        }
      }
      rowt[tid] = row < n ? t : ignore_index;
      rowc[tid][0] = L;
      rowc[tid][1] = G;
      rowc[tid][2] = H;
      rowc[tid][3] = NGH;
    }
    __syncthreads();
    // All of this thread's loads go out before any arithmetic: chunk u is
    // row tid / CPR + RPS u, columns (tid % CPR) E + [0, E).
    constexpr int NU = kTR / RPS;
    const int ch = (tid % CPR) * E;
    const int64_t col = col0 + ch;
    const bool whole = col + E <= v;  // the chunk lies inside the row
    uint4 w[NU];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int r = tid / CPR + RPS * u;
      const int64_t row = r0 + r;
      w[u] = make_uint4(0u, 0u, 0u, 0u);
      if (whole && row < n && rowt[r] != ignore_index)
        w[u] = load_stream(static_cast<const char*>(zsaved) +
                           (row * ld_z + col) * (ZBF16 ? 2 : 4));
    }
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int r = tid / CPR + RPS * u;
      const int64_t row = r0 + r;
      const int64_t t = rowt[r];
      const bool live = row < n && t != ignore_index;
      float zv[E];
      const uint32_t q[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
      if constexpr (ZBF16) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          zv[2 * e] = bf16_lo(q[e]);
          zv[2 * e + 1] = bf16_hi(q[e]);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) zv[e] = __uint_as_float(q[e]);
      }
      if (live && !whole) {  // the row's last, partial chunk: element loads
#pragma unroll
        for (int e = 0; e < E; ++e)
          zv[e] = col + e < v
                      ? (ZBF16 ? bf16_lo(static_cast<const uint16_t*>(zsaved)[row * ld_z + col + e])
                               : static_cast<const float*>(zsaved)[row * ld_z + col + e])
                      : 0.0f;
      }
      const float L = rowc[r][0], G = rowc[r][1], H = rowc[r][2], NGH = rowc[r][3];
      uint16_t b[E];
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float d = live && col + e < v
                            ? dz_value(zv[e], L, G, H, NGH, col + e == t, inv_t, scaled,
                                       with_ent, round_bf16)
                            : 0.0f;
        b[e] = bf16_bits(d);
      }
      if constexpr (ZBF16) {
        *reinterpret_cast<uint4*>(&tile[r][ch]) =
            make_uint4(b[0] | (uint32_t(b[1]) << 16), b[2] | (uint32_t(b[3]) << 16),
                       b[4] | (uint32_t(b[5]) << 16), b[6] | (uint32_t(b[7]) << 16));
      } else {
        *reinterpret_cast<uint2*>(&tile[r][ch]) =
            make_uint2(b[0] | (uint32_t(b[1]) << 16), b[2] | (uint32_t(b[3]) << 16));
      }
    }
    __syncthreads();
    // pieces (16-row block rb, K step ks) of the tile
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int q = tid + 256 * u;
      const int p = q >> 6, e = q & 63;
      const int rb = p >> 3, ks = p & 7;
      const int r = rb * 16 + (e >> 2), c = ks * 32 + (e & 3) * 8;
      store_stream(dz + gemm::kblocked_index(r0 + r, cl0 + c, vc_steps),
                   *reinterpret_cast<const uint4*>(&tile[r][c]));
    }
    __syncthreads();
  }
}

// C[m_out, n_out] = A[., K] B[., K]^T on the mfma_gemm.h tile, both operands
// K32-blocked (lda / ldb: elements between 16-row blocks, so A and B may be a
// K range of a wider operand); the accumulators start from Cin (fp32,
// [m_out, ldcin]) when it is set, else from zero, and continue its K walk.
// BF16OUT rounds the fp32 accumulators to bf16 (RNE) on the way out.
// One role's share of the tile (gemm::mainloop_role): each role runs its
// own copy from the accumulator load to the store, so that no accumulator
// crosses the branch between the two loop bodies.
template <bool BF16OUT, bool LOADER, int AF, int BF>
__device__ __forceinline__ void gemm_out_tile(gemm::Stages& st, const uint16_t* __restrict__ A,
                                              int64_t lda, int64_t arows, int a_kvalid,
                                              const uint16_t* __restrict__ B, int64_t ldb,
                                              int64_t brows, int b_kvalid, int ksteps, int64_t m0,
                                              int64_t n0, int64_t m_out, int64_t n_out,
                                              const float* Cin, int64_t ldcin, void* C,
                                              int64_t ldc) {
  constexpr int MI = 8, NJ = 4, WM = 128, WN = 64;
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wave / 4, wn = wave % 4;
  const int li = lane % 16, g = lane / 16;
  f32x4 acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  if (Cin) {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t row = m0 + wm * WM + i * 16 + 4 * g + q;
        if (row >= m_out) continue;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int64_t col = n0 + wn * WN + j * 16 + li;
          if (col < n_out) acc[i][j][q] = Cin[row * ldcin + col];
        }
      }
  }
  if constexpr (AF != gemm::kKContig || BF != gemm::kKContig)
    gemm::mainloop_ko<AF, BF, LOADER>(st, A, lda, m0, arows, a_kvalid, B, ldb, n0, brows,
                                      b_kvalid, ksteps, acc);
  else
    gemm::mainloop_role<true, true, LOADER>(st, A, lda, m0, arows, B, ldb, n0, brows, ksteps,
                                            acc);
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t row = m0 + wm * WM + i * 16 + 4 * g + q;
      if (row >= m_out) continue;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int64_t col = n0 + wn * WN + j * 16 + li;
        if (col < n_out) {
          if (BF16OUT)
            static_cast<uint16_t*>(C)[row * ldc + col] = bf16_bits(acc[i][j][q]);
          else
            static_cast<float*>(C)[row * ldc + col] = acc[i][j][q];
        }
      }
    }
}

// AF / BF: the operand's form (mfma_gemm.h: K32-blocked, or K-outer with
// its ld and kvalid = the lines that hold data).
template <bool BF16OUT, int AF, int BF>
__global__ __launch_bounds__(gemm::kThreads) void gemm_out_kernel(
    const uint16_t* __restrict__ A, int64_t lda, int64_t arows, int a_kvalid,
    const uint16_t* __restrict__ B, int64_t ldb, int64_t brows, int b_kvalid, int ksteps,
    int mblocks, int nblocks, int64_t m_out, int64_t n_out, const float* Cin, int64_t ldcin,
    void* C, int64_t ldc) {
  __shared__ __align__(16) gemm::Stages st;
  int mb, nb;
  gemm::tile_coords(gemm::xcd_logical(blockIdx.x, mblocks * nblocks), mblocks, nblocks, mb, nb);
  const int64_t m0 = static_cast<int64_t>(mb) * kT;
  const int64_t n0 = static_cast<int64_t>(nb) * kT;
  if (gemm::loader_wave())
    gemm_out_tile<BF16OUT, true, AF, BF>(st, A, lda, arows, a_kvalid, B, ldb, brows,
                                             b_kvalid, ksteps, m0, n0, m_out, n_out, Cin, ldcin,
                                             C, ldc);
  else
    gemm_out_tile<BF16OUT, false, AF, BF>(st, A, lda, arows, a_kvalid, B, ldb, brows,
                                              b_kvalid, ksteps, m0, n0, m_out, n_out, Cin, ldcin,
                                              C, ldc);
}

// Zero rows x cols of C (a sum over no tokens).
template <bool BF16OUT>
__global__ __launch_bounds__(256) void fill_zero_kernel(void* C, int64_t ldc, int64_t rows,
                                                        int64_t cols) {
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < rows * cols;
       i += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t r = i / cols, c = i - r * cols;
    if (BF16OUT)
      static_cast<uint16_t*>(C)[r * ldc + c] = 0;
    else
      static_cast<float*>(C)[r * ldc + c] = 0.0f;
  }
}

int64_t round_tile(int64_t x) { return (x + kT - 1) / kT * kT; }

// grid of a tile walk over rows_p rows in kTR-row tiles (grid-stride beyond
// 65535 row tiles) and cols columns in kTC-column tiles
dim3 tile_grid(int64_t rows_p, int64_t cols) {
  const int64_t rt = rows_p / kTR;
  return dim3(static_cast<unsigned>((cols + kTC - 1) / kTC),
              static_cast<unsigned>(rt < 65535 ? rt : 65535));
}

// dst = the K32-blocked [cols, K = rows_p] transpose of src [rows, ld]
// (rows past `rows` zero).
void launch_transpose(const uint16_t* src, int64_t ld, int64_t rows, int64_t rows_p,
                      int64_t cols, uint16_t* dst, hipStream_t s) {
  hipLaunchKernelGGL(transpose_blocked, tile_grid(rows_p, cols), dim3(256), 0, s, src, ld, rows,
                     rows_p, cols, dst);
}

// C = A B^T (+ Cin), A [arows, k] and B [brows, k] in the forms af / bf
// (mfma_gemm.h): K32-blocked with 16-row block strides lda, ldb (elements),
// or K-outer with their ld and a_kvalid / b_kvalid lines holding data.
void launch_gemm(bool bf16, int af, const uint16_t* A, int64_t lda, int64_t arows, int64_t a_kvalid,
                 int bf, const uint16_t* B, int64_t ldb, int64_t brows, int64_t b_kvalid,
                 int64_t k, int64_t m_out, int64_t n_out, const float* cin, int64_t ldcin,
                 void* C, int64_t ldc, hipStream_t s) {
  const int mblocks = static_cast<int>((m_out + kT - 1) / kT);
  const int nblocks = static_cast<int>((n_out + kT - 1) / kT);
  const int ksteps = static_cast<int>(k / gemm::kK);
  const int akv = static_cast<int>(a_kvalid), bkv = static_cast<int>(b_kvalid);
#define ITL_GEMM(BF16, AF, BF)                                                                   \
  hipLaunchKernelGGL((gemm_out_kernel<BF16, AF, BF>), dim3(mblocks * nblocks),                   \
                     dim3(gemm::kThreads), 0, s, A, lda, arows, akv, B, ldb, brows, bkv, ksteps, \
                     mblocks, nblocks, m_out, n_out, cin, ldcin, C, ldc)
  constexpr int KC = gemm::kKContig, KO = gemm::kKOuter, KB = gemm::kKOuterBlocked;
  if (af == KC && bf == KC) {
    if (bf16) ITL_GEMM(true, KC, KC); else ITL_GEMM(false, KC, KC);
  } else if (af == KC && bf == KO) {
    if (bf16) ITL_GEMM(true, KC, KO); else ITL_GEMM(false, KC, KO);
  } else {  // af == KB, bf == KC
    if (bf16) ITL_GEMM(true, KB, KC); else ITL_GEMM(false, KB, KC);
  }
#undef ITL_GEMM
}

}  // namespace

int64_t linear_bwd_chunk(int64_t v, int64_t vocab_chunk) {
  const int64_t vp = round_tile(v);
  const int64_t c = vocab_chunk > 0 ? round_tile(vocab_chunk) : kDefaultChunk;
  return c < vp ? c : vp;
}

LinearBwdLayout linear_bwd_layout(int64_t n, int64_t h, int64_t v, int32_t flags,
                                  int64_t vocab_chunk) {
  const bool need_dh = flags & kBwdDhidden, need_dw = flags & kBwdDweight;
  const bool saved = flags & kBwdSaved;
  LinearBwdLayout l;
  l.np = round_tile(n);
  l.vp = round_tile(v);
  l.vc = linear_bwd_chunk(v, vocab_chunk);
  const int64_t nchunks = (l.vp + l.vc - 1) / l.vc;
  auto up = [](int64_t b) { return (b + 255) / 256 * 256; };
  int64_t off = 0;
  auto take = [&](bool use, int64_t bytes) {
    if (!use) return int64_t{-1};
    const int64_t at = off;
    off += up(bytes);
    return at;
  };
  l.hb = take(!saved, l.np * h * 2);                      // blocked h for the recompute
  l.ht = take(need_dw, h * l.np * 2);                     // h^T for dW
  l.dz = take(need_dh || need_dw, l.np * l.vc * 2);       // dz_c for dh and dW
  l.dh32 = take(need_dh && (flags & kBwdBf16Out) && nchunks > 1,
                n * h * 4);                               // fp32 dh between chunks
  l.total = off;
  return l;
}

void launch_linear_bwd(const uint16_t* hidden, int64_t ld_h, const uint16_t* weight, int64_t ld_w,
                       int64_t n, int64_t h, int64_t v, Targets targets, int64_t ignore,
                       const void* zsaved, int32_t z_bf16, int64_t ld_z,
                       const uint16_t* prepared, const float* lse,
                       const float* grad, float inv_t, int32_t round_bf16, const float* ent,
                       const float* gent, bool bf16_out, void* dh, int64_t ld_dh, void* dw,
                       int64_t ld_dw, int64_t vocab_chunk, char* ws, hipStream_t s) {
  if (n == 0) {
    // dh has no rows; dW is a sum over no tokens.
    if (dw) {
      const int64_t want = (v * h + 255) / 256;
      const unsigned blocks = static_cast<unsigned>(want < 8192 ? want : 8192);
      if (bf16_out)
        hipLaunchKernelGGL(fill_zero_kernel<true>, dim3(blocks), dim3(256), 0, s, dw, ld_dw, v, h);
      else
        hipLaunchKernelGGL(fill_zero_kernel<false>, dim3(blocks), dim3(256), 0, s, dw, ld_dw, v, h);
    }
    return;
  }
  const int32_t flags = (dh ? kBwdDhidden : 0) | (dw ? kBwdDweight : 0) |
                        (prepared ? kBwdPrepared : 0) | (zsaved ? kBwdSaved : 0) |
                        (bf16_out ? kBwdBf16Out : 0);
  const LinearBwdLayout l = linear_bwd_layout(n, h, v, flags, vocab_chunk);
  auto at = [&](int64_t off) { return off < 0 ? nullptr : reinterpret_cast<uint16_t*>(ws + off); };
  uint16_t* hb = at(l.hb);
  uint16_t* ht = at(l.ht);
  uint16_t* dz = at(l.dz);
  float* dh32 = l.dh32 < 0 ? nullptr : reinterpret_cast<float*>(ws + l.dh32);
  const int mblocks = static_cast<int>(l.np / kT), vblocks = static_cast<int>(l.vp / kT);
  const int64_t hsteps = h / gemm::kK, npsteps = l.np / gemm::kK, vpsteps = l.vp / gemm::kK;
  const bool plain = inv_t == 1.0f && !ent && !round_bf16;
  const uint16_t* wop = prepared ? prepared_blocked_w(prepared) : weight;
  const int64_t ldw = prepared ? int64_t{0} : ld_w;
  if (!zsaved) launch_block_rows(hidden, ld_h, n, l.np, h, hb, s);
  if (dw) launch_transpose(hidden, ld_h, n, l.np, h, ht, s);
  for (int64_t c0 = 0; c0 < l.vp; c0 += l.vc) {
    const int64_t c1 = c0 + l.vc < l.vp ? c0 + l.vc : l.vp;
    const int64_t cols = c1 - c0, csteps = cols / gemm::kK;
    const int vb0 = static_cast<int>(c0 / kT), vcb = static_cast<int>(cols / kT);
    const bool first = c0 == 0, last = c1 == l.vp;
    // dz_c of the chunk's columns
    if (!zsaved) {
#define ITL_DZ(WB, PL)                                                                            \
  hipLaunchKernelGGL((linear_dz_kernel<WB, PL>), dim3(mblocks * vcb), dim3(gemm::kThreads), 0,   \
                     s, hb, ld_h, wop, ldw, n, h, v, mblocks, vblocks, vb0, vcb, targets.p,      \
                     targets.is32, ignore, lse, grad, inv_t, round_bf16, ent, gent, dz)
      if (prepared) {
        if (plain) ITL_DZ(true, true); else ITL_DZ(true, false);
      } else {
        if (plain) ITL_DZ(false, true); else ITL_DZ(false, false);
      }
#undef ITL_DZ
    } else {
      const int64_t rt = l.np / kTR;
      const dim3 grid(static_cast<unsigned>(cols / kTC), static_cast<unsigned>(rt < 65535 ? rt : 65535));
      if (z_bf16)
        hipLaunchKernelGGL(linear_dz_saved_kernel<true>, grid, dim3(256), 0, s, zsaved, ld_z, n, v,
                           l.np, targets.p, targets.is32, ignore, lse, grad, inv_t, round_bf16, ent,
                           gent, c0, cols, dz);
      else
        hipLaunchKernelGGL(linear_dz_saved_kernel<false>, grid, dim3(256), 0, s, zsaved, ld_z, n,
                           v, l.np, targets.p, targets.is32, ignore, lse, grad, inv_t, round_bf16,
                           ent, gent, c0, cols, dz);
    }
    // dW[c0, c1) = dz_c^T h: K = every token, ascending (final rows); dz_c
    // read along its token axis (K-outer)
    if (dw && c0 < v) {
      const int64_t rows = (c1 < v ? c1 : v) - c0;
      launch_gemm(bf16_out, gemm::kKOuterBlocked, dz, csteps, cols, l.np, gemm::kKContig, ht,
                  npsteps * 512, h, -1, l.np, rows, h, nullptr, 0,
                  static_cast<char*>(dw) + c0 * ld_dw * (bf16_out ? 2 : 4), ld_dw, s);
    }
    // dh += dz_c W[c0, c1): K = the chunk's vocabulary, continuing the fp32
    // accumulators of the previous chunks (in dh itself for fp32 output, in
    // dh32 for bf16 output, rounded on the last chunk)
    if (dh) {
      const uint16_t* wtc;
      int64_t ldwt;
      if (prepared) {  // the prepared W^T [h, Vp]: columns [c0, c1)
        wtc = prepared_blocked_wt(prepared, v, h) + (c0 / gemm::kK) * 512;
        ldwt = vpsteps * 512;
      } else {  // W[c0, c1) as it is: K-outer, its rows the lines
        wtc = weight + c0 * ld_w;
        ldwt = ld_w;
      }
      const float* cin = first ? nullptr : (dh32 ? dh32 : static_cast<const float*>(dh));
      const int64_t ldcin = dh32 ? h : ld_dh;
      const bool out_bf16 = bf16_out && last;
      void* cout = bf16_out && !last ? static_cast<void*>(dh32) : dh;
      const int64_t ldc = bf16_out && !last ? h : ld_dh;
      launch_gemm(out_bf16, gemm::kKContig, dz, csteps * 512, l.np, -1,
                  prepared ? gemm::kKContig : gemm::kKOuter, wtc, ldwt, h,
                  prepared ? -1 : (c1 < v ? c1 : v) - c0, cols, n, h, cin, ldcin, cout, ldc, s);
    }
  }
  (void)hsteps;
}

int64_t prepared_bytes(int64_t v, int64_t h) { return 2 * h * round_tile(v) * 2; }

const uint16_t* prepared_blocked_wt(const uint16_t* p, int64_t v, int64_t h) {
  return p + h * round_tile(v);
}

void launch_prepare_weight(const uint16_t* weight, int64_t ld_w, int64_t v, int64_t h,
                           uint16_t* prepared, hipStream_t s) {
  const int64_t vp = round_tile(v);
  launch_block_rows(weight, ld_w, v, vp, h, prepared, s);
  launch_transpose(weight, ld_w, v, vp, h, prepared + h * vp, s);
}

void launch_block_rows(const uint16_t* src, int64_t ld, int64_t rows, int64_t rows_p, int64_t k,
                       uint16_t* dst, hipStream_t s, int* zero, int nzero) {
  const int64_t want = (rows_p * (k / 8) + 255) / 256;
  const unsigned blocks = static_cast<unsigned>(want < 1 ? 1 : want < 8192 ? want : 8192);
  hipLaunchKernelGGL(block_rows_bf16, dim3(blocks), dim3(256), 0, s, src, ld, rows, rows_p, k,
                     dst, zero, nzero);
}

}  // namespace itl
