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
// Kernels (the products on the 256 x 256 tile of mfma_gemm.h):
//   block_rows_bf16   : h [N, H] -> the K32-blocked copy the recomputed
//                       product reads;
//   linear_dz_kernel  : h x W^T tile -> dz in registers -> transposed, then
//                       row-major LDS tile -> dz^T [Vp, Np] and dz [Np, Vp];
//   linear_dz_saved_kernel: the same dz and dz^T from saved logits, 64 x 64
//                       tiles streamed through LDS;
//   transpose_block_bf16: W [V, H] -> W^T [H, Vp], h [N, H] -> h^T [H, Np];
//   gemm_out_kernel   : C = A B^T with fp32 or RNE-bf16 output.
// Every operand the backward writes for a product (dz, dz^T, W^T, h^T and
// the blocked h) is in the K32-blocked layout of mfma_gemm.h: the same
// values, read with whole-line loads.  Np, Vp are N and V rounded up to
// multiples of 256; padded rows and columns hold zeros and add exact zeros to
// the K walks.
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

// dst = the K32-blocked [gridDim.x * 64 rows, K = rows_p] operand with
// element (c, r) = r < rows ? src[r][c] : 0 (rows_p a multiple of 64).  64 x 64
// tiles through LDS; 16-byte global accesses.
__global__ __launch_bounds__(256) void transpose_block_bf16(const uint16_t* __restrict__ src,
                                                            int64_t ld_src, int64_t rows,
                                                            int64_t rows_p,
                                                            uint16_t* __restrict__ dst) {
  __shared__ uint16_t tile[64][64 + 2];
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * 64;
  const int t = threadIdx.x;
  for (int64_t r0 = static_cast<int64_t>(blockIdx.y) * 64; r0 < rows_p;
       r0 += static_cast<int64_t>(gridDim.y) * 64) {
    {
      const int r = t / 4, cs = (t % 4) * 16;
      uint4 a = make_uint4(0u, 0u, 0u, 0u), b = a;
      if (r0 + r < rows) {
        const uint16_t* p = src + (r0 + r) * ld_src + c0 + cs;
        a = *reinterpret_cast<const uint4*>(p);
        b = *reinterpret_cast<const uint4*>(p + 8);
      }
      const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        tile[r][cs + 2 * e] = static_cast<uint16_t>(w[e] & 0xffffu);
        tile[r][cs + 2 * e + 1] = static_cast<uint16_t>(w[e] >> 16);
      }
    }
    __syncthreads();
    {
      const int c = t / 4, rs = (t % 4) * 16;
      uint32_t w[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        w[e] = static_cast<uint32_t>(tile[rs + 2 * e][c]) |
               (static_cast<uint32_t>(tile[rs + 2 * e + 1][c]) << 16);
      uint16_t* p = dst + gemm::kblocked_index(c0 + c, r0 + rs, rows_p / gemm::kK);
      *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
      *reinterpret_cast<uint4*>(p + 8) = make_uint4(w[4], w[5], w[6], w[7]);
    }
    __syncthreads();
  }
}

// dst = the K32-blocked [rows_p, K = k] copy of src [rows, k] (rows past
// rows zero); one 16-byte chunk per thread in destination order.
__global__ __launch_bounds__(256) void block_rows_bf16(const uint16_t* __restrict__ src,
                                                       int64_t ld, int64_t rows, int64_t rows_p,
                                                       int64_t k, uint16_t* __restrict__ dst) {
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

// hidden K32-blocked (mblocks * 256 rows); weight row-major, or K32-blocked
// with vblocks * 256 rows when WBLK (a prepared weight).  PLAIN: launched
// only when no option is on (no rounding, T = 1, no entropy term), so the
// epilogue skips their operations instead of selecting around them.
template <bool WBLK, bool PLAIN>
__global__ __launch_bounds__(gemm::kThreads) void linear_dz_kernel(
    const uint16_t* __restrict__ hidden, int64_t ld_h, const uint16_t* __restrict__ weight,
    int64_t ld_w, int64_t n, int64_t hdim, int64_t v, int mblocks, int vblocks,
    const void* __restrict__ tgt, int32_t tgt32, int64_t ignore_index,
    const float* __restrict__ lse,
    const float* __restrict__ grad, float inv_t, int32_t round_bf16,
    const float* __restrict__ ent, const float* __restrict__ gent, uint16_t* __restrict__ dz,
    uint16_t* __restrict__ dzt) {
  const Targets targets{tgt, tgt32};
  __shared__ __align__(16) SmemDz sm;
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wave / 4, wn = wave % 4;
  const int li = lane % 16, g = lane / 16;

  int mb, vb;
  gemm::tile_coords(gemm::xcd_logical(blockIdx.x, mblocks * vblocks), mblocks, vblocks, mb, vb);
  const int64_t m0 = static_cast<int64_t>(mb) * kT;
  const int64_t v0 = static_cast<int64_t>(vb) * kT;
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
  gemm::mainloop<true, WBLK>(sm.u.st, hidden, 0, m0, static_cast<int64_t>(mblocks) * kT, weight,
                             ld_w, v0, WBLK ? static_cast<int64_t>(vblocks) * kT : v,
                             static_cast<int>(hdim / gemm::kK), acc);
  __syncthreads();

  // dz of every element (dz_value; 0 on ignored / padded rows and columns),
  // rounded to bf16.  Lane (li, g) holds rows 4g .. 4g+3 of each 16 x 16
  // block, so its four values of a column pack into 8 contiguous bytes of the
  // transposed tile.
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
  // dz^T: tile[c][r] (column-major), then out in K32-blocked order: 128
  // pieces of 16 rows x 32 tokens, one contiguous KiB each.
  const int64_t np_steps = static_cast<int64_t>(mblocks) * (kT / gemm::kK);
  const int64_t vp_steps = static_cast<int64_t>(vblocks) * (kT / gemm::kK);
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int lc = wn * 64 + j * 16 + li;
      const int lr = wm * 128 + i * 16 + 4 * g;
      *reinterpret_cast<uint2*>(&sm.u.tile[lc][lr]) = make_uint2(dv[i][j][0], dv[i][j][1]);
    }
  __syncthreads();
  for (int idx = tid; idx < kT * 32; idx += gemm::kThreads) {
    const int piece = idx >> 6, e = idx & 63;
    const int c = (piece >> 3) * 16 + (e >> 2), r = (piece & 7) * 32 + (e & 3) * 8;
    store_stream(dzt + gemm::kblocked_index(v0 + c, m0 + r, np_steps),
                 *reinterpret_cast<const uint4*>(&sm.u.tile[c][r]));
  }
  __syncthreads();
  // dz: tile[r][c] (row-major), then out in K32-blocked order.
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
    store_stream(dz + gemm::kblocked_index(m0 + r, v0 + c, vp_steps),
                 *reinterpret_cast<const uint4*>(&sm.u.tile[r][c]));
  }
}

// dz and dz^T from the forward's saved unscaled logits (fp32, or bf16 with
// ZBF16; [n, ld_z], 16-byte aligned rows) instead of the recomputed product:
// the same values through the same dz_value, so the same bits.  64 x 64
// tiles of [Np, Vp]: thread (r = tid / 4, 16 columns from (tid % 4) * 16)
// reads its 16 logits with 16-byte loads, writes its 16 dz along the row,
// and the tile leaves transposed through LDS for dz^T (both K32-blocked).
// Rows past n or ignored, and columns past v, get 0 without reading the
// logits.
constexpr int kST = 64;

template <bool ZBF16>
__global__ __launch_bounds__(256) void linear_dz_saved_kernel(
    const void* __restrict__ zsaved, int64_t ld_z, int64_t n, int64_t v, int64_t np_rows,
    const void* __restrict__ tgt, int32_t tgt32, int64_t ignore_index,
    const float* __restrict__ lse, const float* __restrict__ grad, float inv_t,
    int32_t round_bf16, const float* __restrict__ ent, const float* __restrict__ gent,
    int64_t vp_cols, uint16_t* __restrict__ dz, uint16_t* __restrict__ dzt) {
  const Targets targets{tgt, tgt32};
  __shared__ uint16_t tile[kST][kST + 8];
  const int tid = threadIdx.x;
  const int r = tid / 4, cs = (tid % 4) * 16;
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * kST;
  const bool scaled = inv_t != 1.0f;
  const bool with_ent = ent != nullptr;
  for (int64_t r0 = static_cast<int64_t>(blockIdx.y) * kST; r0 < np_rows;
       r0 += static_cast<int64_t>(gridDim.y) * kST) {
    const int64_t row = r0 + r;
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
    const bool live = row < n && t != ignore_index;
    float zv[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) zv[u] = 0.0f;
    const int64_t col = c0 + cs;
    if (live) {
      if (col + 16 <= v) {
        if constexpr (ZBF16) {
          const uint16_t* p = static_cast<const uint16_t*>(zsaved) + row * ld_z + col;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const uint4 w = load_stream(p + 8 * h);
            const uint32_t q[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              zv[8 * h + 2 * e] = bf16_lo(q[e]);
              zv[8 * h + 2 * e + 1] = bf16_hi(q[e]);
            }
          }
        } else {
          const float* p = static_cast<const float*>(zsaved) + row * ld_z + col;
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            const uint4 w = load_stream(p + 4 * h);
            zv[4 * h] = __uint_as_float(w.x);
            zv[4 * h + 1] = __uint_as_float(w.y);
            zv[4 * h + 2] = __uint_as_float(w.z);
            zv[4 * h + 3] = __uint_as_float(w.w);
          }
        }
      } else {
#pragma unroll
        for (int u = 0; u < 16; ++u)
          if (col + u < v)
            zv[u] = ZBF16 ? bf16_lo(static_cast<const uint16_t*>(zsaved)[row * ld_z + col + u])
                          : static_cast<const float*>(zsaved)[row * ld_z + col + u];
      }
    }
    uint32_t packed[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint16_t b[2];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int u = 2 * e + k;
        const float d = live && col + u < v
                            ? dz_value(zv[u], L, G, H, NGH, col + u == t, inv_t, scaled,
                                       with_ent, round_bf16)
                            : 0.0f;
        b[k] = bf16_bits(d);
        tile[r][cs + u] = b[k];
      }
      packed[e] = static_cast<uint32_t>(b[0]) | (static_cast<uint32_t>(b[1]) << 16);
    }
    uint16_t* o = dz + gemm::kblocked_index(row, col, vp_cols / gemm::kK);
    store_stream(o, make_uint4(packed[0], packed[1], packed[2], packed[3]));
    store_stream(o + 8, make_uint4(packed[4], packed[5], packed[6], packed[7]));
    __syncthreads();
    {
      const int c = tid / 4, rs = (tid % 4) * 16;
      uint32_t w[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        w[e] = static_cast<uint32_t>(tile[rs + 2 * e][c]) |
               (static_cast<uint32_t>(tile[rs + 2 * e + 1][c]) << 16);
      uint16_t* q = dzt + gemm::kblocked_index(c0 + c, r0 + rs, np_rows / gemm::kK);
      store_stream(q, make_uint4(w[0], w[1], w[2], w[3]));
      store_stream(q + 8, make_uint4(w[4], w[5], w[6], w[7]));
    }
    __syncthreads();
  }
}

// C[m_out, n_out] = A[., K] B[., K]^T on the mfma_gemm.h tile, both operands
// K32-blocked; BF16OUT rounds the fp32 accumulators to bf16 (RNE) on the way
// out.
template <bool BF16OUT>
__global__ __launch_bounds__(gemm::kThreads) void gemm_out_kernel(
    const uint16_t* __restrict__ A, int64_t lda, int64_t arows, const uint16_t* __restrict__ B,
    int64_t ldb, int64_t brows, int ksteps, int mblocks, int nblocks, int64_t m_out,
    int64_t n_out, void* __restrict__ C, int64_t ldc) {
  __shared__ __align__(16) gemm::Stages st;
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wave / 4, wn = wave % 4;
  const int li = lane % 16, g = lane / 16;
  int mb, nb;
  gemm::tile_coords(gemm::xcd_logical(blockIdx.x, mblocks * nblocks), mblocks, nblocks, mb, nb);
  const int64_t m0 = static_cast<int64_t>(mb) * kT;
  const int64_t n0 = static_cast<int64_t>(nb) * kT;
  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  gemm::mainloop<true, true>(st, A, lda, m0, arows, B, ldb, n0, brows, ksteps, acc);
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t row = m0 + wm * 128 + i * 16 + 4 * g + q;
      if (row >= m_out) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t col = n0 + wn * 64 + j * 16 + li;
        if (col < n_out) {
          if (BF16OUT)
            static_cast<uint16_t*>(C)[row * ldc + col] = bf16_bits(acc[i][j][q]);
          else
            static_cast<float*>(C)[row * ldc + col] = acc[i][j][q];
        }
      }
    }
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

// grid rows of a transpose over rows_p (grid-stride beyond 65535 blocks)
unsigned tgrid(int64_t rows_p) {
  const int64_t b = rows_p / 64;
  return static_cast<unsigned>(b < 65535 ? b : 65535);
}

// C = A B^T, A [arows, k] and B [brows, k] K32-blocked.
void launch_gemm(bool bf16, const uint16_t* A, int64_t arows, const uint16_t* B, int64_t brows,
                 int64_t k, int64_t m_out, int64_t n_out, void* C, int64_t ldc, hipStream_t s) {
  const int mblocks = static_cast<int>((m_out + kT - 1) / kT);
  const int nblocks = static_cast<int>((n_out + kT - 1) / kT);
  const int ksteps = static_cast<int>(k / gemm::kK);
  if (bf16)
    hipLaunchKernelGGL(gemm_out_kernel<true>, dim3(mblocks * nblocks), dim3(gemm::kThreads), 0, s,
                       A, int64_t{0}, arows, B, int64_t{0}, brows, ksteps, mblocks, nblocks,
                       m_out, n_out, C, ldc);
  else
    hipLaunchKernelGGL(gemm_out_kernel<false>, dim3(mblocks * nblocks), dim3(gemm::kThreads), 0,
                       s, A, int64_t{0}, arows, B, int64_t{0}, brows, ksteps, mblocks, nblocks,
                       m_out, n_out, C, ldc);
}

}  // namespace

LinearBwdLayout linear_bwd_layout(int64_t n, int64_t h, int64_t v) {
  const int64_t np = round_tile(n), vp = round_tile(v);
  auto up = [](int64_t b) { return (b + 255) / 256 * 256; };
  LinearBwdLayout l;
  l.np = np;
  l.vp = vp;
  l.wt = 0;
  l.ht = l.wt + up(h * vp * 2);
  l.dz = l.ht + up(h * np * 2);
  l.dzt = l.dz + up(np * vp * 2);
  l.hb = l.dzt + up(vp * np * 2);
  l.total = l.hb + up(np * h * 2);
  return l;
}

void launch_linear_bwd(const uint16_t* hidden, int64_t ld_h, const uint16_t* weight, int64_t ld_w,
                       int64_t n, int64_t h, int64_t v, Targets targets, int64_t ignore,
                       const void* zsaved, int32_t z_bf16, int64_t ld_z,
                       const uint16_t* prepared, const float* lse,
                       const float* grad, float inv_t, int32_t round_bf16, const float* ent,
                       const float* gent, bool bf16_out, void* dh, int64_t ld_dh, void* dw,
                       int64_t ld_dw, char* ws, hipStream_t s) {
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
  const LinearBwdLayout l = linear_bwd_layout(n, h, v);
  uint16_t* wt = reinterpret_cast<uint16_t*>(ws + l.wt);
  uint16_t* ht = reinterpret_cast<uint16_t*>(ws + l.ht);
  uint16_t* dz = reinterpret_cast<uint16_t*>(ws + l.dz);
  uint16_t* dzt = reinterpret_cast<uint16_t*>(ws + l.dzt);
  uint16_t* hb = reinterpret_cast<uint16_t*>(ws + l.hb);
  const int mblocks = static_cast<int>(l.np / kT), vblocks = static_cast<int>(l.vp / kT);
  if (!zsaved) {
    launch_block_rows(hidden, ld_h, n, l.np, h, hb, s);
    const bool plain = inv_t == 1.0f && !ent && !round_bf16;
    const uint16_t* wop = prepared ? prepared_blocked_w(prepared) : weight;
    const int64_t ldw = prepared ? int64_t{0} : ld_w;
#define ITL_DZ(WB, PL)                                                                           \
  hipLaunchKernelGGL((linear_dz_kernel<WB, PL>), dim3(mblocks * vblocks), dim3(gemm::kThreads), \
                     0, s, hb, ld_h, wop, ldw, n, h, v, mblocks, vblocks, targets.p,            \
                     targets.is32, ignore, lse, grad, inv_t, round_bf16, ent, gent, dz, dzt)
    if (prepared) {
      if (plain) ITL_DZ(true, true); else ITL_DZ(true, false);
    } else {
      if (plain) ITL_DZ(false, true); else ITL_DZ(false, false);
    }
#undef ITL_DZ
  } else {
    const int64_t rb = l.np / kST;
    const dim3 grid(static_cast<unsigned>(l.vp / kST), static_cast<unsigned>(rb < 65535 ? rb : 65535));
    if (z_bf16)
      hipLaunchKernelGGL(linear_dz_saved_kernel<true>, grid, dim3(256), 0, s, zsaved, ld_z, n, v,
                         l.np, targets.p, targets.is32, ignore, lse, grad, inv_t, round_bf16, ent,
                         gent, l.vp, dz, dzt);
    else
      hipLaunchKernelGGL(linear_dz_saved_kernel<false>, grid, dim3(256), 0, s, zsaved, ld_z, n,
                         v, l.np, targets.p, targets.is32, ignore, lse, grad, inv_t, round_bf16,
                         ent, gent, l.vp, dz, dzt);
  }
  if (dh) {
    // W^T: the caller's prepared copy (linear_logp_prepare_weight, the same
    // values) or made here
    const uint16_t* wtb = prepared ? prepared_blocked_wt(prepared, v, h) : wt;
    if (!prepared)
      hipLaunchKernelGGL(transpose_block_bf16, dim3(static_cast<unsigned>(h / 64), tgrid(l.vp)),
                         dim3(256), 0, s, weight, ld_w, v, l.vp, wt);
    launch_gemm(bf16_out, dz, l.np, wtb, h, l.vp, n, h, dh, ld_dh, s);
  }
  if (dw) {
    hipLaunchKernelGGL(transpose_block_bf16, dim3(static_cast<unsigned>(h / 64), tgrid(l.np)),
                       dim3(256), 0, s, hidden, ld_h, n, l.np, ht);
    launch_gemm(bf16_out, dzt, l.vp, ht, h, l.np, v, h, dw, ld_dw, s);
  }
}

int64_t prepared_bytes(int64_t v, int64_t h) { return 2 * h * round_tile(v) * 2; }

const uint16_t* prepared_blocked_wt(const uint16_t* p, int64_t v, int64_t h) {
  return p + h * round_tile(v);
}

void launch_prepare_weight(const uint16_t* weight, int64_t ld_w, int64_t v, int64_t h,
                           uint16_t* prepared, hipStream_t s) {
  const int64_t vp = round_tile(v);
  launch_block_rows(weight, ld_w, v, vp, h, prepared, s);
  hipLaunchKernelGGL(transpose_block_bf16, dim3(static_cast<unsigned>(h / 64), tgrid(vp)),
                     dim3(256), 0, s, weight, ld_w, v, vp, prepared + h * vp);
}

void launch_block_rows(const uint16_t* src, int64_t ld, int64_t rows, int64_t rows_p, int64_t k,
                       uint16_t* dst, hipStream_t s) {
  const int64_t want = (rows_p * (k / 8) + 255) / 256;
  const unsigned blocks = static_cast<unsigned>(want < 8192 ? want : 8192);
  hipLaunchKernelGGL(block_rows_bf16, dim3(blocks), dim3(256), 0, s, src, ld, rows, rows_p, k,
                     dst);
}

}  // namespace itl
