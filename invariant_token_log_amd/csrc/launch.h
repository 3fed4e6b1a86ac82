// Internal launchers (not part of the C ABI).  Arguments are checked by the
// callers in api.hip before any of these runs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace itl {

enum { kF32 = 0, kBF16 = 1, kF16 = 2 };

// Row targets as the caller stores them (int64 or int32), widened to int64 on
// read.  Kernels take the pointer as a __restrict__ parameter and build this
// view inside, so that uniform target reads stay scalar loads.
struct Targets {
  const void* p;
  int32_t is32;
  __host__ __device__ __forceinline__ int64_t operator[](int64_t r) const {
    return is32 ? static_cast<int64_t>(static_cast<const int32_t*>(p)[r])
                : static_cast<const int64_t*>(p)[r];
  }
};

void launch_fwd_fused(int dtype, bool vec, int chunks, const void* logits, int64_t ld,
                      int64_t n, int64_t v, Targets targets, int64_t ignore, int ntiles,
                      float* logp, float* lse, float* ent, int* status, hipStream_t s);

// pw == nullptr: no entropy moment.
void launch_fwd_partials(int dtype, bool vec, int chunks, const void* logits, int64_t ld,
                         int64_t n, int64_t v, Targets targets, int64_t ignore, int k_begin,
                         int k_end, float* pm, float* ps, float* pw, float* pt, hipStream_t s);

// Partial (r, k) of the [n, T] / [T, n] tables sits at r * row_stride + k * tile_stride.
// ent == nullptr: no entropy (pw unused).
void launch_fwd_merge(const float* pm, const float* ps, const float* pw, const float* pt,
                      int64_t n, int ntiles, int64_t row_stride, int64_t tile_stride, int64_t v,
                      Targets targets, int64_t ignore, float* logp, float* lse, float* ent,
                      int* status, hipStream_t s);

// ent == nullptr: no entropy term (gent unused).
void launch_bwd(int dtype, bool vec, const void* logits, int64_t ld, int64_t n, int64_t v,
                Targets targets, int64_t ignore, const float* lse, const float* grad,
                const float* ent, const float* gent, void* dlogits, int64_t ld_out,
                hipStream_t s);

// Fused LM-head statistics: writes the row-major [n, T] partials (and the
// entropy moments when pw is set) and the target logits of every active row
// (T = ceil(v / 256)).  The logits are multiplied by inv_t before any
// statistic; z (optional) receives the unscaled logits, fp32 or bf16.  wblk:
// the K32-blocked weight of a prepared weight (prepared_blocked_w), or null;
// the tiles then read it instead of weight (the same values).  hb:
// linear_fwd_blocked_bytes(n, h) bytes of scratch for the K32-blocked copy of
// hidden (unused, may be null, when that is 0).
void launch_linear_partials(const uint16_t* hidden, int64_t ld_h, const uint16_t* weight,
                            int64_t ld_w, int64_t n, int64_t h, int64_t v, Targets targets,
                            int64_t ignore, float* pm, float* ps, float* pt, float inv_t,
                            int32_t round_bf16, float* pw, void* z, int32_t z_bf16, int64_t ld_z,
                            const uint16_t* wblk, uint16_t* hb, hipStream_t s);

// Bytes of the forward's scratch: the blocked hidden copy (round_up(n, 256)
// * h * 2) and the tile-queue counters after it when the 256-row tile runs
// (n > 128), else 0.
int64_t linear_fwd_blocked_bytes(int64_t n, int64_t h);

constexpr int kLinearTile = 256;

// Compute units per XCD of the current device (its CU count / 8), looked up
// once per device.
int xcd_cus();

// Fused LM-head backward.  The vocabulary is walked in chunks of vc columns
// (a multiple of 256; kDefaultChunk unless the caller asks for another), so
// the workspace holds one chunk's dz_c [np, vc], the blocked hidden rows
// [np, h] (logits recomputed), h^T [h, np] (dW), and the fp32 dh [n, h]
// between chunks (bf16 dh over several chunks); only the
// regions the call uses (flags).  The weight needs no copy: dh reads it as
// it is, as a K-outer operand (or the prepared transpose).  Byte
// offsets, -1 for a region not used; np, vp = n, v rounded up to 256.
constexpr int64_t kDefaultChunk = 32768;
enum { kBwdDhidden = 1, kBwdDweight = 2, kBwdPrepared = 4, kBwdSaved = 8, kBwdBf16Out = 16 };
struct LinearBwdLayout {
  int64_t np, vp, vc;
  int64_t hb, ht, dz, dh32, total;
};
int64_t linear_bwd_chunk(int64_t v, int64_t vocab_chunk);
LinearBwdLayout linear_bwd_layout(int64_t n, int64_t h, int64_t v, int32_t flags,
                                  int64_t vocab_chunk);

// dh [n, h] and/or dW [v, h] (either may be null) as fp32 or bf16 (bf16_out).
// inv_t: reciprocal temperature (1 = none); ent / gent: row entropy and its
// upstream gradient (both null = no entropy term).  zsaved (fp32, or bf16
// with z_bf16; [n, ld_z]) holds the forward's unscaled logits to read instead
// of recomputing them, or is null.  prepared (or null) is the caller's
// prepared weight (launch_prepare_weight): its blocked W feeds the recomputed
// product and its W^T the dh product as K-contiguous operands (without it,
// the dh product reads W's rows in place as a K-outer operand, with the same
// bits).  vocab_chunk: columns per chunk (0 = kDefaultChunk), any value
// gives the same bits; ws: linear_bwd_layout(...).total bytes.
void launch_linear_bwd(const uint16_t* hidden, int64_t ld_h, const uint16_t* weight, int64_t ld_w,
                       int64_t n, int64_t h, int64_t v, Targets targets, int64_t ignore,
                       const void* zsaved, int32_t z_bf16, int64_t ld_z,
                       const uint16_t* prepared, const float* lse,
                       const float* grad, float inv_t, int32_t round_bf16, const float* ent,
                       const float* gent, bool bf16_out, void* dh, int64_t ld_dh, void* dw,
                       int64_t ld_dw, int64_t vocab_chunk, char* ws, hipStream_t s);

// Prepared weight, bf16, both parts K32-blocked (mfma_gemm.h) with vp =
// round_up(v, 256): W [vp rows, K = h] (rows v.. zero), then W^T [h rows,
// K = vp] (columns v.. zero), from W [v, ld_w]; prepared_bytes(v, h) bytes.
int64_t prepared_bytes(int64_t v, int64_t h);
inline const uint16_t* prepared_blocked_w(const uint16_t* p) { return p; }
const uint16_t* prepared_blocked_wt(const uint16_t* p, int64_t v, int64_t h);
void launch_prepare_weight(const uint16_t* weight, int64_t ld_w, int64_t v, int64_t h,
                           uint16_t* prepared, hipStream_t s);

// dst = the K32-blocked [rows_p, K = k] copy of src [rows, ld] (rows_p, k
// multiples of 16 and 32; rows past `rows` zero); also sets the nzero ints at
// zero (may be null) to 0.
void launch_block_rows(const uint16_t* src, int64_t ld, int64_t rows, int64_t rows_p, int64_t k,
                       uint16_t* dst, hipStream_t s, int* zero = nullptr, int nzero = 0);

}  // namespace itl
