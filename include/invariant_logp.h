/*
 * invariant_logp.h -- C ABI of the batch-invariant selected-token
 * log-probability library for AMD Instinct MI355X (gfx950).
 *
 * Operation ("Batch-Invariant LogP", opening definition and Reference
 * Semantics): for every row r of a [N, V] logits matrix with target t_r,
 *     logp[r] = logits[r, t_r] - logsumexp(logits[r, :])
 * A row whose target equals ignore_index outputs 0 and receives a zero
 * gradient; any other target outside [0, V) is invalid.
 *
 * Arithmetic contract ("Batch-Invariant LogP", Tensor Parallel; the contract
 * vocabulary of the RFC "[RFC][ROCm] End-to-end optimization of bitwise VIME
 * R/R beyond native P/P", section Contract boundary):
 *   - the vocabulary is cut into fixed tiles of tile_width columns over the
 *     global column index; columns >= V are -inf and never read;
 *   - every tile gives an fp32 pair (m_k = tile max, s_k = sum exp(x - m_k))
 *     through one fixed summation tree that depends only on the column
 *     position inside the tile, the tile width and the dtype;
 *   - the T = ceil(V / tile_width) pairs are merged in one fixed ascending
 *     order: M = max m_k, acc = fma(s_k, exp(m_k - M), acc),
 *     LSE = M + log(acc);
 *   - the target logit is copied from the tile that holds it, never summed;
 *     logp = target_logit - LSE in fp32.
 * Hence a row's output bits depend only on that row's logits, its target,
 * ignore_index and tile_width: not on N, on the row's position, on its
 * neighbours, on the launch geometry or on num_shards.
 *
 * Conventions for every entry point:
 *   - pointers are DEVICE pointers owned by the caller unless noted; the
 *     library allocates nothing, frees nothing and keeps no pointer after it
 *     returns;
 *   - work is enqueued on `hip_stream` (a hipStream_t; NULL = the default
 *     stream) and runs asynchronously; the caller keeps every buffer alive
 *     until the stream has finished it;
 *   - all arguments are checked on the host before any HIP call; on an error
 *     nothing is enqueued and no output is touched;
 *   - every output element is written, ignored rows included;
 *   - the return value is a logp_status code; no C++ exception crosses the
 *     ABI.
 */
#ifndef INVARIANT_LOGP_H
#define INVARIANT_LOGP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
enum logp_status {
  LOGP_OK = 0,
  LOGP_ERR_NULL = 1,      /* a required pointer is NULL */
  LOGP_ERR_SHAPE = 2,     /* n < 0, v < 1, ld < v, h < 1, or T too large */
  LOGP_ERR_DTYPE = 3,     /* unknown dtype code */
  LOGP_ERR_TILE = 4,      /* tile_width not supported for this dtype/op */
  LOGP_ERR_ALIGN = 5,     /* fused LM-head operand not 16-byte aligned */
  LOGP_ERR_SHARDS = 6,    /* num_shards < 1 or not a divisor of v */
  LOGP_ERR_WORKSPACE = 7, /* workspace NULL or smaller than required */
  LOGP_ERR_TARGET = 8,    /* validate = 1 found an active target outside [0, v) */
  LOGP_ERR_HIP = 9,       /* a HIP launch or copy failed */
  LOGP_ERR_VALUE = 10,    /* a scalar argument is out of range (temperature,
                             rounding), or the stream is not on the current
                             device (linear_logp_fwd_noalloc) */
  LOGP_ERR_SCRATCH = 11   /* linear_logp_fwd_noalloc: the call needs more than
                             LOGP_NOALLOC_SCRATCH_BYTES of scratch */
};

/* Logits element types ("Batch-Invariant LogP", Tensor Contract: fp32 / fp16
 * / bf16 logits). */
enum logp_dtype {
  LOGP_F32 = 0,   /* IEEE binary32 */
  LOGP_BF16 = 1,  /* bfloat16, widened exactly to fp32 before any arithmetic */
  LOGP_F16 = 2    /* IEEE binary16, widened exactly to fp32 before any arithmetic */
};

/* Target index types (the Tensor Contract's integer target_ids). */
enum logp_index_dtype {
  LOGP_I64 = 0,  /* int64 */
  LOGP_I32 = 1   /* int32 */
};

/* Rounding point of the fused LM head's logits ("[RFC][ROCm] End-to-end
 * optimization of bitwise VIME R/R beyond native P/P", Contract-versioned
 * arithmetic change and Workstream 1).  Where a value is rounded to bf16 is
 * part of a contract version, so fusing two steps must keep a bf16 rounding
 * that the unfused pair had.  LOGP_ROUND_BF16 selects the variant contract
 * whose statistics see the bf16 logits an unfused bf16 LM head stores. */
enum logp_rounding {
  LOGP_ROUND_NONE = 0,  /* statistics on the fp32 accumulators */
  LOGP_ROUND_BF16 = 1   /* statistics on RNE_bf16(accumulator), widened exactly */
};

/*
 * Workspace of logp_fwd, in bytes.  It is 0 for num_shards == 1 with
 * validate == 0 (the fused single-launch path).  Otherwise it holds the
 * [T, n] tile partials (m, s and the entropy moment w, fp32), the copied
 * target logits [n] and a 256-byte status block.  Returns 0 for arguments
 * logp_fwd would reject.
 */
size_t logp_fwd_workspace_bytes(int64_t n, int64_t v, int32_t tile_width,
                                int32_t num_shards, int32_t validate);

/*
 * Selected-token log-probability and row LSE ("Batch-Invariant LogP",
 * Entry Point, Tensor Contract and Tensor Parallel).
 *
 *   logits        [n, ld] row-major, first v columns used; dtype LOGP_F32,
 *                 LOGP_BF16 or LOGP_F16.  Any alignment is accepted; rows
 *                 whose start is 16-byte aligned stream with 128-bit loads.
 *   targets       [n] of target_dtype (LOGP_I64 or LOGP_I32; LOGP_ERR_DTYPE
 *                 otherwise).
 *   ignore_index  rows with this target give logp = +0, lse = +0 and are not
 *                 read.
 *   tile_width    vocabulary tile width W: 512, 1024, 2048, 4096 or 8192 for
 *                 bf16 and fp16; 256, 512, 1024, 2048 or 4096 for fp32.  T =
 *                 ceil(v / W) must not exceed 4096.  W is part of the
 *                 arithmetic contract (it fixes the summation tree).
 *   num_shards    S >= 1, v % S == 0: the vocabulary is split into S nominal
 *                 ranges of v/S columns; shard s owns the tiles whose first
 *                 column lies in its range, computes their partials in its own
 *                 launch into the shared [T, n] table (the byte-only
 *                 all-gather of the Tensor Parallel section), the owner of the
 *                 target's tile copies the target logit, and one merge launch
 *                 follows.  Results are bitwise equal for every S.
 *   validate      0: no synchronisation; an active row whose target is
 *                 outside [0, v) gets logp = NaN and nothing out of bounds is
 *                 read.  1: the same, then the call waits for the stream and
 *                 returns LOGP_ERR_TARGET if any such row was seen.
 *   logp_out      fp32 [n].
 *   lse_out       fp32 [n], may be NULL.  Saved for logp_bwd.
 *   entropy_out   fp32 [n] or NULL: the full-vocabulary entropy
 *                 H = -sum_j p_j log p_j of each row ("Batch-Invariant LogP",
 *                 VIME CP=2 runtime provider: entropy on request, merged in
 *                 the same fixed order).  Each tile also folds
 *                 w = sum e^(x - m) (x - m) in its sumexp tree; the merge
 *                 folds b = fma(fma(s_k, m_k - M, w_k), e^(m_k - M), b) next
 *                 to the LSE chain and H = log(acc) - b / acc.  Ignored rows
 *                 give 0.  logp and lse have the same bits with or without it.
 *   workspace     device buffer of at least logp_fwd_workspace_bytes(...)
 *                 bytes (may be NULL when that is 0), 256-byte aligned.
 */
int32_t logp_fwd(const void* logits, int32_t dtype, int64_t n, int64_t v,
                 int64_t ld, const void* targets, int32_t target_dtype,
                 int64_t ignore_index, int32_t tile_width, int32_t num_shards,
                 int32_t validate, float* logp_out, float* lse_out,
                 float* entropy_out, void* workspace, size_t workspace_bytes,
                 void* hip_stream);

/*
 * Gradient of logp with respect to the logits ("Batch-Invariant LogP",
 * Batch-Invariance: the tile-wise backward reusing the forward's per-row
 * LSE; Reference Semantics: ignored rows get a zero gradient).
 *
 *   dlogits[r, j] = RNE_dtype( g[r] * u ),  u = 1 - p if j == t_r, else -p,
 *   p = exp(x[r, j] - lse[r]) with the same exp primitive as the forward;
 *   with the entropy term, -gH[r] p (x - lse[r] + H[r]) is added by one fma
 *   before the rounding.
 *
 *   logits, dtype, n, v, ld, targets, target_dtype, ignore_index: as for
 *               logp_fwd.
 *   tile_width  accepted for symmetry with logp_fwd and checked the same
 *               way; it does not change any bit (the backward is elementwise).
 *   lse         fp32 [n] from logp_fwd.
 *   grad_logp   fp32 [n], the upstream gradient g.
 *   entropy, grad_entropy
 *               fp32 [n] each, both NULL (no entropy term) or both set: the
 *               row entropy from logp_fwd and its upstream gradient gH.
 *   dlogits_out [n, ld_out] of the logits dtype; ld_out >= v; columns >= v
 *               are not written.  Ignored rows are written +0 without reading
 *               the logits.  It may be exactly the logits buffer (same
 *               pointer and ld_out == ld: in place); partial overlap is
 *               undefined.  A row with an invalid target gets u = -p.
 */
int32_t logp_bwd(const void* logits, int32_t dtype, int64_t n, int64_t v,
                 int64_t ld, const void* targets, int32_t target_dtype,
                 int64_t ignore_index, int32_t tile_width, const float* lse,
                 const float* grad_logp, const float* entropy,
                 const float* grad_entropy, void* dlogits_out, int64_t ld_out,
                 void* hip_stream);

/*
 * Prepared LM-head weight ("[RFC][ROCm] End-to-end optimization of bitwise
 * VIME R/R beyond native P/P", Workstream 3: prepared [K, N] weights are
 * reused and refreshed when the weight changes): fills `prepared` (device,
 * caller-owned, prepared_bytes >= linear_logp_prepared_bytes(v, h), 16-byte
 * aligned) from weight [v, ld_w] bf16 with the weight re-laid for the
 * products' loads: the weight itself (for the forward and the backward's
 * recomputed logits) and its transpose (for the backward's dhidden), both
 * bf16 with the vocabulary padded with zeros to round_up(v, 256), in a
 * layout private to the library.  linear_logp_fwd and linear_logp_bwd read
 * it instead of the weight where it helps and give the same bits.  h a
 * multiple of 64.  Errors: LOGP_ERR_SHAPE (sizes, a short buffer),
 * LOGP_ERR_NULL, LOGP_ERR_ALIGN (weight rows or prepared not 16-byte
 * aligned).  Prepare again whenever the weight changes; a prepared buffer of
 * another weight gives wrong results, unchecked.  linear_logp_prepared_bytes
 * gives 2 * h * round_up(v, 256) * 2 (0 for arguments that are refused).
 */
size_t linear_logp_prepared_bytes(int64_t v, int64_t h);
int32_t linear_logp_prepare_weight(const void* weight, int64_t ld_w, int64_t v, int64_t h,
                                   void* prepared, size_t prepared_bytes, void* hip_stream);

/*
 * Workspace of linear_logp_fwd in bytes: the [n, T] partials (m, s, w) for
 * T = ceil(v / tile_width), the copied target logits [n] and, for n > 128, a
 * copy of hidden re-laid for the product's loads (round_up(n, 256) * h * 2
 * bytes) and 512 bytes of counters that hand out the product's last tiles
 * to whichever part of the GPU is free first.  Returns 0 for arguments
 * linear_logp_fwd would reject.
 */
size_t linear_logp_fwd_workspace_bytes(int64_t n, int64_t h, int64_t v, int32_t tile_width);

/*
 * Fused LM-head + selected-token log-probability ("[RFC][ROCm] End-to-end
 * optimization of bitwise VIME R/R beyond native P/P", Workstream 3):
 *   z[r, j] = sum_k hidden[r, k] * weight[j, k]   (fp32, never stored)
 *   logp[r] = z[r, t_r] - LSE(z[r, :])
 * The products run on bf16 MFMA with fp32 accumulation, one accumulator per
 * output, K walked in ascending fixed blocks with no split-K; the tile
 * statistics of the logp contract are taken on the fp32 z in the GEMM
 * epilogue, then merged in the fixed ascending order.
 *
 *   hidden      bf16 [n, ld_h], first h columns used.
 *   weight      bf16 [v, ld_w] (vocabulary-major LM-head weight).
 *   h           hidden size, a multiple of 64.
 *   tile_width  the statistic tile: must be 256 (the kernel's vocabulary
 *               block).
 *   hidden, weight, ld_h and ld_w must give 16-byte aligned rows
 *   (LOGP_ERR_ALIGN otherwise).
 *   targets, target_dtype, ignore_index, logp_out, lse_out (may be NULL),
 *   entropy_out (may be NULL): as logp_fwd, with no validation (invalid
 *   active targets give logp = NaN), taken over the scaled logits.
 *   temperature finite and > 0 with a finite fp32 reciprocal, i.e. at least
 *               about 2.9e-39 (LOGP_ERR_VALUE otherwise): the logits enter
 *               every statistic as z * fl32(1 / temperature) (the proposed
 *               operator's temperature, applied at this one point); 1 leaves
 *               them unchanged.
 *   logits_rounding
 *               LOGP_ROUND_NONE: z is the fp32 accumulator.  LOGP_ROUND_BF16:
 *               z is replaced by RNE_bf16(accumulator) before anything else
 *               (logits output, temperature, every statistic, the target
 *               copy).  Other values: LOGP_ERR_VALUE.
 *   logits_out  [n, ld_logits] (ld_logits >= v) of logits_dtype (LOGP_F32 or
 *               LOGP_BF16, RNE) receiving the unscaled z, or NULL ("return
 *               logits" for sampling).  logp, lse and entropy have the same
 *               bits either way.
 *   prepared, prepared_bytes
 *               NULL, or linear_logp_prepare_weight's buffer for this weight
 *               (short: LOGP_ERR_SHAPE; not 16-byte aligned: LOGP_ERR_ALIGN),
 *               read instead of weight; the same bits.
 *   workspace   at least linear_logp_fwd_workspace_bytes(...) bytes,
 *               256-byte aligned.
 */
int32_t linear_logp_fwd(const void* hidden, int64_t ld_h, const void* weight,
                        int64_t ld_w, int64_t n, int64_t h, int64_t v,
                        const void* targets, int32_t target_dtype,
                        int64_t ignore_index, int32_t tile_width, float temperature,
                        int32_t logits_rounding, float* logp_out, float* lse_out,
                        float* entropy_out,
                        void* logits_out, int32_t logits_dtype, int64_t ld_logits,
                        const void* prepared, size_t prepared_bytes,
                        void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * Size of the static scratch array behind linear_logp_fwd_noalloc: 64 MiB of
 * device memory on every GPU the library runs on, held until the process
 * ends.
 */
#define LOGP_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * linear_logp_fwd without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  Same arguments (minus workspace and
 * workspace_bytes), same kernels, same bits as linear_logp_fwd.
 *
 * Scratch: the library's static device array of LOGP_NOALLOC_SCRATCH_BYTES
 * bytes stands in for the workspace.  The call needs
 * linear_logp_fwd_workspace_bytes(n, h, v, tile_width) <=
 * LOGP_NOALLOC_SCRATCH_BYTES (at h = 4096, v = 151936 that is n <= 4352;
 * n <= 128 needs only the partial tables, 7 KiB per row at that v), else it
 * returns LOGP_ERR_SCRATCH with nothing enqueued.  It calls no allocator.
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents (no value in it has to start at zero: each one read is first
 * written by the same call), so calls that overlap on one GPU (two streams,
 * or two host threads) race and must be serialised by the caller.
 * The first call on a device looks up the array's device address with that
 * device current; hip_stream must belong to the current device
 * (LOGP_ERR_VALUE otherwise).  Make that first call outside graph capture.
 */
int32_t linear_logp_fwd_noalloc(const void* hidden, int64_t ld_h, const void* weight,
                                int64_t ld_w, int64_t n, int64_t h, int64_t v,
                                const void* targets, int32_t target_dtype,
                                int64_t ignore_index, int32_t tile_width, float temperature,
                                int32_t logits_rounding, float* logp_out, float* lse_out,
                                float* entropy_out,
                                void* logits_out, int32_t logits_dtype, int64_t ld_logits,
                                const void* prepared, size_t prepared_bytes, void* hip_stream);

/* Options of a linear_logp_bwd call, for its workspace size. */
enum logp_bwd_flags {
  LOGP_BWD_DHIDDEN = 1,       /* dhidden requested */
  LOGP_BWD_DWEIGHT = 2,       /* dweight requested */
  LOGP_BWD_PREPARED = 4,      /* a prepared weight is passed */
  LOGP_BWD_SAVED_LOGITS = 8,  /* the forward's logits are passed (no recompute) */
  LOGP_BWD_BF16_OUT = 16      /* out_dtype is LOGP_BF16 */
};

/*
 * Workspace of linear_logp_bwd in bytes for a call with these options
 * (flags: logp_bwd_flags of the call) and vocabulary chunk (vocab_chunk: as
 * linear_logp_bwd's).  The backward walks the vocabulary in chunks, so the
 * workspace holds one chunk's dz (bf16 [Np, C]; both products read it), a
 * re-laid copy of hidden ([Np, h], none with saved logits), hidden^T ([h,
 * Np], only for dweight) and, for bf16 dhidden over several chunks, the fp32
 * dhidden between chunks ([n, h]); Np = n rounded up to 256, C = the chunk
 * width.  The weight is read where it is (or from the prepared buffer).
 * About 0.34 GB at n = h = 4096, v = 151936 with the default chunk and both
 * outputs, prepared weight or not.  0 when n = 0 or for arguments
 * linear_logp_bwd would reject.
 */
size_t linear_logp_bwd_workspace_bytes(int64_t n, int64_t h, int64_t v, int32_t tile_width,
                                       int32_t flags, int64_t vocab_chunk);

/*
 * Backward of the fused LM head + log-probability ("[RFC][ROCm] End-to-end
 * optimization of bitwise VIME R/R beyond native P/P", Workstream 3: the
 * backward recomputes the fixed logit tiles from the saved LSE; "Batch-
 * Invariant LogP", Batch-Invariance and Reference Semantics: the logit
 * gradient is g * (onehot - softmax), zero on ignored rows):
 *   z  = hidden weight^T          (recomputed with the forward's MFMA walk,
 *                                  RNE_bf16 under LOGP_ROUND_BF16)
 *   x  = z * fl32(1 / temperature)
 *   dz = RNE_bf16((g * (onehot(t) - p) - gH p (x - lse + H)) * fl32(1 / temperature)),
 *        p = exp(x - lse), the entropy term only when requested
 *   dhidden = dz weight           (fp32 accumulation, K = vocabulary ascending)
 *   dweight = dz^T hidden         (fp32 accumulation, K = tokens ascending)
 * No product is split, so dhidden[r] depends only on row r and dweight is
 * deterministic for a given row order.
 *
 *   hidden, ld_h, weight, ld_w, n, h, v, targets, target_dtype,
 *   ignore_index, tile_width:
 *               as linear_logp_fwd (h a multiple of 64, tile_width 256,
 *               16-byte aligned rows).
 *   temperature, logits_rounding
 *               as linear_logp_fwd (the forward's values; the rounding is
 *               passed straight through, as an unfused bf16 LM head's
 *               gradient is).
 *   saved_logits, saved_dtype, ld_saved
 *               NULL: z is recomputed on the MFMA tile (no [n, v] memory is
 *               kept between forward and backward).  Otherwise the
 *               forward's unscaled logits output ([n, ld_saved], ld_saved
 *               >= v, 16-byte aligned rows, else LOGP_ERR_SHAPE /
 *               LOGP_ERR_ALIGN), read instead of recomputing z: the
 *               "retain logits" side of the memory trade-off the fused
 *               operator's backward leaves open.  The values are the same,
 *               so dhidden and dweight have the same bits either way.
 *               saved_dtype LOGP_F32, or LOGP_BF16 only with
 *               LOGP_ROUND_BF16 (where the bf16 logits are exactly z);
 *               otherwise LOGP_ERR_DTYPE.
 *   prepared, prepared_bytes
 *               NULL: the backward reads weight as it is.  Otherwise
 *               linear_logp_prepare_weight's buffer for this weight (short:
 *               LOGP_ERR_SHAPE; not 16-byte aligned: LOGP_ERR_ALIGN), read
 *               instead: the same values, so the same bits, in layouts that
 *               load faster (the prepared weight is reused while the weight
 *               does not change, e.g. over the micro-batches of one
 *               optimiser step).
 *   lse         fp32 [n] from linear_logp_fwd.
 *   grad_logp   fp32 [n], the upstream gradient g.
 *   entropy, grad_entropy
 *               fp32 [n] each, both NULL or both set: the forward's entropy
 *               and its upstream gradient gH.
 *   out_dtype   LOGP_F32 (the accumulators) or LOGP_BF16 (RNE of them).
 *   dhidden     [n, ld_dh] of out_dtype, or NULL to skip that product.
 *   dweight     [v, ld_dw] of out_dtype, or NULL to skip that product (with
 *               n = 0 it is written with zeros).  At least one is non-NULL.
 *               Both are overwritten, not accumulated into (an fp32 dhidden
 *               holds partial sums while the call runs).
 *   vocab_chunk vocabulary columns per pass (rounded up to a multiple of 256;
 *               0 = the library's default, 32768).  Per chunk the backward
 *               forms dz for those columns, finishes their dweight rows (K =
 *               every token, ascending) and continues the dhidden
 *               accumulators (K = vocabulary, ascending across the chunks).
 *               Any value gives the same bits; it trades workspace for
 *               launches.  Negative: LOGP_ERR_SHAPE.
 *   workspace   at least linear_logp_bwd_workspace_bytes(n, h, v, tile_width,
 *               <this call's flags>, vocab_chunk) bytes, 256-byte aligned
 *               (may be NULL when that is 0).
 * Active targets outside [0, v) are not checked: such a row gets no one-hot
 * term.
 */
int32_t linear_logp_bwd(const void* hidden, int64_t ld_h, const void* weight, int64_t ld_w,
                        int64_t n, int64_t h, int64_t v, const void* targets,
                        int32_t target_dtype, int64_t ignore_index, int32_t tile_width,
                        float temperature, int32_t logits_rounding, const void* saved_logits,
                        int32_t saved_dtype, int64_t ld_saved, const void* prepared,
                        size_t prepared_bytes, const float* lse, const float* grad_logp,
                        const float* entropy, const float* grad_entropy, int32_t out_dtype,
                        void* dhidden, int64_t ld_dh, void* dweight, int64_t ld_dw,
                        int64_t vocab_chunk, void* workspace, size_t workspace_bytes,
                        void* hip_stream);

/* Short English text for a status code (static storage, host memory). */
const char* logp_status_str(int32_t status);

/* Identifier of the arithmetic contracts this library implements (static
 * storage, host memory): tile tree, merge order, exp/log primitives, MFMA
 * form and K walk.  Two compiled libraries that report the same string
 * produce the same bits. */
const char* logp_contract_id(void);

#ifdef __cplusplus
}
#endif

#endif /* INVARIANT_LOGP_H */
