// C ABI of the library: argument checks (all before any HIP call), workspace
// layout, and the launch sequence of each entry point.
#include "invariant_logp.h"
#include "launch.h"

#include <cmath>
#include <mutex>

namespace {

static_assert(itl::kBwdDhidden == LOGP_BWD_DHIDDEN && itl::kBwdDweight == LOGP_BWD_DWEIGHT &&
                  itl::kBwdPrepared == LOGP_BWD_PREPARED &&
                  itl::kBwdSaved == LOGP_BWD_SAVED_LOGITS && itl::kBwdBf16Out == LOGP_BWD_BF16_OUT,
              "backward option flags");

constexpr int kMaxTiles = 4096;
constexpr size_t kAlign = 256;

size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Chunks per lane for a supported (dtype, tile width), else 0.
int chunks_for(int32_t dtype, int32_t w) {
  const int per = dtype == LOGP_F32 ? 256 : 512;  // one 16-byte chunk per lane
  if (w < per || w % per) return 0;
  const int c = w / per;
  return (c == 1 || c == 2 || c == 4 || c == 8 || c == 16) ? c : 0;
}

int elt_size(int32_t dtype) { return dtype == LOGP_F32 ? 4 : 2; }

bool valid_dtype(int32_t dtype) {
  return dtype == LOGP_F32 || dtype == LOGP_BF16 || dtype == LOGP_F16;
}

bool valid_index(int32_t target_dtype) {
  return target_dtype == LOGP_I64 || target_dtype == LOGP_I32;
}

itl::Targets targets_of(const void* p, int32_t target_dtype) {
  return itl::Targets{p, target_dtype == LOGP_I32 ? 1 : 0};
}

// Temperature of the fused LM head.  The logits are multiplied by its
// reciprocal rounded once to fp32 (1 stays exactly 1), so a temperature is
// usable when it is finite, > 0 and that reciprocal is finite too (below
// about 2.9e-39 it overflows to +inf, which would turn every logit into inf
// or NaN).
float inv_temperature(float t) { return static_cast<float>(1.0 / static_cast<double>(t)); }
bool valid_temperature(float t) {
  return std::isfinite(t) && t > 0.0f && std::isfinite(inv_temperature(t));
}
bool valid_rounding(int32_t r) { return r == LOGP_ROUND_NONE || r == LOGP_ROUND_BF16; }

bool aligned16(const void* p, int64_t ld, int32_t dtype) {
  return (reinterpret_cast<uintptr_t>(p) % 16 == 0) && ((ld * elt_size(dtype)) % 16 == 0);
}

// Common checks of logp_fwd / logp_bwd that involve no pointer.
int32_t check_stream_args(int32_t dtype, int64_t n, int64_t v, int64_t ld, int32_t w) {
  if (!valid_dtype(dtype)) return LOGP_ERR_DTYPE;
  if (n < 0 || v < 1 || ld < v) return LOGP_ERR_SHAPE;
  if (chunks_for(dtype, w) == 0) return LOGP_ERR_TILE;
  if ((v + w - 1) / w > kMaxTiles) return LOGP_ERR_SHAPE;
  return LOGP_OK;
}

// Workspace layout of logp_fwd and of the fused LM head's partials:
// [status block | pm | ps | pw | pt (n)], each table T x n fp32.
struct FwdLayout {
  size_t pm, ps, pw, pt, total;
};

FwdLayout fwd_layout(int64_t n, int64_t ntiles, bool tables, int32_t validate) {
  FwdLayout l{0, 0, 0, 0, 0};
  if (!tables) {
    l.total = validate ? kAlign : 0;
    return l;
  }
  const size_t table =
      round_up(static_cast<size_t>(ntiles) * static_cast<size_t>(n) * sizeof(float));
  l.pm = kAlign;
  l.ps = l.pm + table;
  l.pw = l.ps + table;
  l.pt = l.pw + table;
  l.total = l.pt + round_up(static_cast<size_t>(n) * sizeof(float));
  return l;
}

// The fused forward's workspace: the partial tables, then the blocked hidden.
size_t linear_fwd_total(int64_t n, int64_t h, int64_t ntiles, size_t* hb_offset) {
  const size_t tables = fwd_layout(n, ntiles, true, 0).total;
  if (hb_offset) *hb_offset = round_up(tables);
  return round_up(tables) + round_up(static_cast<size_t>(itl::linear_fwd_blocked_bytes(n, h)));
}

int32_t hip_status() {
  return hipGetLastError() == hipSuccess ? LOGP_OK : LOGP_ERR_HIP;
}

// ---------------------------------------------------------------------------
// Static scratch of linear_logp_fwd_noalloc: one array per GPU (each device
// that loads the library holds its own copy until the process ends).  In
// host code `scratch` names a host-side stand-in, not device memory: its
// device address is looked up once per device (hipGetSymbolAddress with that
// device current) and only that address is ever handed to kernels.
// ---------------------------------------------------------------------------
__device__ __align__(256) unsigned char scratch[LOGP_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array (looked up on the
// first call on that device).  The stream, when given, must belong to the
// current device.
int32_t static_scratch(hipStream_t s, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return LOGP_ERR_HIP;
  if (s) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(s, &sdev) != hipSuccess) return LOGP_ERR_HIP;
    if (sdev != dev) return LOGP_ERR_VALUE;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return LOGP_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return LOGP_OK;
}

// linear_logp_fwd with the caller's workspace, or (use_static) with the
// current device's static scratch array in its place.
int32_t linear_fwd_run(const void* hidden, int64_t ld_h, const void* weight, int64_t ld_w,
                       int64_t n, int64_t h, int64_t v, const void* targets,
                       int32_t target_dtype, int64_t ignore_index, int32_t tile_width,
                       float temperature, int32_t logits_rounding, float* logp_out,
                       float* lse_out, float* entropy_out, void* logits_out,
                       int32_t logits_dtype, int64_t ld_logits, const void* prepared,
                       size_t prepared_bytes, void* workspace, size_t workspace_bytes,
                       bool use_static, void* hip_stream) {

  if (n < 0 || v < 1 || h < 1 || h % 64 || ld_h < h || ld_w < h) return LOGP_ERR_SHAPE;
  if (!valid_index(target_dtype)) return LOGP_ERR_DTYPE;
  if (logits_out && logits_dtype != LOGP_F32 && logits_dtype != LOGP_BF16) return LOGP_ERR_DTYPE;
  if (logits_out && ld_logits < v) return LOGP_ERR_SHAPE;
  if (!valid_temperature(temperature) || !valid_rounding(logits_rounding)) return LOGP_ERR_VALUE;
  const itl::Targets tg = targets_of(targets, target_dtype);
  if (tile_width != itl::kLinearTile) return LOGP_ERR_TILE;
  const int64_t ntiles = (v + tile_width - 1) / tile_width;
  if (ntiles > (int64_t{1} << 24) || (n + 127) / 128 * ntiles > (int64_t{1} << 30))
    return LOGP_ERR_SHAPE;
  const FwdLayout lay = fwd_layout(n, ntiles, true, 0);
  size_t hb_off = 0;
  const size_t need = linear_fwd_total(n, h, ntiles, &hb_off);
  if (n == 0) return LOGP_OK;
  if (!hidden || !weight || !targets || !logp_out) return LOGP_ERR_NULL;
  if (!aligned16(hidden, ld_h, LOGP_BF16) || !aligned16(weight, ld_w, LOGP_BF16))
    return LOGP_ERR_ALIGN;
  if (prepared) {
    if (prepared_bytes < linear_logp_prepared_bytes(v, h)) return LOGP_ERR_SHAPE;
    if (reinterpret_cast<uintptr_t>(prepared) % 16) return LOGP_ERR_ALIGN;
  }
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  if (use_static) {
    if (need > LOGP_NOALLOC_SCRATCH_BYTES) return LOGP_ERR_SCRATCH;
    const int32_t st = static_scratch(s, &workspace);
    if (st != LOGP_OK) return st;
  } else if (!workspace || workspace_bytes < need ||
             reinterpret_cast<uintptr_t>(workspace) % kAlign) {
    return LOGP_ERR_WORKSPACE;
  }
  char* ws = static_cast<char*>(workspace);
  float* pm = reinterpret_cast<float*>(ws + lay.pm);
  float* ps = reinterpret_cast<float*>(ws + lay.ps);
  float* pw = entropy_out ? reinterpret_cast<float*>(ws + lay.pw) : nullptr;
  float* pt = reinterpret_cast<float*>(ws + lay.pt);
  (void)hipGetLastError();
  itl::launch_linear_partials(static_cast<const uint16_t*>(hidden), ld_h,
                              static_cast<const uint16_t*>(weight), ld_w, n, h, v, tg,
                              ignore_index, pm, ps, pt, inv_temperature(temperature),
                              logits_rounding == LOGP_ROUND_BF16 ? 1 : 0, pw, logits_out,
                              logits_dtype == LOGP_BF16 ? 1 : 0, ld_logits,
                              prepared ? itl::prepared_blocked_w(
                                             static_cast<const uint16_t*>(prepared))
                                       : nullptr,
                              reinterpret_cast<uint16_t*>(ws + hb_off), s);
  itl::launch_fwd_merge(pm, ps, pw, pt, n, static_cast<int>(ntiles), ntiles, 1, v, tg,
                        ignore_index, logp_out, lse_out, entropy_out, nullptr, s);
  return hip_status();
}

}  // namespace

extern "C" {

size_t logp_fwd_workspace_bytes(int64_t n, int64_t v, int32_t tile_width, int32_t num_shards,
                                int32_t validate) {
  if (check_stream_args(LOGP_BF16, n, v, v, tile_width) != LOGP_OK &&
      check_stream_args(LOGP_F32, n, v, v, tile_width) != LOGP_OK)
    return 0;
  if (num_shards < 1 || v % num_shards) return 0;
  return fwd_layout(n, (v + tile_width - 1) / tile_width, num_shards > 1, validate).total;
}

int32_t logp_fwd(const void* logits, int32_t dtype, int64_t n, int64_t v, int64_t ld,
                 const void* targets, int32_t target_dtype, int64_t ignore_index,
                 int32_t tile_width, int32_t num_shards, int32_t validate, float* logp_out,
                 float* lse_out, float* entropy_out, void* workspace, size_t workspace_bytes,
                 void* hip_stream) {
  int32_t st = check_stream_args(dtype, n, v, ld, tile_width);
  if (st != LOGP_OK) return st;
  if (!valid_index(target_dtype)) return LOGP_ERR_DTYPE;
  const itl::Targets tg = targets_of(targets, target_dtype);
  if (num_shards < 1 || v % num_shards) return LOGP_ERR_SHARDS;
  const int ntiles = static_cast<int>((v + tile_width - 1) / tile_width);
  const FwdLayout lay = fwd_layout(n, ntiles, num_shards > 1, validate);
  if (n == 0) return LOGP_OK;
  if (!logits || !targets || !logp_out) return LOGP_ERR_NULL;
  if (lay.total) {
    if (!workspace || workspace_bytes < lay.total ||
        reinterpret_cast<uintptr_t>(workspace) % kAlign)
      return LOGP_ERR_WORKSPACE;
  }
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  char* ws = static_cast<char*>(workspace);
  int* status = validate ? reinterpret_cast<int*>(ws) : nullptr;
  const int chunks = chunks_for(dtype, tile_width);
  const bool vec = aligned16(logits, ld, dtype);
  (void)hipGetLastError();
  if (status && hipMemsetAsync(status, 0, sizeof(int), s) != hipSuccess) return LOGP_ERR_HIP;
  if (num_shards == 1) {
    itl::launch_fwd_fused(dtype, vec, chunks, logits, ld, n, v, tg, ignore_index, ntiles,
                          logp_out, lse_out, entropy_out, status, s);
  } else {
    float* pm = reinterpret_cast<float*>(ws + lay.pm);
    float* ps = reinterpret_cast<float*>(ws + lay.ps);
    float* pw = entropy_out ? reinterpret_cast<float*>(ws + lay.pw) : nullptr;
    float* pt = reinterpret_cast<float*>(ws + lay.pt);
    const int64_t per = v / num_shards;
    for (int32_t sh = 0; sh < num_shards; ++sh) {
      // Shard sh owns the tiles whose first column lies in [sh*per, (sh+1)*per).
      const int kb = static_cast<int>((sh * per + tile_width - 1) / tile_width);
      const int ke = static_cast<int>(((sh + 1) * per + tile_width - 1) / tile_width);
      if (ke > kb)
        itl::launch_fwd_partials(dtype, vec, chunks, logits, ld, n, v, tg, ignore_index, kb,
                                 ke, pm, ps, pw, pt, s);
    }
    itl::launch_fwd_merge(pm, ps, pw, pt, n, ntiles, 1, n, v, tg, ignore_index, logp_out,
                          lse_out, entropy_out, status, s);
  }
  st = hip_status();
  if (st != LOGP_OK) return st;
  if (status) {
    int flag = 0;
    if (hipMemcpyAsync(&flag, status, sizeof(int), hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
      return LOGP_ERR_HIP;
    if (flag) return LOGP_ERR_TARGET;
  }
  return LOGP_OK;
}

int32_t logp_bwd(const void* logits, int32_t dtype, int64_t n, int64_t v, int64_t ld,
                 const void* targets, int32_t target_dtype, int64_t ignore_index,
                 int32_t tile_width, const float* lse, const float* grad_logp,
                 const float* entropy, const float* grad_entropy, void* dlogits_out,
                 int64_t ld_out, void* hip_stream) {
  int32_t st = check_stream_args(dtype, n, v, ld, tile_width);
  if (st != LOGP_OK) return st;
  if (!valid_index(target_dtype)) return LOGP_ERR_DTYPE;
  if (ld_out < v) return LOGP_ERR_SHAPE;
  if (n == 0) return LOGP_OK;
  if (!logits || !targets || !lse || !grad_logp || !dlogits_out) return LOGP_ERR_NULL;
  if ((entropy == nullptr) != (grad_entropy == nullptr)) return LOGP_ERR_NULL;
  const bool vec = aligned16(logits, ld, dtype) && aligned16(dlogits_out, ld_out, dtype);
  (void)hipGetLastError();
  itl::launch_bwd(dtype, vec, logits, ld, n, v, targets_of(targets, target_dtype), ignore_index,
                  lse, grad_logp, entropy, grad_entropy, dlogits_out, ld_out,
                  static_cast<hipStream_t>(hip_stream));
  return hip_status();
}

size_t linear_logp_fwd_workspace_bytes(int64_t n, int64_t h, int64_t v, int32_t tile_width) {
  if (n < 0 || v < 1 || h < 64 || h % 64 || tile_width != itl::kLinearTile) return 0;
  const int64_t ntiles = (v + tile_width - 1) / tile_width;
  return linear_fwd_total(n, h, ntiles, nullptr);
}

int32_t linear_logp_fwd(const void* hidden, int64_t ld_h, const void* weight, int64_t ld_w,
                        int64_t n, int64_t h, int64_t v, const void* targets,
                        int32_t target_dtype, int64_t ignore_index, int32_t tile_width,
                        float temperature, int32_t logits_rounding, float* logp_out,
                        float* lse_out, float* entropy_out, void* logits_out,
                        int32_t logits_dtype, int64_t ld_logits, const void* prepared,
                        size_t prepared_bytes, void* workspace, size_t workspace_bytes,
                        void* hip_stream) {
  return linear_fwd_run(hidden, ld_h, weight, ld_w, n, h, v, targets, target_dtype,
                        ignore_index, tile_width, temperature, logits_rounding, logp_out, lse_out,
                        entropy_out, logits_out, logits_dtype, ld_logits, prepared,
                        prepared_bytes, workspace, workspace_bytes, false, hip_stream);
}

int32_t linear_logp_fwd_noalloc(const void* hidden, int64_t ld_h, const void* weight,
                                int64_t ld_w, int64_t n, int64_t h, int64_t v,
                                const void* targets, int32_t target_dtype, int64_t ignore_index,
                                int32_t tile_width, float temperature, int32_t logits_rounding,
                                float* logp_out, float* lse_out, float* entropy_out,
                                void* logits_out, int32_t logits_dtype, int64_t ld_logits,
                                const void* prepared, size_t prepared_bytes, void* hip_stream) {
  return linear_fwd_run(hidden, ld_h, weight, ld_w, n, h, v, targets, target_dtype,
                        ignore_index, tile_width, temperature, logits_rounding, logp_out, lse_out,
                        entropy_out, logits_out, logits_dtype, ld_logits, prepared,
                        prepared_bytes, nullptr, 0, true, hip_stream);
}

size_t linear_logp_bwd_workspace_bytes(int64_t n, int64_t h, int64_t v, int32_t tile_width,
                                       int32_t flags, int64_t vocab_chunk) {
  if (n < 0 || v < 1 || h < 64 || h % 64 || tile_width != itl::kLinearTile) return 0;
  if (vocab_chunk < 0 || flags < 0 || flags > 31) return 0;
  if (n == 0) return 0;
  return static_cast<size_t>(itl::linear_bwd_layout(n, h, v, flags, vocab_chunk).total);
}

int32_t linear_logp_bwd(const void* hidden, int64_t ld_h, const void* weight, int64_t ld_w,
                        int64_t n, int64_t h, int64_t v, const void* targets,
                        int32_t target_dtype, int64_t ignore_index, int32_t tile_width,
                        float temperature, int32_t logits_rounding, const void* saved_logits,
                        int32_t saved_dtype, int64_t ld_saved, const void* prepared,
                        size_t prepared_bytes, const float* lse, const float* grad_logp,
                        const float* entropy, const float* grad_entropy, int32_t out_dtype,
                        void* dhidden, int64_t ld_dh, void* dweight, int64_t ld_dw,
                        int64_t vocab_chunk, void* workspace, size_t workspace_bytes,
                        void* hip_stream) {
  if (n < 0 || v < 1 || h < 64 || h % 64 || ld_h < h || ld_w < h) return LOGP_ERR_SHAPE;
  if (vocab_chunk < 0 || vocab_chunk > (int64_t{1} << 40)) return LOGP_ERR_SHAPE;
  if (v > (int64_t{1} << 31) || n > (int64_t{1} << 31) ||
      ((n + 255) / 256) * ((v + 255) / 256) > (int64_t{1} << 30) ||
      ((v + 255) / 256) * ((h + 255) / 256) > (int64_t{1} << 30))
    return LOGP_ERR_SHAPE;
  if (tile_width != itl::kLinearTile) return LOGP_ERR_TILE;
  if (out_dtype != LOGP_F32 && out_dtype != LOGP_BF16) return LOGP_ERR_DTYPE;
  if (!valid_index(target_dtype)) return LOGP_ERR_DTYPE;
  if (!valid_temperature(temperature) || !valid_rounding(logits_rounding)) return LOGP_ERR_VALUE;
  if (saved_logits) {
    if (saved_dtype != LOGP_F32 &&
        !(saved_dtype == LOGP_BF16 && logits_rounding == LOGP_ROUND_BF16))
      return LOGP_ERR_DTYPE;
    if (ld_saved < v) return LOGP_ERR_SHAPE;
    if (!aligned16(saved_logits, ld_saved, saved_dtype)) return LOGP_ERR_ALIGN;
  }
  if (prepared) {
    if (prepared_bytes < linear_logp_prepared_bytes(v, h)) return LOGP_ERR_SHAPE;
    if (reinterpret_cast<uintptr_t>(prepared) % 16) return LOGP_ERR_ALIGN;
  }
  if (!dhidden && !dweight) return LOGP_ERR_NULL;
  if ((dhidden && ld_dh < h) || (dweight && ld_dw < h)) return LOGP_ERR_SHAPE;
  if (n == 0 && !dweight) return LOGP_OK;
  if (!weight || (n > 0 && (!hidden || !targets || !lse || !grad_logp))) return LOGP_ERR_NULL;
  if ((entropy == nullptr) != (grad_entropy == nullptr)) return LOGP_ERR_NULL;
  if ((n > 0 && !aligned16(hidden, ld_h, LOGP_BF16)) || !aligned16(weight, ld_w, LOGP_BF16))
    return LOGP_ERR_ALIGN;
  const int32_t flags = (dhidden ? LOGP_BWD_DHIDDEN : 0) | (dweight ? LOGP_BWD_DWEIGHT : 0) |
                        (prepared ? LOGP_BWD_PREPARED : 0) |
                        (saved_logits ? LOGP_BWD_SAVED_LOGITS : 0) |
                        (out_dtype == LOGP_BF16 ? LOGP_BWD_BF16_OUT : 0);
  const size_t need = linear_logp_bwd_workspace_bytes(n, h, v, tile_width, flags, vocab_chunk);
  if (need && (!workspace || workspace_bytes < need ||
               reinterpret_cast<uintptr_t>(workspace) % kAlign))
    return LOGP_ERR_WORKSPACE;
  (void)hipGetLastError();
  itl::launch_linear_bwd(static_cast<const uint16_t*>(hidden), ld_h,
                         static_cast<const uint16_t*>(weight), ld_w, n, h, v,
                         targets_of(targets, target_dtype), ignore_index, saved_logits,
                         saved_dtype == LOGP_BF16 ? 1 : 0, ld_saved,
                         static_cast<const uint16_t*>(prepared), lse, grad_logp,
                         inv_temperature(temperature), logits_rounding == LOGP_ROUND_BF16 ? 1 : 0,
                         entropy, grad_entropy,
                         out_dtype == LOGP_BF16, dhidden, ld_dh, dweight, ld_dw, vocab_chunk,
                         static_cast<char*>(workspace), static_cast<hipStream_t>(hip_stream));
  return hip_status();
}

size_t linear_logp_prepared_bytes(int64_t v, int64_t h) {
  if (v < 1 || h < 64 || h % 64 || v > (int64_t{1} << 31)) return 0;
  return static_cast<size_t>(itl::prepared_bytes(v, h));
}

int32_t linear_logp_prepare_weight(const void* weight, int64_t ld_w, int64_t v, int64_t h,
                                   void* prepared, size_t prepared_bytes, void* hip_stream) {
  if (v < 1 || h < 64 || h % 64 || ld_w < h || v > (int64_t{1} << 31)) return LOGP_ERR_SHAPE;
  if (prepared_bytes < linear_logp_prepared_bytes(v, h)) return LOGP_ERR_SHAPE;
  if (!weight || !prepared) return LOGP_ERR_NULL;
  if (!aligned16(weight, ld_w, LOGP_BF16) || reinterpret_cast<uintptr_t>(prepared) % 16)
    return LOGP_ERR_ALIGN;
  (void)hipGetLastError();
  itl::launch_prepare_weight(static_cast<const uint16_t*>(weight), ld_w, v, h,
                             static_cast<uint16_t*>(prepared),
                             static_cast<hipStream_t>(hip_stream));
  return hip_status();
}

const char* logp_status_str(int32_t status) {
  switch (status) {
    case LOGP_OK: return "ok";
    case LOGP_ERR_NULL: return "a required pointer is NULL";
    case LOGP_ERR_SHAPE: return "unsupported or inconsistent shape";
    case LOGP_ERR_DTYPE: return "unknown dtype";
    case LOGP_ERR_TILE: return "unsupported tile width";
    case LOGP_ERR_ALIGN: return "operand rows are not 16-byte aligned";
    case LOGP_ERR_SHARDS: return "num_shards must be >= 1 and divide v";
    case LOGP_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case LOGP_ERR_TARGET: return "an active target lies outside [0, v)";
    case LOGP_ERR_HIP: return "HIP launch or copy failed";
    case LOGP_ERR_VALUE:
      return "invalid scalar argument (temperature, logits rounding, or a stream of another device)";
    case LOGP_ERR_SCRATCH:
      return "the call needs more scratch than the no-allocation entry point's static buffer holds";
    default: return "unknown status";
  }
}

const char* logp_contract_id(void) {
  return "itl.logp.v1[tile=lane-asc-fold+xor1..32;tilestat=two-pass;merge=asc-fma;"
         "exp=v_exp_f32((a-b)*log2e);log=v_log_f32*ln2;bwd=rne(g*(onehot-p))]"
         "+itl.linear_logp.v1[mfma=f32_16x16x32_bf16;k=asc32-nosplit;tile=256;"
         "tilestat=4x64(lane-asc-fold4+xor1..8)+(q0+q1)+(q2+q3);"
         "temp=z*fl32(1/T);"
         "bwd=dz:rne_bf16((g*(onehot-p)+fma(-gH,p*(x-lse+H)))*fl32(1/T)),"
         "dh:dz*W(k=vocab-asc32),dW:dz^T*h(k=token-asc32)]"
         "+entropy[w=sum e*(x-m) same tree;merge b=fma(fma(s,m-M,w),e,b);H=log(acc)-b/acc]"
         "+itl.linear_logp_bf16z.v1[as itl.linear_logp.v1 with z=rne_bf16(acc) first]"
         "/gfx950";
}

}  // extern "C"
