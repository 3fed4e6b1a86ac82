// Bandwidth probes for bench.py (not part of the logp library's C ABI): the
// HBM read and copy rates that this GPU reaches with the access pattern of
// the streaming kernels, measured in the same run as the kernels themselves,
// as a measured denominator next to the 8 TB/s vendor figure.
//
// Pattern: one 16-byte chunk per thread, the launch walking the buffer in
// address order, non-temporal loads (and stores for the copy) -- the
// pattern of logp_bwd_kernel and of the forward's tile loads.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

// Folds every chunk into a per-thread value and stores it only when it
// equals a value no input here produces, so the loads cannot be dropped.
__global__ __launch_bounds__(kThreads) void read_probe(const u32x4_t* __restrict__ src,
                                                       int64_t chunks, unsigned key,
                                                       unsigned* __restrict__ sink) {
  const int64_t c = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (c >= chunks) return;
  const u32x4_t w = __builtin_nontemporal_load(src + c);
  const unsigned f = (w.x ^ w.y) + (w.z ^ w.w);
  if (f == key) sink[0] = f;
}

__global__ __launch_bounds__(kThreads) void copy_probe(const u32x4_t* __restrict__ src,
                                                       u32x4_t* __restrict__ dst,
                                                       int64_t chunks) {
  const int64_t c = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (c >= chunks) return;
  __builtin_nontemporal_store(__builtin_nontemporal_load(src + c), dst + c);
}

unsigned blocks_for(int64_t chunks) {
  return static_cast<unsigned>((chunks + kThreads - 1) / kThreads);
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16, < 2^40) at `src` (16-byte aligned) on
// `stream`; `sink` is one device unsigned that is written only in the
// unlikely case that a folded chunk equals 0x9e3779b9.  Returns 0, or 1 for
// bad arguments, 2 for a launch error.
int itl_probe_read(const void* src, size_t bytes, unsigned* sink, void* stream) {
  if (!src || !sink || bytes % 16 || reinterpret_cast<uintptr_t>(src) % 16 ||
      bytes >= (size_t{1} << 40))
    return 1;
  const int64_t chunks = static_cast<int64_t>(bytes / 16);
  if (chunks == 0) return 0;
  (void)hipGetLastError();
  hipLaunchKernelGGL(read_probe, dim3(blocks_for(chunks)), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4_t*>(src), chunks,
                     0x9e3779b9u, sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// Copies `bytes` (a multiple of 16, < 2^40) from `src` to `dst` (both
// 16-byte aligned, not overlapping) on `stream`.  Returns 0, 1 or 2 as above.
int itl_probe_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (!src || !dst || bytes % 16 || reinterpret_cast<uintptr_t>(src) % 16 ||
      reinterpret_cast<uintptr_t>(dst) % 16 || bytes >= (size_t{1} << 40))
    return 1;
  const int64_t chunks = static_cast<int64_t>(bytes / 16);
  if (chunks == 0) return 0;
  (void)hipGetLastError();
  hipLaunchKernelGGL(copy_probe, dim3(blocks_for(chunks)), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4_t*>(src),
                     static_cast<u32x4_t*>(dst), chunks);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
