// Calibration kernel for measurement only (not part of the shard step): a
// plain streaming copy of a known number of bytes, one 16-byte unit per
// thread in a one-shot grid (the fastest copy shape measured on MI355X).
// Timing it gives the achievable copy bandwidth; profiling it gives the
// factor between the hardware byte counters and bytes actually moved.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ void calib_copy(const u32x4* __restrict__ src, u32x4* __restrict__ dst, int64_t n16) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n16) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}
}  // namespace

// Copy `bytes` (a multiple of 16; both pointers 16-byte aligned) on `stream`
// with `threads` (64..1024, a multiple of 64) threads per workgroup.
// Returns 0 or a hipError_t.
extern "C" int zero_calib_copy(const void* src, void* dst, int64_t bytes, int threads,
                               hipStream_t stream) {
  if (!src || !dst || bytes < 0 || (bytes & 15) || threads < 64 || threads > 1024 ||
      (threads & 63) || (((uintptr_t)src | (uintptr_t)dst) & 15))
    return (int)hipErrorInvalidValue;
  const int64_t n16 = bytes / 16;
  const int64_t blocks = (n16 + threads - 1) / threads;
  if (blocks < 1 || blocks > 0x7FFFFFFF) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(calib_copy, dim3((uint32_t)blocks), dim3(threads), 0, stream,
                     (const u32x4*)src, (u32x4*)dst, n16);
  return (int)hipGetLastError();
}
