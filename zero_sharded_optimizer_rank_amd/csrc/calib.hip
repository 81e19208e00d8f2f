// Calibration kernel for measurement only (not part of the shard step): a
// plain streaming copy of a known number of bytes.  Timing it gives the
// achievable HBM bandwidth on the box; profiling it gives the factor between
// the hardware byte counters and bytes actually moved.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void calib_copy(const u32x4* __restrict__ src,
                                                  u32x4* __restrict__ dst, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride)
    __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}
}  // namespace

// Copy `bytes` (a multiple of 16; both pointers 16-byte aligned) on `stream`
// with `blocks` workgroups of 256 threads.  Returns 0 or a hipError_t.
extern "C" int zero_calib_copy(const void* src, void* dst, int64_t bytes, int blocks,
                               hipStream_t stream) {
  if (!src || !dst || bytes < 0 || (bytes & 15) || blocks < 1 || (((uintptr_t)src | (uintptr_t)dst) & 15))
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(calib_copy, dim3(blocks), dim3(256), 0, stream, (const u32x4*)src, (u32x4*)dst,
                     bytes / 16);
  return (int)hipGetLastError();
}
