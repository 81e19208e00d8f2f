// The whole shard step for callers that cannot allocate device memory (code
// under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc): zero_reduce_adam_step with the reduce's workspace (the
// finalize ticket, the second-level partials and one partial per reduce
// workgroup) taken from a library-held device array instead of a caller
// buffer.  The kernels are the ones zero_reduce_adam_step launches.
//
// The array is a file-scope __device__ variable: every GPU the library runs
// on holds its own copy, at its own address, until the process ends.  In
// host code its name only stands in for the symbol; the device address comes
// from hipGetSymbolAddress, resolved once per device (with that device
// current) on the first call there and kept in g_scratch[].  Every call on a
// device shares that device's array, so calls that overlap on one GPU (two
// streams, or two threads) race on it.  Nothing in it needs clearing: the
// reduce kernel arms the finalize's ticket itself, and the partials are
// written before they are read in every call.
#include <atomic>
#include <mutex>

#include <hip/hip_runtime.h>

#include "host_internal.h"
#include "zero_internal.h"
#include "zero_shard.h"

namespace zk {
namespace {

// Largest reduce workspace the array holds: ticket, the second-level
// partials and one 16-byte partial per 512-element reduce workgroup of the
// largest accepted shard.
constexpr size_t kScratchBytes =
    kTicketBytes + (size_t)kFinBlocks * kPartialBytes +
    (size_t)(ZERO_NOALLOC_MAX_SHARD / 512) * kPartialBytes;
static_assert(kScratchBytes % 256 == 0, "whole 256-byte lines");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// This device's address of `scratch`, resolved on first use.
int scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return host::hip_status((int)e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return host::fail(ZERO_EINVAL, "device %d outside 0..%d", dev, kMaxDevices - 1);
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress((void**)&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return host::hip_status((int)e, "hipGetSymbolAddress(scratch)");
      if (!p) return host::fail(ZERO_EHIP, "hipGetSymbolAddress(scratch) gave NULL");
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return ZERO_OK;
}

}  // namespace
}  // namespace zk

using namespace zk::host;

extern "C" int zero_reduce_adam_step_noalloc(const zero_plan_t* plan, int32_t rank,
                                             const uint16_t* const* contrib, float* master,
                                             float* m, float* v, uint16_t* param16_slot,
                                             float* grad_out, const zero_step_args_t* args,
                                             zero_step_result_t* dev_result,
                                             hipStream_t stream) {
  g_err[0] = 0;
  int rc = check_plan_rank(plan, rank);
  if (!rc) rc = check_adam_args(args);
  if (rc) return rc;
  if (plan->shard > ZERO_NOALLOC_MAX_SHARD)
    return fail(ZERO_ENOSPC,
                "shard %lld elements exceeds the library scratch of this call (at most %lld); "
                "use zero_reduce_adam_step with a workspace",
                (long long)plan->shard, (long long)ZERO_NOALLOC_MAX_SHARD);
  rc = check_rows(plan, contrib);
  if (!rc) rc = check_adam_ptrs(plan, grad_out, master, m, v, param16_slot, dev_result);
  if (rc) return rc;
  const size_t ws_bytes = zk::workspace_bytes_for_blocks(zk::k1_blocks(plan->shard));
  if (ws_bytes > zk::kScratchBytes)
    return fail(ZERO_ENOSPC, "workspace %zu bytes > scratch %zu", ws_bytes, zk::kScratchBytes);
  void* ws = nullptr;
  rc = zk::scratch_ptr(&ws);
  if (rc) return rc;
  const zk::FinalizeArgs fa = finalize_args(plan, args);
  rc = hip_status(zk::launch_reduce_check(contrib, (int)plan->world_size, plan->shard,
                                          (float)fa.inv64, grad_out, ws, fa, dev_result, stream),
                  "reduce_check launch");
  // another rank's overflow makes the finalize skip the step: no update launch
  if (rc || plan->shard == 0 || args->other_overflow) return rc;
  return hip_status(zk::launch_adam(grad_out, master, m, v, param16_slot, plan->shard,
                                    adam_scalars(args), dev_result, stream),
                    "adam launch");
}
