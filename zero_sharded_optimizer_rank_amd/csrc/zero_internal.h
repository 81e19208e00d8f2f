// Internal interface between the host-side C ABI (zero_host.cpp) and the
// device kernels with their launchers (zero_kernels.hip).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "zero_shard.h"

namespace zk {

constexpr int kThreads = 256;        // threads per workgroup (four 64-wide waves)
constexpr int kFinBlocks = 256;      // most workgroups of the partial-sum kernel
constexpr size_t kTicketBytes = 256; // ticket word (armed by the reduce kernel), padded
constexpr size_t kPartialBytes = 16;
constexpr int64_t kRestoreBlocks = 2048;  // most workgroups of the slot restore

// fp64 inputs of the norm / clip / skip decision.
struct FinalizeArgs {
  double inv64;     // 1 / (N * loss_scale)
  double max_norm;  // <= 0: no clipping
  double other_sq;  // fp64 stand-in for the other ranks' squared norm
  uint64_t other_lo, other_hi;
  int32_t other_overflow;
  int32_t pad;
};

// fp32 Adam coefficients, each rounded once from fp64 on the host.
struct AdamScalars {
  float b1, omb1, b2, omb2, eps, step_size, sqrt_bc2, decay;
};

// Workgroups of the reduce and Adam kernels for a shard, and the workspace
// the reduce needs: ticket, kFinBlocks second-level partials, one partial per
// reduce workgroup.
int64_t k1_blocks(int64_t shard);
int64_t k1_blocks_deferred(int64_t shard);  // the reduce's deferred form (fewer, deeper workgroups)
int64_t k2_blocks(int64_t shard);
size_t workspace_bytes_for_blocks(int64_t reduce_blocks);
size_t workspace_bytes(int64_t shard);

// Launchers: arguments already validated.  Return hipSuccess or the error.
int launch_reduce_check(const uint16_t* const* contrib, int n, int64_t shard, float inv32,
                        float* grad, void* workspace, const FinalizeArgs& fa,
                        zero_step_result_t* res, hipStream_t stream);
int launch_partials_finalize(void* workspace, int64_t n_partials, const FinalizeArgs& fa,
                             zero_step_result_t* res, hipStream_t stream);
int launch_finalize(const FinalizeArgs& fa, zero_step_result_t* res, hipStream_t stream);
int launch_finalize_empty(const FinalizeArgs& fa, zero_step_result_t* res, hipStream_t stream);
int launch_adam(const float* grad, float* master, float* m, float* v, uint16_t* slot,
                int64_t shard, const AdamScalars& sc, const zero_step_result_t* res,
                hipStream_t stream);
void* workspace_partials(void* workspace);

// Single pass for steps without clipping: reduce, exact squares and the
// update from the `in` state into the distinct `out` state and slot, then the
// partial sums and finalize.  No gradient is written.
int64_t k12_blocks(int64_t shard);
int launch_reduce_adam_1pass(const uint16_t* const* contrib, int n, int64_t shard, float inv32,
                             const float* master_in, const float* m_in, const float* v_in,
                             float* master_out, float* m_out, float* v_out, uint16_t* slot_out,
                             const AdamScalars& sc, void* workspace, const FinalizeArgs& fa,
                             zero_step_result_t* res, hipStream_t stream);

// Recast the slot from the master when res->skip (16-bit fp16 or bf16 slot).
int launch_slot_restore(const float* master, uint16_t* slot, int64_t shard, bool bf16,
                        const zero_step_result_t* res, hipStream_t stream);

// bf16 path (the norm is a fixed pairwise fp64 tree; see zero_device.h).
int64_t k1_blocks_bf16(int64_t shard);
int launch_reduce_check_bf16(const uint16_t* const* contrib, int n, int64_t shard, float inv32,
                             float* grad, void* workspace, const FinalizeArgs& fa,
                             zero_step_result_t* res, hipStream_t stream);
int launch_finalize_bf16(const FinalizeArgs& fa, zero_step_result_t* res, hipStream_t stream);
int launch_reduce_adam_1pass_bf16(const uint16_t* const* contrib, int n, int64_t shard,
                                  float inv32, const float* master_in, const float* m_in,
                                  const float* v_in, float* master_out, float* m_out,
                                  float* v_out, uint16_t* slot_out, const AdamScalars& sc,
                                  void* workspace, const FinalizeArgs& fa,
                                  zero_step_result_t* res, hipStream_t stream);
int launch_adam_bf16(const float* grad, float* master, float* m, float* v, uint16_t* slot,
                     int64_t shard, const AdamScalars& sc, const zero_step_result_t* res,
                     hipStream_t stream);

// Multi-unit forms (zero_units.hip): the unit table lives in device memory.
// launch_store_table writes a host table there through kernel arguments.
int launch_store_table(const zero_unit_buffers_t* units_host, int32_t n_units,
                       zero_unit_buffers_t* units_dev, hipStream_t stream);
// `blocks` is the one-chunk workgroup count zero_units_prepare recorded;
// *n_partials receives the partials written (fewer when the deferred form
// runs, above N = 8).
int launch_units_reduce(const zero_unit_buffers_t* units_dev, int32_t n_units, int64_t blocks,
                        int n, float inv32, void* workspace, int64_t* n_partials,
                        hipStream_t stream);
int launch_units_adam(const zero_unit_buffers_t* units_dev, int32_t n_units, int64_t blocks,
                      const AdamScalars& sc, const zero_step_result_t* res, hipStream_t stream);
int launch_units_slot_restore(const zero_unit_buffers_t* units_dev, int32_t n_units,
                              int64_t max_shard, const zero_step_result_t* res,
                              hipStream_t stream);
int launch_units_reduce_adam_1pass(const zero_unit_buffers_t* units_dev,
                                   const zero_unit_buffers_t* outs_dev, int32_t n_units,
                                   int64_t blocks, int n, float inv32, const AdamScalars& sc,
                                   void* workspace, hipStream_t stream);

}  // namespace zk
