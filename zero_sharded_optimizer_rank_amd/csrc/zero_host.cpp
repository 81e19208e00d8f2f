// Host side of the C ABI: shard planner, model-state bytes, loss scaler,
// argument checks, fp64 -> fp32 scalar preparation, and the kernel launches.
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include <hip/hip_runtime_api.h>

#include "host_internal.h"
#include "zero_internal.h"
#include "zero_shard.h"

namespace zk {
namespace host {

thread_local char g_err[512];

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Checks shared by the device entry points.
int check_plan_rank(const zero_plan_t* plan, int32_t rank) {
  if (!plan) return fail(ZERO_EINVAL, "plan is NULL");
  if (plan->world_size < 1 || plan->world_size > ZERO_MAX_RANKS)
    return fail(ZERO_EINVAL, "world_size %lld outside 1..%d", (long long)plan->world_size,
                ZERO_MAX_RANKS);
  if (rank < 0 || rank >= plan->world_size)
    return fail(ZERO_EINVAL, "rank %d outside 0..%lld", rank, (long long)plan->world_size - 1);
  if (plan->shard < 0 || plan->shard > ZERO_MAX_SHARD)
    return fail(ZERO_EINVAL, "shard %lld outside 0..%lld", (long long)plan->shard,
                (long long)ZERO_MAX_SHARD);
  if (plan->psi_padded != plan->shard * plan->world_size || plan->psi < 0 ||
      plan->psi > plan->psi_padded)
    return fail(ZERO_EINVAL, "inconsistent plan");
  return ZERO_OK;
}

int check_norm_args(const zero_step_args_t* a) {
  if (!a) return fail(ZERO_EINVAL, "args is NULL");
  if (!(a->loss_scale > 0.0) || !isfinite(a->loss_scale))
    return fail(ZERO_EINVAL, "loss_scale must be finite and > 0");
  if (!(a->other_sq >= 0.0) || !isfinite(a->other_sq))
    return fail(ZERO_EINVAL, "other_sq must be finite and >= 0");
  if (isnan(a->max_grad_norm)) return fail(ZERO_EINVAL, "max_grad_norm is NaN");
  return ZERO_OK;
}

int check_adam_args(const zero_step_args_t* a) {
  int rc = check_norm_args(a);
  if (rc) return rc;
  if (!(a->lr >= 0.0) || !isfinite(a->lr)) return fail(ZERO_EINVAL, "lr must be finite and >= 0");
  if (!(a->eps >= 0.0) || !isfinite(a->eps)) return fail(ZERO_EINVAL, "eps must be finite and >= 0");
  if (!(a->beta1 >= 0.0 && a->beta1 < 1.0) || !(a->beta2 >= 0.0 && a->beta2 < 1.0))
    return fail(ZERO_EINVAL, "betas must lie in [0, 1)");
  if (!isfinite(a->weight_decay)) return fail(ZERO_EINVAL, "weight_decay is not finite");
  if (a->step < 1) return fail(ZERO_EINVAL, "step must be >= 1");
  return ZERO_OK;
}

zk::FinalizeArgs finalize_args(const zero_plan_t* plan, const zero_step_args_t* a) {
  zk::FinalizeArgs fa;
  fa.inv64 = 1.0 / ((double)plan->world_size * a->loss_scale);
  fa.max_norm = a->max_grad_norm;
  fa.other_sq = a->other_sq;
  fa.other_lo = a->other_q_lo;
  fa.other_hi = a->other_q_hi;
  fa.other_overflow = a->other_overflow ? 1 : 0;
  fa.pad = 0;
  return fa;
}

// Coefficients in fp64 from the decimal hyperparameters, each rounded to fp32
// once; beta^t as t left-to-right fp64 products.  Once both powers are at or
// below 2^-54, 1 - p rounds to exactly 1 (a tie at 2^-54 goes to the even 1),
// and further products only shrink them, so the loop stops there.
zk::AdamScalars adam_scalars(const zero_step_args_t* a) {
  double p1 = a->beta1, p2 = a->beta2;
  for (int64_t i = 1; i < a->step; ++i) {
    if (p1 <= 0x1p-54 && p2 <= 0x1p-54) break;
    p1 *= a->beta1;
    p2 *= a->beta2;
  }
  zk::AdamScalars s;
  s.b1 = (float)a->beta1;
  s.omb1 = (float)(1.0 - a->beta1);
  s.b2 = (float)a->beta2;
  s.omb2 = (float)(1.0 - a->beta2);
  s.eps = (float)a->eps;
  s.step_size = (float)(a->lr / (1.0 - p1));
  s.sqrt_bc2 = (float)sqrt(1.0 - p2);
  s.decay = (float)(1.0 - a->lr * a->weight_decay);
  return s;
}

// The N contribution rows of a reduce.
int check_rows(const zero_plan_t* plan, const uint16_t* const* contrib) {
  if (plan->shard == 0) return ZERO_OK;
  if (!contrib) return fail(ZERO_EINVAL, "contrib is NULL");
  for (int64_t r = 0; r < plan->world_size; ++r) {
    if (!contrib[r]) return fail(ZERO_EINVAL, "contrib[%lld] is NULL", (long long)r);
    if (!aligned(contrib[r], 16))
      return fail(ZERO_EALIGN, "contrib[%lld] not 16-byte aligned", (long long)r);
  }
  return ZERO_OK;
}

// Contribution rows, workspace and result of a reduce.
int check_reduce_inputs(const zero_plan_t* plan, const uint16_t* const* contrib, void* workspace,
                        size_t ws_bytes, zero_step_result_t* dev_result) {
  if (!dev_result) return fail(ZERO_EINVAL, "dev_result is NULL");
  if (!aligned(dev_result, 8)) return fail(ZERO_EALIGN, "dev_result not 8-byte aligned");
  if (!workspace) return fail(ZERO_EINVAL, "workspace is NULL");
  if (!aligned(workspace, 16)) return fail(ZERO_EALIGN, "workspace not 16-byte aligned");
  const size_t need = zk::workspace_bytes(plan->shard);
  if (ws_bytes < need) return fail(ZERO_ENOSPC, "workspace %zu bytes < %zu", ws_bytes, need);
  return check_rows(plan, contrib);
}

int check_reduce_ptrs(const zero_plan_t* plan, const uint16_t* const* contrib, float* grad_out,
                      void* workspace, size_t ws_bytes, zero_step_result_t* dev_result) {
  const int rc = check_reduce_inputs(plan, contrib, workspace, ws_bytes, dev_result);
  if (rc || plan->shard == 0) return rc;
  if (!grad_out) return fail(ZERO_EINVAL, "grad_out is NULL");
  if (!aligned(grad_out, 16)) return fail(ZERO_EALIGN, "grad_out not 16-byte aligned");
  return ZERO_OK;
}

int check_adam_ptrs(const zero_plan_t* plan, const float* grad, float* master, float* m, float* v,
                    uint16_t* slot, const zero_step_result_t* dev_result) {
  if (!dev_result) return fail(ZERO_EINVAL, "dev_result is NULL");
  if (!aligned(dev_result, 8)) return fail(ZERO_EALIGN, "dev_result not 8-byte aligned");
  if (plan->shard == 0) return ZERO_OK;
  if (!grad || !master || !m || !v || !slot) return fail(ZERO_EINVAL, "NULL state pointer");
  if (!aligned(grad, 16) || !aligned(master, 16) || !aligned(m, 16) || !aligned(v, 16))
    return fail(ZERO_EALIGN, "grad, master, m and v must be 16-byte aligned");
  if (!aligned(slot, 2)) return fail(ZERO_EALIGN, "param16_slot not 2-byte aligned");
  return ZERO_OK;
}

int hip_status(int e, const char* what) {
  if (e == hipSuccess) return ZERO_OK;
  return fail(ZERO_EHIP, "%s: %s", what, hipGetErrorString((hipError_t)e));
}

}  // namespace host
}  // namespace zk

using namespace zk::host;

extern "C" {

const char* zero_last_error(void) { return g_err; }

int zero_plan(const int64_t* numels, int32_t n_tensors, int32_t world_size, int32_t align_elems,
              zero_plan_t* plan_out, int64_t* offsets_out) {
  g_err[0] = 0;
  if (n_tensors < 0 || (n_tensors > 0 && !numels) || !plan_out)
    return fail(ZERO_EINVAL, "bad tensor list or NULL plan_out");
  if (world_size < 1) return fail(ZERO_EINVAL, "world_size must be >= 1");
  if (align_elems < 1) return fail(ZERO_EINVAL, "align_elems must be >= 1");
  int64_t acc = 0;
  for (int32_t i = 0; i < n_tensors; ++i) {
    if (numels[i] < 0) return fail(ZERO_EINVAL, "numel %d is negative", i);
    if (offsets_out) offsets_out[i] = acc;
    if (numels[i] > INT64_MAX / 2 - acc) return fail(ZERO_EINVAL, "psi overflows int64");
    acc += numels[i];
  }
  const int64_t per_rank = acc / world_size + (acc % world_size ? 1 : 0);
  const int64_t shard = (per_rank / align_elems + (per_rank % align_elems ? 1 : 0)) * align_elems;
  if (shard > INT64_MAX / world_size) return fail(ZERO_EINVAL, "padded size overflows int64");
  plan_out->psi = acc;
  plan_out->world_size = world_size;
  plan_out->align = align_elems;
  plan_out->shard = shard;
  plan_out->psi_padded = shard * world_size;
  return ZERO_OK;
}

int64_t zero_plan_real(const zero_plan_t* plan, int32_t rank) {
  if (!plan || rank < 0 || rank >= plan->world_size) return -1;
  int64_t r = plan->psi - (int64_t)rank * plan->shard;
  if (r < 0) r = 0;
  if (r > plan->shard) r = plan->shard;
  return r;
}

int zero_plan_segments(const zero_plan_t* plan, const int64_t* numels, const int64_t* offsets,
                       int32_t n_tensors, int32_t rank, zero_segment_t* out, int32_t cap,
                       int32_t* n_out) {
  g_err[0] = 0;
  if (!plan || (n_tensors > 0 && (!numels || !offsets)) || n_tensors < 0 || !n_out || cap < 0 ||
      (cap > 0 && !out))
    return fail(ZERO_EINVAL, "NULL or negative argument");
  if (rank < 0 || rank >= plan->world_size) return fail(ZERO_EINVAL, "bad rank %d", rank);
  const int64_t a = (int64_t)rank * plan->shard, b = a + plan->shard;
  int32_t k = 0;
  for (int32_t t = 0; t < n_tensors; ++t) {
    const int64_t lo = offsets[t] > a ? offsets[t] : a;
    const int64_t end = offsets[t] + numels[t];
    const int64_t hi = end < b ? end : b;
    if (lo < hi) {
      if (k < cap) {
        out[k].tensor = t;
        out[k].reserved = 0;
        out[k].tensor_begin = lo - offsets[t];
        out[k].shard_begin = lo - a;
        out[k].length = hi - lo;
      }
      ++k;
    }
  }
  *n_out = k;
  if (k > cap) return fail(ZERO_ENOSPC, "%d segments, capacity %d", k, cap);
  return ZERO_OK;
}

double zero_state_bytes(int32_t stage, double psi, double n, double k) {
  if (stage < 0 || stage > 3 || !(psi >= 0.0) || !(n >= 1.0) || !(k >= 0.0)) return -1.0;
  switch (stage) {
    case 0: return (2.0 + 2.0 + k) * psi;
    case 1: return 4.0 * psi + k * psi / n;
    case 2: return 2.0 * psi + (2.0 + k) * psi / n;
    default: return (4.0 + k) * psi / n;
  }
}

size_t zero_workspace_bytes(const zero_plan_t* plan) {
  if (!plan || plan->shard < 0 || plan->shard > ZERO_MAX_SHARD) return 0;
  return zk::workspace_bytes(plan->shard);
}

int zero_reduce_check(const zero_plan_t* plan, int32_t rank, const uint16_t* const* contrib,
                      const zero_step_args_t* args, float* grad_out, void* workspace,
                      size_t ws_bytes, zero_step_result_t* dev_result, hipStream_t stream) {
  g_err[0] = 0;
  int rc = check_plan_rank(plan, rank);
  if (!rc) rc = check_norm_args(args);
  if (!rc) rc = check_reduce_ptrs(plan, contrib, grad_out, workspace, ws_bytes, dev_result);
  if (rc) return rc;
  const zk::FinalizeArgs fa = finalize_args(plan, args);
  return hip_status(zk::launch_reduce_check(contrib, (int)plan->world_size, plan->shard,
                                            (float)fa.inv64, grad_out, workspace, fa, dev_result,
                                            stream),
                    "reduce_check launch");
}

int zero_finalize(const zero_plan_t* plan, const zero_step_args_t* args,
                  zero_step_result_t* dev_result, hipStream_t stream) {
  g_err[0] = 0;
  int rc = check_plan_rank(plan, 0);
  if (!rc) rc = check_norm_args(args);
  if (rc) return rc;
  if (!dev_result) return fail(ZERO_EINVAL, "dev_result is NULL");
  if (!aligned(dev_result, 8)) return fail(ZERO_EALIGN, "dev_result not 8-byte aligned");
  return hip_status(zk::launch_finalize(finalize_args(plan, args), dev_result, stream),
                    "finalize launch");
}

int zero_adam_apply(const zero_plan_t* plan, int32_t rank, const float* grad, float* master,
                    float* m, float* v, uint16_t* param16_slot, const zero_step_args_t* args,
                    const zero_step_result_t* dev_result, hipStream_t stream) {
  g_err[0] = 0;
  int rc = check_plan_rank(plan, rank);
  if (!rc) rc = check_adam_args(args);
  if (!rc) rc = check_adam_ptrs(plan, grad, master, m, v, param16_slot, dev_result);
  if (rc) return rc;
  if (plan->shard == 0) return ZERO_OK;
  return hip_status(zk::launch_adam(grad, master, m, v, param16_slot, plan->shard,
                                    adam_scalars(args), dev_result, stream),
                    "adam launch");
}

int zero_reduce_adam_step(const zero_plan_t* plan, int32_t rank, const uint16_t* const* contrib,
                          float* master, float* m, float* v, uint16_t* param16_slot,
                          float* grad_out, void* workspace, size_t ws_bytes,
                          const zero_step_args_t* args, zero_step_result_t* dev_result,
                          hipStream_t stream) {
  g_err[0] = 0;
  int rc = check_plan_rank(plan, rank);
  if (!rc) rc = check_adam_args(args);
  if (!rc) rc = check_reduce_ptrs(plan, contrib, grad_out, workspace, ws_bytes, dev_result);
  if (!rc) rc = check_adam_ptrs(plan, grad_out, master, m, v, param16_slot, dev_result);
  if (rc) return rc;
  rc = zero_reduce_check(plan, rank, contrib, args, grad_out, workspace, ws_bytes, dev_result,
                         stream);
  // another rank's overflow makes the finalize skip the step: the update
  // kernel would only start and exit, so it is not launched
  if (rc || args->other_overflow) return rc;
  return zero_adam_apply(plan, rank, grad_out, master, m, v, param16_slot, args, dev_result,
                         stream);
}

// [a, a + na) and [b, b + nb) share a byte.
static bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

// Checks of the single-pass calls: no clipping, reduce inputs, state
// pointers, and no out buffer overlapping an in buffer or another out buffer.
static int check_1pass(const zero_plan_t* plan, int32_t rank, const uint16_t* const* contrib,
                       const float* master_in, const float* m_in, const float* v_in,
                       float* master_out, float* m_out, float* v_out,
                       uint16_t* param16_slot_out, void* workspace, size_t ws_bytes,
                       const zero_step_args_t* args, zero_step_result_t* dev_result) {
  int rc = check_plan_rank(plan, rank);
  if (!rc) rc = check_adam_args(args);
  if (rc) return rc;
  if (args->max_grad_norm > 0.0)
    return fail(ZERO_EINVAL,
                "max_grad_norm > 0: clipping needs the whole norm before any update "
                "(use the two-pass step)");
  rc = check_reduce_inputs(plan, contrib, workspace, ws_bytes, dev_result);
  if (rc) return rc;
  const int64_t S = plan->shard;
  if (S == 0) return ZERO_OK;
  if (!master_in || !m_in || !v_in || !master_out || !m_out || !v_out || !param16_slot_out)
    return fail(ZERO_EINVAL, "NULL state pointer");
  if (!aligned(master_in, 16) || !aligned(m_in, 16) || !aligned(v_in, 16) ||
      !aligned(master_out, 16) || !aligned(m_out, 16) || !aligned(v_out, 16))
    return fail(ZERO_EALIGN, "master, m and v (in and out) must be 16-byte aligned");
  if (!aligned(param16_slot_out, 2)) return fail(ZERO_EALIGN, "slot_out not 2-byte aligned");
  const size_t b4 = 4 * (size_t)S, b2 = 2 * (size_t)S;
  const void* ins[3] = {master_in, m_in, v_in};
  const void* outs[4] = {master_out, m_out, v_out, param16_slot_out};
  const size_t out_bytes[4] = {b4, b4, b4, b2};
  for (int o = 0; o < 4; ++o) {
    for (int i = 0; i < 3; ++i)
      if (overlap(outs[o], out_bytes[o], ins[i], b4))
        return fail(ZERO_EINVAL, "an output state buffer overlaps an input state buffer");
    for (int q = 0; q < o; ++q)
      if (overlap(outs[o], out_bytes[o], outs[q], out_bytes[q]))
        return fail(ZERO_EINVAL, "output state buffers overlap");
  }
  return ZERO_OK;
}

int zero_reduce_adam_step_1pass(const zero_plan_t* plan, int32_t rank,
                                const uint16_t* const* contrib, const float* master_in,
                                const float* m_in, const float* v_in, float* master_out,
                                float* m_out, float* v_out, uint16_t* param16_slot_out,
                                void* workspace, size_t ws_bytes, const zero_step_args_t* args,
                                zero_step_result_t* dev_result, hipStream_t stream) {
  g_err[0] = 0;
  const int rc = check_1pass(plan, rank, contrib, master_in, m_in, v_in, master_out, m_out,
                             v_out, param16_slot_out, workspace, ws_bytes, args, dev_result);
  if (rc) return rc;
  const zk::FinalizeArgs fa = finalize_args(plan, args);
  return hip_status(zk::launch_reduce_adam_1pass(contrib, (int)plan->world_size, plan->shard,
                                                 (float)fa.inv64, master_in, m_in, v_in,
                                                 master_out, m_out, v_out, param16_slot_out,
                                                 adam_scalars(args), workspace, fa, dev_result,
                                                 stream),
                    "reduce_adam_1pass launch");
}

int zero_reduce_adam_step_1pass_bf16(const zero_plan_t* plan, int32_t rank,
                                     const uint16_t* const* contrib, const float* master_in,
                                     const float* m_in, const float* v_in, float* master_out,
                                     float* m_out, float* v_out, uint16_t* param_bf16_slot_out,
                                     void* workspace, size_t ws_bytes,
                                     const zero_step_args_t* args,
                                     zero_step_result_t* dev_result, hipStream_t stream) {
  g_err[0] = 0;
  int rc = check_1pass(plan, rank, contrib, master_in, m_in, v_in, master_out, m_out, v_out,
                       param_bf16_slot_out, workspace, ws_bytes, args, dev_result);
  if (!rc && (args->other_q_lo || args->other_q_hi))
    rc = fail(ZERO_EINVAL, "the bf16 path takes the other ranks' share as other_sq only");
  if (rc) return rc;
  const zk::FinalizeArgs fa = finalize_args(plan, args);
  return hip_status(zk::launch_reduce_adam_1pass_bf16(
                        contrib, (int)plan->world_size, plan->shard, (float)fa.inv64, master_in,
                        m_in, v_in, master_out, m_out, v_out, param_bf16_slot_out,
                        adam_scalars(args), workspace, fa, dev_result, stream),
                    "reduce_adam_1pass_bf16 launch");
}

static int slot_restore(const zero_plan_t* plan, int32_t rank, const float* master,
                        uint16_t* slot, const zero_step_result_t* dev_result, bool bf16,
                        hipStream_t stream) {
  g_err[0] = 0;
  int rc = check_plan_rank(plan, rank);
  if (rc) return rc;
  if (!dev_result) return fail(ZERO_EINVAL, "dev_result is NULL");
  if (!aligned(dev_result, 8)) return fail(ZERO_EALIGN, "dev_result not 8-byte aligned");
  if (plan->shard == 0) return ZERO_OK;
  if (!master || !slot) return fail(ZERO_EINVAL, "NULL state pointer");
  if (!aligned(master, 4)) return fail(ZERO_EALIGN, "master not 4-byte aligned");
  if (!aligned(slot, 2)) return fail(ZERO_EALIGN, "slot not 2-byte aligned");
  if (overlap(master, 4 * (size_t)plan->shard, slot, 2 * (size_t)plan->shard))
    return fail(ZERO_EINVAL, "slot overlaps master");
  return hip_status(zk::launch_slot_restore(master, slot, plan->shard, bf16, dev_result, stream),
                    "slot restore launch");
}

int zero_slot_restore(const zero_plan_t* plan, int32_t rank, const float* master,
                      uint16_t* param16_slot, const zero_step_result_t* dev_result,
                      hipStream_t stream) {
  return slot_restore(plan, rank, master, param16_slot, dev_result, false, stream);
}

int zero_slot_restore_bf16(const zero_plan_t* plan, int32_t rank, const float* master,
                           uint16_t* param_bf16_slot, const zero_step_result_t* dev_result,
                           hipStream_t stream) {
  return slot_restore(plan, rank, master, param_bf16_slot, dev_result, true, stream);
}

int zero_reduce_check_bf16(const zero_plan_t* plan, int32_t rank, const uint16_t* const* contrib,
                           const zero_step_args_t* args, float* grad_out, void* workspace,
                           size_t ws_bytes, zero_step_result_t* dev_result, hipStream_t stream) {
  g_err[0] = 0;
  int rc = check_plan_rank(plan, rank);
  if (!rc) rc = check_norm_args(args);
  if (!rc && (args->other_q_lo || args->other_q_hi))
    rc = fail(ZERO_EINVAL, "the bf16 path takes the other ranks' share as other_sq only");
  if (!rc) rc = check_reduce_ptrs(plan, contrib, grad_out, workspace, ws_bytes, dev_result);
  if (rc) return rc;
  const zk::FinalizeArgs fa = finalize_args(plan, args);
  return hip_status(zk::launch_reduce_check_bf16(contrib, (int)plan->world_size, plan->shard,
                                                 (float)fa.inv64, grad_out, workspace, fa,
                                                 dev_result, stream),
                    "bf16 reduce_check launch");
}

int zero_finalize_bf16(const zero_plan_t* plan, const zero_step_args_t* args,
                       zero_step_result_t* dev_result, hipStream_t stream) {
  g_err[0] = 0;
  int rc = check_plan_rank(plan, 0);
  if (!rc) rc = check_norm_args(args);
  if (!rc && (args->other_q_lo || args->other_q_hi))
    rc = fail(ZERO_EINVAL, "the bf16 path takes the other ranks' share as other_sq only");
  if (rc) return rc;
  if (!dev_result) return fail(ZERO_EINVAL, "dev_result is NULL");
  if (!aligned(dev_result, 8)) return fail(ZERO_EALIGN, "dev_result not 8-byte aligned");
  return hip_status(zk::launch_finalize_bf16(finalize_args(plan, args), dev_result, stream),
                    "bf16 finalize launch");
}

int zero_adam_apply_bf16(const zero_plan_t* plan, int32_t rank, const float* grad, float* master,
                         float* m, float* v, uint16_t* param_bf16_slot,
                         const zero_step_args_t* args, const zero_step_result_t* dev_result,
                         hipStream_t stream) {
  g_err[0] = 0;
  int rc = check_plan_rank(plan, rank);
  if (!rc) rc = check_adam_args(args);
  if (!rc) rc = check_adam_ptrs(plan, grad, master, m, v, param_bf16_slot, dev_result);
  if (rc) return rc;
  if (plan->shard == 0) return ZERO_OK;
  return hip_status(zk::launch_adam_bf16(grad, master, m, v, param_bf16_slot, plan->shard,
                                         adam_scalars(args), dev_result, stream),
                    "bf16 adam launch");
}

int zero_reduce_adam_step_bf16(const zero_plan_t* plan, int32_t rank,
                               const uint16_t* const* contrib, float* master, float* m, float* v,
                               uint16_t* param_bf16_slot, float* grad_out, void* workspace,
                               size_t ws_bytes, const zero_step_args_t* args,
                               zero_step_result_t* dev_result, hipStream_t stream) {
  g_err[0] = 0;
  int rc = check_plan_rank(plan, rank);
  if (!rc) rc = check_adam_args(args);
  if (!rc) rc = check_reduce_ptrs(plan, contrib, grad_out, workspace, ws_bytes, dev_result);
  if (!rc) rc = check_adam_ptrs(plan, grad_out, master, m, v, param_bf16_slot, dev_result);
  if (rc) return rc;
  rc = zero_reduce_check_bf16(plan, rank, contrib, args, grad_out, workspace, ws_bytes, dev_result,
                              stream);
  if (rc || args->other_overflow) return rc;  // a certain skip: no update launch
  return zero_adam_apply_bf16(plan, rank, grad_out, master, m, v, param_bf16_slot, args,
                              dev_result, stream);
}

int zero_plan_units(const int64_t* numels, int32_t n_tensors, const int32_t* unit_of_tensor,
                    int32_t world_size, int32_t align_elems, zero_unit_plan_t* plan_out,
                    zero_unit_info_t* units_out, int32_t units_cap) {
  g_err[0] = 0;
  if (n_tensors < 0 || (n_tensors > 0 && (!numels || !unit_of_tensor)) || !plan_out ||
      units_cap < 0 || (units_cap > 0 && !units_out))
    return fail(ZERO_EINVAL, "NULL or negative argument");
  if (world_size < 1 || align_elems < 1) return fail(ZERO_EINVAL, "world_size and align >= 1");
  int64_t n_units = 0;
  for (int32_t i = 0; i < n_tensors; ++i) {
    const int32_t u = unit_of_tensor[i];
    if (numels[i] < 0) return fail(ZERO_EINVAL, "numel %d is negative", i);
    if ((i == 0 && u != 0) || (i > 0 && u != unit_of_tensor[i - 1] && u != unit_of_tensor[i - 1] + 1))
      return fail(ZERO_EINVAL, "units must be consecutive runs numbered from 0 (tensor %d)", i);
    n_units = (int64_t)u + 1;
  }
  int64_t psi = 0, roff = 0, t = 0;
  for (int64_t u = 0; u < n_units; ++u) {
    int64_t pu = 0;
    for (; t < n_tensors && unit_of_tensor[t] == u; ++t) {
      if (numels[t] > INT64_MAX / 4 - pu) return fail(ZERO_EINVAL, "unit size overflows");
      pu += numels[t];
    }
    const int64_t per = pu / world_size + (pu % world_size ? 1 : 0);
    const int64_t su = (per / align_elems + (per % align_elems ? 1 : 0)) * align_elems;
    if (u < units_cap) {
      units_out[u].psi = pu;
      units_out[u].shard = su;
      units_out[u].flat_offset = psi;
      units_out[u].rank_offset = roff;
    }
    if (pu > INT64_MAX / 4 - psi || su > INT64_MAX / 4 - roff)
      return fail(ZERO_EINVAL, "sizes overflow");
    psi += pu;
    roff += su;
  }
  plan_out->n_units = n_units;
  plan_out->world_size = world_size;
  plan_out->align = align_elems;
  plan_out->psi = psi;
  plan_out->rank_shard = roff;
  if (n_units > units_cap) return fail(ZERO_ENOSPC, "%lld units, capacity %d", (long long)n_units, units_cap);
  return ZERO_OK;
}

namespace {

// Checks a unit table and computes each unit's first workgroups; with
// `fill`, stores them, else compares them.
int units_layout(zero_unit_buffers_t* units, const zero_unit_buffers_t* cunits, int32_t n_units,
                 bool fill, int64_t* k1_total, int64_t* k2_total) {
  if (n_units < 0 || (n_units > 0 && !cunits)) return fail(ZERO_EINVAL, "bad unit table");
  int64_t b1 = 0, b2 = 0;
  for (int32_t u = 0; u < n_units; ++u) {
    const zero_unit_buffers_t& x = cunits[u];
    if (x.shard < 0 || x.shard > ZERO_MAX_SHARD)
      return fail(ZERO_EINVAL, "unit %d: shard outside 0..%lld", u, (long long)ZERO_MAX_SHARD);
    if (x.shard > 0) {
      if (!x.contrib || !x.grad || !x.master || !x.m || !x.v || !x.param16)
        return fail(ZERO_EINVAL, "unit %d: NULL pointer", u);
      if (x.ld < x.shard || (x.ld & 7))
        return fail(ZERO_EINVAL, "unit %d: ld must be >= shard and a multiple of 8", u);
      if (!aligned(x.contrib, 16) || !aligned(x.grad, 16) || !aligned(x.master, 16) ||
          !aligned(x.m, 16) || !aligned(x.v, 16))
        return fail(ZERO_EALIGN, "unit %d: contrib, grad, master, m, v need 16-byte alignment", u);
      if (!aligned(x.param16, 2)) return fail(ZERO_EALIGN, "unit %d: param16 not 2-byte aligned", u);
    }
    const int64_t n2 = x.shard > 0 ? zk::k2_blocks(x.shard) : 0;
    if (fill) {
      units[u].reduce_block = b1;
      units[u].adam_block = b2;
    } else if (x.reduce_block != b1 || x.adam_block != b2) {
      return fail(ZERO_EINVAL, "unit table not prepared by zero_units_prepare (unit %d)", u);
    }
    b1 += zk::k1_blocks(x.shard);
    b2 += n2;
    if (b1 > 0x7FFFFFFFll || b2 > 0x7FFFFFFFll) return fail(ZERO_EINVAL, "grid too large");
  }
  *k1_total = b1;
  *k2_total = b2;
  return ZERO_OK;
}

// The kernels read the table from device memory.  Each call writes the table
// it has just checked into the caller's device table buffer on its own
// stream, ahead of its kernels, so no kernel can read a table other than the
// one validated on the host (a stale or mismatched device copy is simply
// overwritten).  The entries travel by value in the arguments of a small
// store kernel, so the host table is read before the call returns and no
// copy engine reads caller memory later.
int upload_table(zero_unit_buffers_t* units_dev, const zero_unit_buffers_t* units_host,
                 int32_t n_units, hipStream_t stream) {
  if (n_units == 0) return ZERO_OK;
  if (!units_dev) return fail(ZERO_EINVAL, "units_dev is NULL");
  if (!aligned(units_dev, 8)) return fail(ZERO_EALIGN, "units_dev not 8-byte aligned");
  return hip_status(zk::launch_store_table(units_host, n_units, units_dev, stream),
                    "unit table store launch");
}

}  // namespace

int zero_units_prepare(zero_unit_buffers_t* units, int32_t n_units, int64_t* reduce_blocks_out,
                       int64_t* adam_blocks_out) {
  g_err[0] = 0;
  int64_t b1 = 0, b2 = 0;
  const int rc = units_layout(units, units, n_units, true, &b1, &b2);
  if (rc) return rc;
  if (reduce_blocks_out) *reduce_blocks_out = b1;
  if (adam_blocks_out) *adam_blocks_out = b2;
  return ZERO_OK;
}

size_t zero_units_workspace_bytes(const zero_unit_buffers_t* units, int32_t n_units) {
  int64_t b1 = 0, b2 = 0;
  if (units_layout(nullptr, units, n_units, false, &b1, &b2)) return 0;
  return zk::workspace_bytes_for_blocks(b1);
}

int zero_units_reduce_check(int32_t world_size, const zero_unit_buffers_t* units_host,
                            zero_unit_buffers_t* units_dev, int32_t n_units,
                            const zero_step_args_t* args, void* workspace, size_t ws_bytes,
                            zero_step_result_t* dev_result, hipStream_t stream) {
  g_err[0] = 0;
  if (world_size < 1 || world_size > ZERO_MAX_RANKS)
    return fail(ZERO_EINVAL, "world_size outside 1..%d", ZERO_MAX_RANKS);
  int rc = check_norm_args(args);
  if (rc) return rc;
  int64_t b1 = 0, b2 = 0;
  rc = units_layout(nullptr, units_host, n_units, false, &b1, &b2);
  if (rc) return rc;
  if (n_units > 0 && !units_dev) return fail(ZERO_EINVAL, "units_dev is NULL");
  if (!dev_result) return fail(ZERO_EINVAL, "dev_result is NULL");
  if (!aligned(dev_result, 8)) return fail(ZERO_EALIGN, "dev_result not 8-byte aligned");
  if (!workspace) return fail(ZERO_EINVAL, "workspace is NULL");
  if (!aligned(workspace, 16)) return fail(ZERO_EALIGN, "workspace not 16-byte aligned");
  const size_t need = zk::workspace_bytes_for_blocks(b1);
  if (ws_bytes < need) return fail(ZERO_ENOSPC, "workspace %zu bytes < %zu", ws_bytes, need);
  zero_plan_t pl{0, world_size, 1, 0, 0};
  const zk::FinalizeArgs fa = finalize_args(&pl, args);
  if (b1 == 0)  // no units: Q = 0, nothing overflowed
    return hip_status(zk::launch_finalize_empty(fa, dev_result, stream), "finalize launch");
  rc = upload_table(units_dev, units_host, n_units, stream);
  if (rc) return rc;
  int64_t n_partials = 0;
  rc = hip_status(zk::launch_units_reduce(units_dev, n_units, b1, world_size, (float)fa.inv64,
                                          workspace, &n_partials, stream),
                  "units reduce launch");
  if (rc) return rc;
  return hip_status(zk::launch_partials_finalize(workspace, n_partials, fa, dev_result, stream),
                    "finalize launch");
}

// zero_units_adam_apply with or without the table upload (zero_units_step
// has uploaded it already, ahead of its reduce).
static int units_adam(const zero_unit_buffers_t* units_host, zero_unit_buffers_t* units_dev,
                      int32_t n_units, const zero_step_args_t* args,
                      const zero_step_result_t* dev_result, bool upload, hipStream_t stream) {
  int rc = check_adam_args(args);
  if (rc) return rc;
  int64_t b1 = 0, b2 = 0;
  rc = units_layout(nullptr, units_host, n_units, false, &b1, &b2);
  if (rc) return rc;
  if (n_units > 0 && !units_dev) return fail(ZERO_EINVAL, "units_dev is NULL");
  if (!dev_result) return fail(ZERO_EINVAL, "dev_result is NULL");
  if (!aligned(dev_result, 8)) return fail(ZERO_EALIGN, "dev_result not 8-byte aligned");
  if (b2 == 0) return ZERO_OK;
  if (upload) {
    rc = upload_table(units_dev, units_host, n_units, stream);
    if (rc) return rc;
  }
  return hip_status(zk::launch_units_adam(units_dev, n_units, b2, adam_scalars(args), dev_result,
                                          stream),
                    "units adam launch");
}

int zero_units_adam_apply(const zero_unit_buffers_t* units_host,
                          zero_unit_buffers_t* units_dev, int32_t n_units,
                          const zero_step_args_t* args, const zero_step_result_t* dev_result,
                          hipStream_t stream) {
  g_err[0] = 0;
  return units_adam(units_host, units_dev, n_units, args, dev_result, true, stream);
}

int zero_units_step(int32_t world_size, const zero_unit_buffers_t* units_host,
                    zero_unit_buffers_t* units_dev, int32_t n_units,
                    const zero_step_args_t* args, void* workspace, size_t ws_bytes,
                    zero_step_result_t* dev_result, hipStream_t stream) {
  g_err[0] = 0;
  int rc = check_adam_args(args);
  if (rc) return rc;
  rc = zero_units_reduce_check(world_size, units_host, units_dev, n_units, args, workspace,
                               ws_bytes, dev_result, stream);
  if (rc || args->other_overflow) return rc;  // a certain skip: no update launch
  return units_adam(units_host, units_dev, n_units, args, dev_result, false, stream);
}

int zero_units_step_1pass(int32_t world_size, const zero_unit_buffers_t* units_host,
                          zero_unit_buffers_t* units_dev, const zero_unit_buffers_t* out_host,
                          zero_unit_buffers_t* out_dev, int32_t n_units,
                          const zero_step_args_t* args, void* workspace, size_t ws_bytes,
                          zero_step_result_t* dev_result, hipStream_t stream) {
  g_err[0] = 0;
  if (world_size < 1 || world_size > ZERO_MAX_RANKS)
    return fail(ZERO_EINVAL, "world_size outside 1..%d", ZERO_MAX_RANKS);
  int rc = check_adam_args(args);
  if (rc) return rc;
  if (args->max_grad_norm > 0.0)
    return fail(ZERO_EINVAL,
                "max_grad_norm > 0: clipping needs the whole norm before any update "
                "(use the two-pass step)");
  int64_t b1 = 0, b2 = 0, o1 = 0, o2 = 0;
  rc = units_layout(nullptr, units_host, n_units, false, &b1, &b2);
  if (!rc) rc = units_layout(nullptr, out_host, n_units, false, &o1, &o2);
  if (rc) return rc;
  if (n_units > 0 && (!units_dev || !out_dev)) return fail(ZERO_EINVAL, "a device table is NULL");
  for (int32_t u = 0; u < n_units; ++u) {
    const zero_unit_buffers_t& x = units_host[u];
    const zero_unit_buffers_t& y = out_host[u];
    if (x.shard != y.shard) return fail(ZERO_EINVAL, "unit %d: out table shard differs", u);
    if (x.shard == 0) continue;
    const size_t b4 = 4 * (size_t)x.shard, bh = 2 * (size_t)x.shard;
    const void* ins[3] = {x.master, x.m, x.v};
    const void* outs[4] = {y.master, y.m, y.v, y.param16};
    const size_t ob[4] = {b4, b4, b4, bh};
    for (int o = 0; o < 4; ++o) {
      for (int i = 0; i < 3; ++i)
        if (overlap(outs[o], ob[o], ins[i], b4))
          return fail(ZERO_EINVAL, "unit %d: an output state buffer overlaps an input", u);
      for (int q = 0; q < o; ++q)
        if (overlap(outs[o], ob[o], outs[q], ob[q]))
          return fail(ZERO_EINVAL, "unit %d: output state buffers overlap", u);
    }
  }
  if (!dev_result) return fail(ZERO_EINVAL, "dev_result is NULL");
  if (!aligned(dev_result, 8)) return fail(ZERO_EALIGN, "dev_result not 8-byte aligned");
  if (!workspace) return fail(ZERO_EINVAL, "workspace is NULL");
  if (!aligned(workspace, 16)) return fail(ZERO_EALIGN, "workspace not 16-byte aligned");
  const size_t need = zk::workspace_bytes_for_blocks(b1);
  if (ws_bytes < need) return fail(ZERO_ENOSPC, "workspace %zu bytes < %zu", ws_bytes, need);
  zero_plan_t pl{0, world_size, 1, 0, 0};
  const zk::FinalizeArgs fa = finalize_args(&pl, args);
  if (b1 == 0)
    return hip_status(zk::launch_finalize_empty(fa, dev_result, stream), "finalize launch");
  {
    const size_t tb = (size_t)n_units * sizeof(zero_unit_buffers_t);
    const uintptr_t a = (uintptr_t)units_dev, b = (uintptr_t)out_dev;
    if (a < b + tb && b < a + tb) return fail(ZERO_EINVAL, "units_dev and out_dev overlap");
  }
  rc = upload_table(units_dev, units_host, n_units, stream);
  if (!rc) rc = upload_table(out_dev, out_host, n_units, stream);
  if (rc) return rc;
  rc = hip_status(zk::launch_units_reduce_adam_1pass(units_dev, out_dev, n_units, b1,
                                                     world_size, (float)fa.inv64,
                                                     adam_scalars(args), workspace, stream),
                  "units single-pass launch");
  if (rc) return rc;
  return hip_status(zk::launch_partials_finalize(workspace, b1, fa, dev_result, stream),
                    "finalize launch");
}

int zero_units_slot_restore(const zero_unit_buffers_t* units_host,
                            zero_unit_buffers_t* units_dev, int32_t n_units,
                            const zero_step_result_t* dev_result, hipStream_t stream) {
  g_err[0] = 0;
  int64_t b1 = 0, b2 = 0;
  int rc = units_layout(nullptr, units_host, n_units, false, &b1, &b2);
  if (rc) return rc;
  if (n_units > 0 && !units_dev) return fail(ZERO_EINVAL, "units_dev is NULL");
  if (!dev_result) return fail(ZERO_EINVAL, "dev_result is NULL");
  if (!aligned(dev_result, 8)) return fail(ZERO_EALIGN, "dev_result not 8-byte aligned");
  int64_t max_shard = 0;
  for (int32_t u = 0; u < n_units; ++u) {
    const zero_unit_buffers_t& x = units_host[u];
    if (x.shard > max_shard) max_shard = x.shard;
    if (x.shard > 0 && overlap(x.master, 4 * (size_t)x.shard, x.param16, 2 * (size_t)x.shard))
      return fail(ZERO_EINVAL, "unit %d: slot overlaps master", u);
  }
  if (max_shard == 0) return ZERO_OK;
  rc = upload_table(units_dev, units_host, n_units, stream);
  if (rc) return rc;
  return hip_status(zk::launch_units_slot_restore(units_dev, n_units, max_shard, dev_result,
                                                  stream),
                    "units slot restore launch");
}

int zero_scaler_update(zero_scaler_t* s, int32_t skipped) {
  g_err[0] = 0;
  if (!s || !(s->scale > 0.0)) return fail(ZERO_EINVAL, "NULL scaler or scale <= 0");
  if (skipped) {
    const double next = s->scale * s->backoff;
    s->scale = next > s->min_scale ? next : s->min_scale;
    s->good_steps = 0;
    return ZERO_OK;
  }
  s->t += 1;
  s->good_steps += 1;
  if (s->good_steps >= s->growth_interval) {
    s->scale *= s->growth;
    s->good_steps = 0;
  }
  return ZERO_OK;
}

}  // extern "C"
