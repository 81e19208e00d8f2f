// Host side of the C ABI: shard planner, model-state bytes, loss scaler,
// argument checks, fp64 -> fp32 scalar preparation, and the kernel launches.
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include <hip/hip_runtime_api.h>

#include "zero_internal.h"
#include "zero_shard.h"

namespace {

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
// once; beta^t as t left-to-right fp64 products.
zk::AdamScalars adam_scalars(const zero_step_args_t* a) {
  double p1 = a->beta1, p2 = a->beta2;
  for (int64_t i = 1; i < a->step; ++i) {
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

int check_reduce_ptrs(const zero_plan_t* plan, const uint16_t* const* contrib, float* grad_out,
                      void* workspace, size_t ws_bytes, zero_step_result_t* dev_result) {
  if (!dev_result) return fail(ZERO_EINVAL, "dev_result is NULL");
  if (!aligned(dev_result, 8)) return fail(ZERO_EALIGN, "dev_result not 8-byte aligned");
  if (!workspace) return fail(ZERO_EINVAL, "workspace is NULL");
  if (!aligned(workspace, 16)) return fail(ZERO_EALIGN, "workspace not 16-byte aligned");
  const size_t need = zk::workspace_bytes(plan->shard);
  if (ws_bytes < need) return fail(ZERO_ENOSPC, "workspace %zu bytes < %zu", ws_bytes, need);
  if (plan->shard > 0) {
    if (!contrib) return fail(ZERO_EINVAL, "contrib is NULL");
    for (int64_t r = 0; r < plan->world_size; ++r) {
      if (!contrib[r]) return fail(ZERO_EINVAL, "contrib[%lld] is NULL", (long long)r);
      if (!aligned(contrib[r], 16))
        return fail(ZERO_EALIGN, "contrib[%lld] not 16-byte aligned", (long long)r);
    }
    if (!grad_out) return fail(ZERO_EINVAL, "grad_out is NULL");
    if (!aligned(grad_out, 16)) return fail(ZERO_EALIGN, "grad_out not 16-byte aligned");
  }
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

}  // namespace

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
  if (rc) return rc;
  return zero_adam_apply(plan, rank, grad_out, master, m, v, param16_slot, args, dev_result,
                         stream);
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
