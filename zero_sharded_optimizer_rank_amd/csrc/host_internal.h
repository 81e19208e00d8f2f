// Host-side helpers shared by the C-ABI source files: error reporting,
// argument checks and the fp64 -> fp32 preparation of the Adam scalars.
#pragma once

#include <stdint.h>

#include "zero_internal.h"
#include "zero_shard.h"

namespace zk {
namespace host {

extern thread_local char g_err[512];

// Record a printf-style message for zero_last_error and return `code`.
int fail(int code, const char* fmt, ...);
bool aligned(const void* p, uintptr_t a);
int check_plan_rank(const zero_plan_t* plan, int32_t rank);
int check_norm_args(const zero_step_args_t* a);
int check_adam_args(const zero_step_args_t* a);
int check_rows(const zero_plan_t* plan, const uint16_t* const* contrib);
int check_adam_ptrs(const zero_plan_t* plan, const float* grad, float* master, float* m, float* v,
                    uint16_t* slot, const zero_step_result_t* dev_result);
FinalizeArgs finalize_args(const zero_plan_t* plan, const zero_step_args_t* a);
AdamScalars adam_scalars(const zero_step_args_t* a);
int hip_status(int e, const char* what);

}  // namespace host
}  // namespace zk
