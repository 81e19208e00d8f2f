"""CPU oracle for one data-parallel rank's ZeRO step on its 1/N shard.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything here.  The HIP
library never calls it, and it shares no code with the library: the only code
both sides use is the seeded input generator in ``synth/``.

Every function cites the passage of the pages it follows.  The pages are:
  * "ZeRO-1/2/3 分别优化了什么？和普通 DDP 有什么区别？" (interview notes),
  * the "年糕切片" DeepSpeed ZeRO tutorial (ChatGLM2-6B fine-tuning),
  * "第13篇 · ZeRO", close-reading notes on Rajbhandari et al., ZeRO (2019),
  * "10.6 ZeRO 与 FSDP" (LLM full-stack book).
Where the pages leave a step open (Adam's equations, the clip formula, the
loss-scale rule, the reduction order, padding) the plain reading is taken and
stated at the function.

Pin status: every function here is pinned by a CPU test against something
other than itself (printed numbers, closed forms, a library routine, brute
force); see tests/test_oracle_*.py.  No function is parity-unpinned.
"""
from .zero_oracle import (  # noqa: F401
    FinalizeResult, Plan, Scalars, UnitPlan, adam_apply, exact_sq_units, finalize, nonfinite,
    plan, plan_units, reduce_contributions, scaler_update, segments, shard_step, state_bytes,
    step_scalars, unit_model_index, unit_shard_index, unscale,
    bf16_to_f32, f32_to_bf16, finalize_bf16, pairwise_sum_f64, reduce_contributions_bf16,
    shard_step_bf16, sq_tree,
)
