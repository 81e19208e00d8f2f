/*
 * zero_shard.h -- C ABI of one data-parallel rank's ZeRO step on its 1/N shard,
 * for AMD Instinct MI355X (gfx950).
 *
 * The step (pages: "10.6 ZeRO 与 FSDP", §10.6.1-§10.6.3; "第13篇 · ZeRO", §3.2;
 * "ZeRO-1/2/3 分别优化了什么", sections on ZeRO-1 and ZeRO-2):
 *   1. reduce side of the gradient reduce-scatter, done locally: sum the N
 *      ranks' fp16 contributions to this rank's slice in rank order 0..N-1
 *      with fp32 accumulation, then average and unscale by the loss scale;
 *   2. detect inf/NaN and form the exact partial squared L2 norm; combine it
 *      with the other ranks' into the clip coefficient and the skip decision;
 *   3. mixed-precision Adam/AdamW on the fp32 master, m and v of the shard;
 *   4. cast the new master to fp16 into this rank's slot of the flat
 *      parameter buffer (the all-gather's local slot).
 *
 * Conventions for every entry point:
 *   - int-returning calls return ZERO_OK (0) or a negative zero_status; the
 *     message of the last failure on the calling thread is zero_last_error().
 *   - Device calls are asynchronous on the given HIP stream; results in
 *     device memory are readable once the caller synchronises that stream.
 *   - The library allocates no memory.  Every buffer is owned by the caller
 *     and must stay alive until the stream has passed the call.  The only
 *     device memory the library holds is the fixed scratch array of
 *     zero_reduce_adam_step_noalloc, a variable of its loaded code object.
 *   - Pointers marked "device" are HIP device pointers; "host" are host
 *     pointers read before the call returns.
 *   - A workspace or result buffer used by one call must not be used by an
 *     overlapping call on another stream.
 *   - The buffers passed to one call must not overlap one another (the
 *     kernels read and write them as distinct memory); only the in-place
 *     state arrays (master, m, v) are read and written by the same call.
 *   - Placement (performance only): the kernels stream several buffers at
 *     once; buffers whose starts differ by a multiple of 64 KiB put the same
 *     element of every stream on the same HBM interleave and run a few
 *     percent slower.  Starting consecutive buffers 4 KiB apart modulo
 *     64 KiB (odd multiples of 4 KiB between any two) avoids that.
 *
 * The hyperparameters arrive as fp64 and are rounded to fp32 once on the host
 * (1 - beta1 is f32(0.1), not 1f - 0.9f); beta^t is a product of t fp64
 * factors.  The Adam sequence is Kingma & Ba Adam with bias correction, eps
 * outside the square root, and decoupled weight decay on the old parameter;
 * each fp32 operation is rounded separately (no fused multiply-add), with
 * correctly rounded division and square root.
 */
#ifndef ZERO_SHARD_H
#define ZERO_SHARD_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum zero_status {
  ZERO_OK = 0,
  ZERO_EINVAL = -1, /* bad argument value or size */
  ZERO_EALIGN = -2, /* a pointer lacks the alignment stated below */
  ZERO_ENOSPC = -3, /* a caller buffer is too small */
  ZERO_EHIP = -4    /* a HIP runtime call or kernel launch failed */
};

/* Largest N the device calls accept (contribution pointers travel as kernel
 * arguments). */
#define ZERO_MAX_RANKS 64
/* Largest shard, in elements, the device calls accept. */
#define ZERO_MAX_SHARD ((int64_t)0x7FFFFFF8)

typedef struct zero_plan {
  int64_t psi;        /* real parameters in the flat buffer */
  int64_t world_size; /* N */
  int64_t align;      /* shard size is a multiple of this many elements */
  int64_t shard;      /* S: elements owned by each rank, padding included */
  int64_t psi_padded; /* N * S */
} zero_plan_t;

/*
 * zero_plan: flatten a tensor list and partition it into N equal shards.
 * Pages: "第13篇 · ZeRO", §2.1 (gradients gathered into one flat buffer) and
 * §3.2 (process i stores and updates partition i); "10.6 ZeRO 与 FSDP",
 * §10.6.2 (each GPU owns and updates 1/N).
 *   numels        host [n_tensors], element counts (>= 0), in flat order
 *   world_size    N, >= 1
 *   align_elems   >= 1; S = ceil(psi / N) rounded up to a multiple of it
 *   plan_out      host, filled on success
 *   offsets_out   host [n_tensors], caller-owned: exclusive prefix sum of
 *                 numels (tensor i starts at flat index offsets_out[i]);
 *                 may be NULL
 * Rank r owns flat [r*S, (r+1)*S); flat indexes >= psi are padding, which
 * holds zero contributions and zero state and stays zero.  Pure host code.
 * Errors: ZERO_EINVAL for a NULL numels with n_tensors > 0, n_tensors < 0, a
 * negative numel, world_size < 1, align_elems < 1 or an int64 overflow.
 */
int zero_plan(const int64_t* numels, int32_t n_tensors, int32_t world_size, int32_t align_elems,
              zero_plan_t* plan_out, int64_t* offsets_out);

/* Real (non-padding) elements in rank's shard: clamp(psi - rank*S, 0, S);
 * -1 for a NULL plan or a rank outside [0, N). */
int64_t zero_plan_real(const zero_plan_t* plan, int32_t rank);

typedef struct zero_segment {
  int32_t tensor;       /* index into the tensor list */
  int32_t reserved;
  int64_t tensor_begin; /* first element of the tensor inside this shard */
  int64_t shard_begin;  /* where that element sits in the shard */
  int64_t length;       /* elements in this piece */
} zero_segment_t;

/*
 * zero_plan_segments: the pieces of each tensor that fall in rank's shard,
 * in flat order (same pages as zero_plan).
 *   offsets  host [n_tensors] as returned by zero_plan
 *   out      host [cap], caller-owned; *n_out receives the piece count
 * Errors: ZERO_EINVAL for NULL arguments or a bad rank; ZERO_ENOSPC when more
 * than cap pieces exist (*n_out still receives the count).
 */
int zero_plan_segments(const zero_plan_t* plan, const int64_t* numels, const int64_t* offsets,
                       int32_t n_tensors, int32_t rank, zero_segment_t* out, int32_t cap,
                       int32_t* n_out);

/*
 * zero_state_bytes: model-state bytes per rank for mixed-precision training
 * with K bytes of optimizer state per parameter (K = 12 for Adam: fp32
 * master, momentum and variance).
 *   stage 0 (plain data parallel): (4 + K) psi
 *   stage 1 (optimizer states sharded): 4 psi + K psi / N
 *   stage 2 (+ gradients sharded): 2 psi + (2 + K) psi / N
 *   stage 3 (+ parameters sharded): (4 + K) psi / N
 * Pages: "ZeRO-1/2/3 分别优化了什么" (训练状态的显存构成 and each stage's
 * 显存节省); "第13篇 · ZeRO", §2.2 and §3.2; "10.6 ZeRO 与 FSDP", table 10-2.
 * Returns the byte count, or -1.0 for stage outside 0..3, psi < 0, n < 1,
 * k < 0 or a NaN argument.
 */
double zero_state_bytes(int32_t stage, double psi, double n, double k);

typedef struct zero_step_args {
  double lr, beta1, beta2, eps;
  double weight_decay;   /* decoupled (AdamW); 0 gives Adam */
  double max_grad_norm;  /* <= 0: no clipping */
  double loss_scale;     /* the loss scale the contributions carry, > 0 */
  int64_t step;          /* 1-based Adam step t of this update if it applies */
  double other_sq;       /* other ranks' squared norm as a plain fp64 value, >= 0 */
  uint64_t other_q_lo;   /* other ranks' exact sum of squared fp32 sums, in */
  uint64_t other_q_hi;   /*   units of 2^-48 (128-bit; an exact all-reduce) */
  int32_t other_overflow; /* nonzero: another rank saw inf/NaN */
  int32_t reserved;
} zero_step_args_t;

/*
 * Written to device memory by zero_reduce_check / zero_finalize, read by
 * zero_adam_apply.  With Q = sum over the shard of acc_j^2 in units of 2^-48
 * (exact), inv = 1 / (N * loss_scale) in fp64 and f64() one rounding to
 * nearest even:
 *   own_sq    = ((f64(Q) * 2^-48) * inv) * inv
 *   total_sq  = ((f64(Q + other_q) * 2^-48) * inv) * inv + other_sq
 *   norm      = sqrt(total_sq)
 *   clip_coef = f32(min(1, max_grad_norm / (norm + 1e-6))), or 1 without clipping
 *   skip      = overflow || other_overflow || Q + other_q >= 2^128
 */
typedef struct zero_step_result {
  uint64_t own_q_lo, own_q_hi;
  double own_sq;
  double total_sq;
  double norm;
  float clip_coef;
  int32_t overflow; /* this shard's sums held inf or NaN */
  int32_t skip;     /* the update was (or will be) skipped */
  int32_t reserved;
} zero_step_result_t;

/* Bytes of workspace the reduce (zero_reduce_check and the other calls that
 * take a workspace) needs for plan->shard elements:
 * 256 + 16 * (256 + ceil(ceil(S / 4) / 64)), about S / 16 bytes; 0 for a
 * NULL plan or a shard outside 0..ZERO_MAX_SHARD.  The workspace needs no
 * initialisation (the reduce kernel arms its own counter). */
size_t zero_workspace_bytes(const zero_plan_t* plan);

/*
 * zero_reduce_check: step 1 and 2 for rank's shard of S = plan->shard elements.
 * Pages: "10.6 ZeRO 与 FSDP", §10.6.1 (reduce-scatter: reduce, keep 1/N) and
 * §10.6.2 step 2; "ZeRO-1/2/3 分别优化了什么", ZeRO-2 (each card receives the
 * average of all cards' gradients); the tutorial's "gradient_clipping": 1.0
 * (§4.2) and loss scaling (§4.3).
 *   contrib    host [N] of device pointers; contrib[r] holds rank r's S fp16
 *              values (IEEE binary16 bit patterns) for this shard; 16-byte
 *              aligned (required), 256-byte aligned rows stream about 10%
 *              faster (whole cache lines per wave load)
 *   args       host; loss_scale, max_grad_norm, other_* are read
 *   grad_out   device [S] fp32, 16-byte aligned: g_j = f32(acc_j * f32(inv))
 *              with acc_j = (...((+0 + c_0j) + c_1j) + ...) + c_(N-1)j in fp32
 *   workspace  device, >= zero_workspace_bytes(plan), 16-byte aligned; its
 *              content on entry does not matter
 *   dev_result device, 8-byte aligned; fully written
 * Errors: ZERO_EINVAL (N outside 1..ZERO_MAX_RANKS, bad rank, S outside
 * 0..ZERO_MAX_SHARD, NULL pointers, loss_scale <= 0, other_sq < 0 or not
 * finite, max_grad_norm NaN), ZERO_EALIGN, ZERO_ENOSPC (workspace), ZERO_EHIP.
 */
int zero_reduce_check(const zero_plan_t* plan, int32_t rank, const uint16_t* const* contrib,
                      const zero_step_args_t* args, float* grad_out, void* workspace,
                      size_t ws_bytes, zero_step_result_t* dev_result, hipStream_t stream);

/*
 * zero_finalize: recompute norm, clip_coef and skip of dev_result from its
 * own_q and overflow and from new args (other ranks' values).  The host uses
 * it to stand in for the all-reduce of {Q, overflow} when it simulates
 * several ranks.  dev_result: device, written by an earlier zero_reduce_check.
 * Errors: as zero_reduce_check for args and dev_result.
 */
int zero_finalize(const zero_plan_t* plan, const zero_step_args_t* args,
                  zero_step_result_t* dev_result, hipStream_t stream);

/*
 * zero_adam_apply: steps 3 and 4 unless dev_result->skip.
 * Pages: "10.6 ZeRO 与 FSDP", §10.6.2 step 3 (local 1/N optimizer state and
 * gradient update the local 1/N parameters) and step 4 (all-gather of the
 * updated parameters); "第13篇 · ZeRO", §2.2 (fp32 master, momentum, variance).
 *   grad                device [S] fp32 from zero_reduce_check, 16-byte aligned
 *   master, m, v        device [S] fp32, in place, 16-byte aligned
 *   param16_slot        device [S] fp16 bit patterns = flat16 + rank * S;
 *                       2-byte aligned (any shard offset)
 *   args                host; lr, betas, eps, weight_decay, step, loss_scale
 *   dev_result          device; clip_coef and skip are read
 * Per element, one rounding per line:
 *   gc = g*c;  m = b1*m + (1-b1)*gc;  v = b2*v + (1-b2)*(gc*gc);
 *   den = sqrt(v)/sqrt(1-b2^t) + eps;  u = (m/den) * (lr/(1-b1^t));
 *   p = p*(1-lr*wd) - u;  slot = fp16(p) rounded to nearest even.
 * On a skipped step nothing is written.
 * Errors: ZERO_EINVAL (bad args: lr or eps negative or NaN, a beta outside
 * [0, 1), step < 1, NULL pointers), ZERO_EALIGN, ZERO_EHIP.
 */
int zero_adam_apply(const zero_plan_t* plan, int32_t rank, const float* grad, float* master,
                    float* m, float* v, uint16_t* param16_slot, const zero_step_args_t* args,
                    const zero_step_result_t* dev_result, hipStream_t stream);

/*
 * zero_reduce_adam_step: the whole step, zero_reduce_check then
 * zero_adam_apply, enqueued back to back with no host synchronisation.
 * When args->other_overflow is set the finalize is certain to skip the step,
 * so the update kernel is not launched (dev_result is as after any skip).
 * Arguments and errors as the two calls; nothing is launched if any argument
 * check fails.
 */
int zero_reduce_adam_step(const zero_plan_t* plan, int32_t rank, const uint16_t* const* contrib,
                          float* master, float* m, float* v, uint16_t* param16_slot,
                          float* grad_out, void* workspace, size_t ws_bytes,
                          const zero_step_args_t* args, zero_step_result_t* dev_result,
                          hipStream_t stream);

/*
 * zero_reduce_adam_step_noalloc: zero_reduce_adam_step for callers that
 * cannot allocate device memory or pass a workspace (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  The
 * reduce's workspace comes from a device array the library holds, one per
 * GPU, of 36 MiB + 4352 B: enough for shards of up to ZERO_NOALLOC_MAX_SHARD
 * elements.  The call allocates nothing; the first call on a device resolves
 * that device's array address (a runtime symbol lookup, no allocation), so
 * make one call per device before capturing it in a graph.
 * Every call on a GPU shares that GPU's array: calls that overlap on one GPU
 * (other streams, other threads) race and must not be issued; calls in
 * sequence on one stream are safe.  Kernels, results and bits are those of
 * zero_reduce_adam_step.
 * Arguments: as zero_reduce_adam_step without workspace and ws_bytes.
 * Errors: as zero_reduce_adam_step, plus ZERO_ENOSPC for a shard above
 * ZERO_NOALLOC_MAX_SHARD (checked before anything touches the GPU), and
 * ZERO_EHIP if the device or the array's address cannot be obtained.
 */
#define ZERO_NOALLOC_MAX_SHARD ((int64_t)1207959552) /* 9 * 2^27 */
int zero_reduce_adam_step_noalloc(const zero_plan_t* plan, int32_t rank,
                                  const uint16_t* const* contrib, float* master, float* m,
                                  float* v, uint16_t* param16_slot, float* grad_out,
                                  const zero_step_args_t* args, zero_step_result_t* dev_result,
                                  hipStream_t stream);

/*
 * zero_reduce_adam_step_1pass: the whole step in one streaming pass, for steps
 * without gradient clipping (args->max_grad_norm <= 0), e.g. a GPT-2-sized
 * model trained with dynamic loss scaling and no clipping.  Pages: as
 * zero_reduce_check and zero_adam_apply; the tutorial's loss scaling (§4.3)
 * supplies the only global dependency left, the skip on overflow.
 * Without clipping, no element's update depends on the shard's norm, only on
 * whether any rank overflowed.  So one kernel reduces the contributions, adds
 * the exact squares to the partial sums and applies the update (clip
 * coefficient 1) from the `in` state into a second, distinct `out` state and
 * slot; the finalize then writes dev_result as zero_reduce_check does.  The
 * gradient is never written: the step moves 2N + 26 bytes per element instead
 * of 2N + 34.
 *   contrib, workspace, ws_bytes, dev_result   as zero_reduce_check
 *   master_in, m_in, v_in     device [S] fp32, 16-byte aligned, read only
 *   master_out, m_out, v_out  device [S] fp32, 16-byte aligned, written
 *   param16_slot_out          device [S] fp16 bit patterns, 2-byte aligned:
 *                             either a second flat buffer's slot at rank * S,
 *                             or the live slot itself (see zero_slot_restore)
 *   args                      as zero_reduce_adam_step; max_grad_norm <= 0
 * Results: when dev_result->skip is 0 the out state and slot hold exactly what
 * zero_reduce_adam_step would have left in master, m, v and the slot (the
 * caller adopts them, e.g. by swapping buffer sets); when it is 1 they hold
 * unspecified values and the in state is the unchanged state (the caller
 * keeps it; with a second slot buffer, it also keeps the old slot; with the
 * live slot as param16_slot_out, the slot holds garbage until
 * zero_slot_restore has run after the step's final finalize, and nothing may
 * read it before).  dev_result is bit-identical to zero_reduce_check's with
 * clip_coef 1.  Across ranks, the caller all-reduces own_q and overflow after
 * the pass and calls zero_finalize with the other ranks' values; the skip it
 * writes then decides the adoption on every rank alike.
 * When to use it: it saves the gradient's round trip (8 of 2N + 34 bytes per
 * element), which pays at small N (Llama-3-8B at N = 8: 6.62 ms against
 * 7.59 ms on an MI355X).  At N = 64 the contribution rows are 83% of its bytes
 * and its mixed stream of 67 inputs and 4 outputs runs about 10% below the
 * reduce's rate, so the two-pass step is faster there (GPT-2 shard 0.60
 * against 0.64 ms, flat 7.5B shard 2.75 against 2.93 ms): use
 * zero_reduce_adam_step above N = 8.
 * Errors: as zero_reduce_adam_step, plus ZERO_EINVAL for max_grad_norm > 0,
 * for an out buffer that overlaps an in buffer, and for out buffers that
 * overlap one another.  Nothing is launched if a check fails.
 */
int zero_reduce_adam_step_1pass(const zero_plan_t* plan, int32_t rank,
                                const uint16_t* const* contrib, const float* master_in,
                                const float* m_in, const float* v_in, float* master_out,
                                float* m_out, float* v_out, uint16_t* param16_slot_out,
                                void* workspace, size_t ws_bytes, const zero_step_args_t* args,
                                zero_step_result_t* dev_result, hipStream_t stream);

/*
 * zero_slot_restore / zero_slot_restore_bf16: let a single pass write the live
 * slot in place.  The single pass never reads the slot, so param16_slot_out
 * may be the live slot itself (flat16 + rank * S) instead of a second flat
 * buffer; a skipped step then leaves garbage there.  After the step's final
 * finalize (zero_reduce_adam_step_1pass's own, or zero_finalize after the
 * exchange between ranks), this call rewrites the slot as the fp16 (bf16)
 * cast of `master`, rounded to nearest even, if dev_result->skip is set, and
 * does nothing otherwise; no host synchronisation is needed.  Pass the set
 * the step read (master_in), which a skip leaves unchanged: since every step
 * leaves the slot equal to the cast of the master, this gives back the slot's
 * content before the step.
 *   master        device [S] fp32, 4-byte aligned, read
 *   param16_slot  device [S] 16-bit slot, 2-byte aligned, rewritten on a skip
 *   dev_result    device, as written by the step's finalize; skip is read
 * Errors: ZERO_EINVAL (plan, rank, NULL pointers, slot overlapping master),
 * ZERO_EALIGN, ZERO_EHIP.
 */
int zero_slot_restore(const zero_plan_t* plan, int32_t rank, const float* master,
                      uint16_t* param16_slot, const zero_step_result_t* dev_result,
                      hipStream_t stream);
int zero_slot_restore_bf16(const zero_plan_t* plan, int32_t rank, const float* master,
                           uint16_t* param_bf16_slot, const zero_step_result_t* dev_result,
                           hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* bf16 variant: bfloat16 gradient contributions and parameter slot, no loss
 * scaling needed (the tutorial's §4.3 suggests bf16 where the hardware has it,
 * instead of tuning fp16 loss scaling); fp32 master, m, v and the Adam
 * sequence are unchanged.  bf16 keeps fp32's exponent range, so the shard's
 * squared norm is not the exact integer of the fp16 path but the balanced
 * pairwise tree, in fp64, of the exact squares acc_j^2 over element indices
 * zero-padded to a power of two: one fixed order for every launch shape.
 *   own_sq = (tree * inv) * inv;  total_sq = own_sq + other_sq
 *   (own_q_lo / own_q_hi are 0; args->other_q must be 0)
 * Arguments, layouts and errors as in the fp16 calls; contribution rows and
 * the slot hold bfloat16 bit patterns.  The workspace is the same size.
 * zero_finalize_bf16 keeps dev_result's own_sq and overflow and recomputes
 * total_sq, norm, clip_coef and skip from new args. */
int zero_reduce_check_bf16(const zero_plan_t* plan, int32_t rank, const uint16_t* const* contrib,
                           const zero_step_args_t* args, float* grad_out, void* workspace,
                           size_t ws_bytes, zero_step_result_t* dev_result, hipStream_t stream);
int zero_finalize_bf16(const zero_plan_t* plan, const zero_step_args_t* args,
                       zero_step_result_t* dev_result, hipStream_t stream);
int zero_adam_apply_bf16(const zero_plan_t* plan, int32_t rank, const float* grad, float* master,
                         float* m, float* v, uint16_t* param_bf16_slot,
                         const zero_step_args_t* args, const zero_step_result_t* dev_result,
                         hipStream_t stream);
int zero_reduce_adam_step_bf16(const zero_plan_t* plan, int32_t rank,
                               const uint16_t* const* contrib, float* master, float* m, float* v,
                               uint16_t* param_bf16_slot, float* grad_out, void* workspace,
                               size_t ws_bytes, const zero_step_args_t* args,
                               zero_step_result_t* dev_result, hipStream_t stream);
/* zero_reduce_adam_step_1pass_bf16: zero_reduce_adam_step_1pass with bf16
 * contribution rows and a bf16 slot, and dev_result as zero_reduce_check_bf16
 * writes it (the pairwise tree norm; args->other_q must be 0).  Arguments,
 * results and errors otherwise as zero_reduce_adam_step_1pass. */
int zero_reduce_adam_step_1pass_bf16(const zero_plan_t* plan, int32_t rank,
                                     const uint16_t* const* contrib, const float* master_in,
                                     const float* m_in, const float* v_in, float* master_out,
                                     float* m_out, float* v_out, uint16_t* param_bf16_slot_out,
                                     void* workspace, size_t ws_bytes,
                                     const zero_step_args_t* args,
                                     zero_step_result_t* dev_result, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* ZeRO-Offload form of the update ("10.6 ZeRO 与 FSDP" §10.6.6: the GPU
 * keeps forward and backward, gradients travel to the CPU over PCIe, the CPU
 * updates the parameters from optimizer state held in host memory and sends
 * the fp16 parameters back; the tutorial's offload_optimizer setting).  The
 * reduce, unscale, overflow check and norm stay on the GPU (zero_reduce_check);
 * the fp32 master, m and v live in host memory; the host runs the same
 * separately rounded fp32 Adam sequence as the GPU kernel, so the results
 * are identical bit for bit. */

#define ZERO_MAX_HOST_THREADS 256

/* Pinned host staging for the PCIe pipeline, caller-owned (allocate it with
 * hipHostMalloc or an equivalent pinned allocation): two chunks of fp32
 * gradient and two of fp16 parameters, used alternately so that copies in
 * both directions overlap the host's arithmetic. */
typedef struct zero_offload_staging {
  float* grad_pinned;       /* [2 * chunk] */
  uint16_t* param16_pinned; /* [2 * chunk] */
  int64_t chunk;            /* elements per pipeline chunk: a positive multiple of 64 */
  hipStream_t upload_stream; /* stream for the host-to-device copies of the fp16 chunks, so
                                both PCIe directions run at once; NULL: the call's stream.
                                Caller-owned, default priority. */
} zero_offload_staging_t;

/* Bytes of pinned staging for a chunk size (both buffers); 0 if chunk is not
 * a positive multiple of 64. */
size_t zero_offload_staging_bytes(int64_t chunk);

/*
 * zero_host_adam_apply: the host update on host arrays of `count` elements:
 * Adam/AdamW with clip coefficient clip_coef (in (0, 1]) on grad, in place on
 * master, m, v, and the fp16 (round to nearest even) copy of the new master
 * into param16.  No alignment needed.  threads: 1..ZERO_MAX_HOST_THREADS
 * worker threads (the caller's included).  vector_width: 0 = the widest
 * available, 1 = scalar, 8 = AVX2 + F16C, 16 = AVX-512F; every width gives
 * the same bits.  Synchronous; no GPU involved.
 * Errors: ZERO_EINVAL (bad args as zero_adam_apply, count < 0, NULL arrays,
 * clip_coef outside (0, 1], threads out of range, a width the CPU lacks).
 */
int zero_host_adam_apply(const float* grad, float* master, float* m, float* v,
                         uint16_t* param16, int64_t count, const zero_step_args_t* args,
                         float clip_coef, int32_t threads, int32_t vector_width);

/*
 * zero_offload_adam_apply: the update of the offload form.  Reads the step
 * result (dev_result, written by zero_reduce_check on `stream`), waits for
 * it, and copies it to *result_out when result_out is not NULL.  On a skip it
 * returns with nothing changed.  Otherwise it streams grad_dev (device,
 * fp32 [S]) to the host chunk by chunk, updates master_host, m_host, v_host
 * (host fp32 [S], in place, any alignment) and copies the fp16 parameters
 * into param16_slot_dev (device, = flat16 + rank*S, 2-byte aligned).  The
 * gradient copies run on `stream`, the parameter copies on the staging's
 * upload stream (or `stream`); the call returns when the last copy has
 * finished.
 * Errors: as zero_adam_apply, plus ZERO_EINVAL for bad staging or threads.
 * After a ZERO_EHIP in the middle, the host state may be partly updated.
 */
int zero_offload_adam_apply(const zero_plan_t* plan, int32_t rank, const float* grad_dev,
                            float* master_host, float* m_host, float* v_host,
                            uint16_t* param16_slot_dev, const zero_step_args_t* args,
                            const zero_step_result_t* dev_result,
                            const zero_offload_staging_t* staging, int32_t threads,
                            zero_step_result_t* result_out, hipStream_t stream);

/* zero_offload_step: zero_reduce_check on the GPU, then
 * zero_offload_adam_apply; arguments as those two calls. */
int zero_offload_step(const zero_plan_t* plan, int32_t rank, const uint16_t* const* contrib,
                      float* grad_dev, void* workspace, size_t ws_bytes, float* master_host,
                      float* m_host, float* v_host, uint16_t* param16_slot_dev,
                      const zero_step_args_t* args, zero_step_result_t* dev_result,
                      const zero_offload_staging_t* staging, int32_t threads,
                      zero_step_result_t* result_out, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* ZeRO-3 / FSDP units: each unit (a run of consecutive tensors, e.g. one
 * transformer block) is flattened and sharded on its own, and one launch of
 * each kernel updates every unit a rank holds.  Pages: "10.6 ZeRO 与 FSDP",
 * §10.6.4 (stage 3: each GPU updates its 1/N of the parameters from its 1/N
 * of the optimizer state and gradient) and §10.6.7 (FSDP units are flattened,
 * sharded and gathered together; one unit per transformer block). */

typedef struct zero_unit_plan {
  int64_t n_units, world_size, align;
  int64_t psi;        /* real parameters over all units */
  int64_t rank_shard; /* elements a rank holds over all units (sum of S_u) */
} zero_unit_plan_t;

typedef struct zero_unit_info {
  int64_t psi;         /* real parameters of the unit */
  int64_t shard;       /* S_u = ceil(psi_u / N) rounded up to align */
  int64_t flat_offset; /* first model element of the unit */
  int64_t rank_offset; /* where the unit's shard starts in a rank's concatenation */
} zero_unit_info_t;

/*
 * zero_plan_units: plan FSDP units.  unit_of_tensor[i] is tensor i's unit;
 * units are consecutive runs numbered 0, 1, 2, ...  Unit u is flattened in
 * list order and padded on its own to N * S_u; rank r owns [r*S_u, (r+1)*S_u)
 * of it.  units_out: host [units_cap], caller-owned.  Pure host code.
 * Errors: ZERO_EINVAL (NULL arguments, a negative numel, units not numbered
 * as runs from 0, world_size or align < 1, overflow), ZERO_ENOSPC (more units
 * than units_cap; plan_out is still filled).
 */
int zero_plan_units(const int64_t* numels, int32_t n_tensors, const int32_t* unit_of_tensor,
                    int32_t world_size, int32_t align_elems, zero_unit_plan_t* plan_out,
                    zero_unit_info_t* units_out, int32_t units_cap);

/* One unit's buffers on this rank (all device pointers, all caller-owned). */
typedef struct zero_unit_buffers {
  const uint16_t* contrib; /* N fp16 rows: row r at contrib + r*ld; 16-byte aligned */
  int64_t ld;              /* elements between rows: >= shard, a multiple of 8 */
  float* grad;             /* [shard] fp32, 16-byte aligned (reduce output) */
  float* master;           /* [shard] fp32, 16-byte aligned, in place */
  float* m;                /* [shard] fp32, 16-byte aligned, in place */
  float* v;                /* [shard] fp32, 16-byte aligned, in place */
  uint16_t* param16;       /* [shard] fp16 slot of this rank's piece, 2-byte aligned */
  int64_t shard;           /* S_u, elements (padding included) */
  int64_t reduce_block;    /* first 512-element reduce chunk: set by zero_units_prepare */
  int64_t adam_block;      /* first Adam workgroup: set by zero_units_prepare */
} zero_unit_buffers_t;

/*
 * zero_units_prepare: check a host unit table and fill reduce_block and
 * adam_block; also return the workgroup totals.  The calls below take the
 * prepared host table and a device buffer for it, which each call fills with
 * the table it has just checked before its kernels read it.
 * Errors: ZERO_EINVAL (n_units < 0, NULL pointers, a shard outside
 * 0..ZERO_MAX_SHARD, ld < shard or not a multiple of 8, grid too large),
 * ZERO_EALIGN (alignment as stated in zero_unit_buffers_t).
 */
int zero_units_prepare(zero_unit_buffers_t* units, int32_t n_units, int64_t* reduce_blocks_out,
                       int64_t* adam_blocks_out);

/* Workspace bytes for a prepared table: 256 + 16 * (256 + reduce chunks), the
 * chunk total zero_units_prepare returns (above N = 8 the reduce may write
 * fewer partials).  It needs no initialisation.  0 on bad input. */
size_t zero_units_workspace_bytes(const zero_unit_buffers_t* units, int32_t n_units);

/*
 * zero_units_reduce_check / zero_units_adam_apply / zero_units_step: the
 * flat calls' semantics over all units at once: one squared-norm integer, one
 * overflow flag, one clip coefficient and one skip decision for the rank.
 *   world_size  N (1..ZERO_MAX_RANKS): rows per unit
 *   units_host  host, the prepared table: checked, then read before the call
 *               returns
 *   units_dev   device, n_units * sizeof(zero_unit_buffers_t) bytes, 8-byte
 *               aligned, caller-owned: the call writes units_host there on
 *               `stream` (passed by value through a small kernel's
 *               arguments) ahead of the kernels that read it, so the kernels
 *               only ever see the table checked on the host; its content on
 *               entry does not matter.  Calls in flight at the same time on
 *               different streams need their own units_dev (as they need
 *               their own workspace): each call rewrites it.
 *   workspace, dev_result, args, stream: as in the flat calls
 * Errors: as the flat calls, plus ZERO_EINVAL when units_host was not
 * prepared or units_dev is NULL, ZERO_EALIGN for a misaligned units_dev.
 * Nothing is launched when a check fails.
 */
int zero_units_reduce_check(int32_t world_size, const zero_unit_buffers_t* units_host,
                            zero_unit_buffers_t* units_dev, int32_t n_units,
                            const zero_step_args_t* args, void* workspace, size_t ws_bytes,
                            zero_step_result_t* dev_result, hipStream_t stream);
int zero_units_adam_apply(const zero_unit_buffers_t* units_host,
                          zero_unit_buffers_t* units_dev, int32_t n_units,
                          const zero_step_args_t* args, const zero_step_result_t* dev_result,
                          hipStream_t stream);
int zero_units_step(int32_t world_size, const zero_unit_buffers_t* units_host,
                    zero_unit_buffers_t* units_dev, int32_t n_units,
                    const zero_step_args_t* args, void* workspace, size_t ws_bytes,
                    zero_step_result_t* dev_result, hipStream_t stream);

/*
 * zero_units_step_1pass: zero_reduce_adam_step_1pass over all units at once,
 * for steps without clipping (args->max_grad_norm <= 0).  One launch reduces
 * every unit's rows, adds the exact squares and applies the update from each
 * unit's current master, m, v (units_*) into the master, m, v and param16 of
 * a second prepared table (out_*) with the same shards; no gradient is
 * written.  dev_result is written as zero_units_reduce_check writes it (clip
 * coefficient 1).  When dev_result->skip is 0 the out buffers hold exactly
 * what zero_units_step would have left in the current ones (the caller swaps
 * the tables); when it is 1 they hold unspecified values and the current
 * state is unchanged.  The out table's param16 may point at the live unit
 * slots; then, after a skip, they hold garbage until zero_units_slot_restore
 * has run after the step's final finalize, and nothing may read them before.
 *   units_host, units_dev  the prepared table of the current state: rows
 *                          (contrib, ld) and master, m, v are read; grad is
 *                          not used
 *   out_host, out_dev      a prepared table with the same shards; its master,
 *                          m, v and param16 are written, its other fields are
 *                          not used; out_dev is filled from out_host like
 *                          units_dev, and the two device buffers must not
 *                          overlap
 *   world_size, args, workspace, dev_result, stream: as zero_units_step
 * Errors: as zero_units_step, plus ZERO_EINVAL for max_grad_norm > 0, a shard
 * that differs between the tables, a unit whose out buffers overlap its in
 * buffers or one another, and overlapping device tables.  Nothing is
 * launched when a check fails.
 */
int zero_units_step_1pass(int32_t world_size, const zero_unit_buffers_t* units_host,
                          zero_unit_buffers_t* units_dev, const zero_unit_buffers_t* out_host,
                          zero_unit_buffers_t* out_dev, int32_t n_units,
                          const zero_step_args_t* args, void* workspace, size_t ws_bytes,
                          zero_step_result_t* dev_result, hipStream_t stream);

/*
 * zero_units_slot_restore: zero_slot_restore over all units in one launch,
 * for a unit single pass whose out table points param16 at the live unit
 * slots: if dev_result->skip, every unit's param16 is rewritten as the fp16
 * cast of its master (round to nearest even); otherwise nothing happens.
 *   units_host, units_dev  the prepared table of the current state (the one
 *                          the pass read), with param16 at the live slots;
 *                          units_dev is filled as in zero_units_step
 *   dev_result             as written by the step's final finalize
 * Errors: ZERO_EINVAL (a table not prepared, NULL pointers, a slot that
 * overlaps its unit's master), ZERO_EALIGN, ZERO_EHIP.
 */
int zero_units_slot_restore(const zero_unit_buffers_t* units_host,
                            zero_unit_buffers_t* units_dev, int32_t n_units,
                            const zero_step_result_t* dev_result, hipStream_t stream);

typedef struct zero_scaler {
  double scale;            /* current loss scale */
  double growth, backoff;  /* e.g. 2.0 and 0.5 */
  double min_scale;        /* floor, e.g. 1.0 */
  int64_t growth_interval; /* clean steps before growth, e.g. 1000 */
  int64_t good_steps;      /* clean steps since the last change */
  int64_t t;               /* Adam steps applied so far */
} zero_scaler_t;

/*
 * zero_scaler_update: dynamic loss scaling after a step (host).  The tutorial
 * (§4.3) says fp16 training may need loss scaling; reading: on a skipped step
 * scale = max(scale*backoff, min_scale) and good_steps = 0; otherwise t += 1
 * and after growth_interval clean steps in a row scale *= growth.
 * Errors: ZERO_EINVAL for NULL or a non-positive scale.
 */
int zero_scaler_update(zero_scaler_t* s, int32_t skipped);

/* Message of the last failure on this thread ("" if none). */
const char* zero_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ZERO_SHARD_H */
