// Device kernels of the ZeRO shard step for CDNA4 (gfx950): one flat shard.
//
// K1 (reduce_check): the reduce side of the gradient reduce-scatter, done in
//   HBM ("10.6 ZeRO 与 FSDP", §10.6.1 and §10.6.2 step 2): for each element of
//   the shard, the N fp16 contributions are summed in rank order 0..N-1 into
//   an fp32 accumulator that starts at +0, then scaled by inv = 1/(N*loss
//   scale) and written as the fp32 gradient.  Each thread also forms the
//   overflow flag and the exact sum of acc^2 (a 128-bit integer); each
//   workgroup writes one partial.
// KF (finalize): sums the partials (integer sums, so any order gives the same
//   bits), adds the other ranks' share and makes the clip / skip decision.
// K2 (adam): mixed-precision AdamW on the shard and the fp16 cast into the
//   all-gather slot (§10.6.2 steps 3 and 4), skipped as a whole on overflow.
// K12 (reduce_adam, steps without clipping): K1 and K2 in one pass, reading
//   the current master/m/v and writing a second set and slot, which the
//   caller adopts only if KF finds the step not skipped; no gradient is
//   written.  bf16 forms of K1, K2 and K12 sit at the end of the file.
//
// K1, K2 and K12 stream every element once and use one-shot grids: each thread
// owns one 4-element quad (no grid-stride loop), so workgroups are dispatched
// in address order and retire as they finish; on MI355X this streams
// measurably faster than persistent grids.  Long grids of K1 and K2 go out as
// several launches of consecutive workgroups (launch_segments), which streams
// faster still.  Every load or store instruction
// of a wave covers 512 bytes to 1 KiB contiguous, with nontemporal hints.
// Nothing here is a dense contraction, so no matrix cores are used; HBM
// bandwidth bounds K1, K2 and K12.  The per-quad bodies live in zero_device.h.
#include "zero_device.h"

namespace zk {
namespace {

using namespace dev;

struct ContribTable {
  const uint16_t* p[ZERO_MAX_RANKS];
  __device__ __forceinline__ const uint16_t* row(int r) const { return p[r]; }
};

// b0: the first workgroup of this launch (a long grid runs as several
// launches; see launch_segments).
__global__ __launch_bounds__(ZK_K1_THREADS) void k1_reduce_check(ContribTable ct, int32_t n,
                                                                 int64_t shard, float inv32,
                                                                 float* __restrict__ grad,
                                                                 Partial* __restrict__ partials,
                                                                 uint32_t* __restrict__ ticket,
                                                                 int64_t b0) {
  const int64_t b = b0 + blockIdx.x;
  // KF runs after this kernel on the same stream: arm its ticket here, so the
  // workspace needs no initialisation by the caller.
  if (b == 0 && threadIdx.x == 0) *ticket = 0u;
  const int64_t q_first = b * ZK_K1_THREADS * ZK_K1_QUADS;
  const Partial pt = reduce_block(ct, n, shard, q_first, inv32, grad);
  if (threadIdx.x == 0) partials[b] = pt;
}

// K1 above N = 8: each workgroup covers ZK_K1_DEFER chunks and stores their
// gradients together at the end (see reduce_block_deferred).
__global__ __launch_bounds__(ZK_K1_THREADS) void k1_reduce_check_deferred(
    ContribTable ct, int32_t n, int64_t shard, float inv32, float* __restrict__ grad,
    Partial* __restrict__ partials, uint32_t* __restrict__ ticket, int64_t b0) {
  const int64_t b = b0 + blockIdx.x;
  if (b == 0 && threadIdx.x == 0) *ticket = 0u;
  const int64_t q_first = b * ZK_K1_THREADS * ZK_K1_DEFER;
  const Partial pt = reduce_block_deferred<ZK_K1_DEFER>(ct, n, shard, q_first, inv32, grad);
  if (threadIdx.x == 0) partials[b] = pt;
}

__global__ __launch_bounds__(kThreads) void kf_reduce_finalize(
    const Partial* __restrict__ partials, int64_t n_partials, Partial* __restrict__ level2,
    uint32_t* __restrict__ ticket, FinalizeArgs fa, zero_step_result_t* __restrict__ res) {
  reduce_partials_and_finalize(partials, n_partials, level2, ticket, fa, res);
}

__global__ void k_finalize(FinalizeArgs fa, zero_step_result_t* res) {
  if (threadIdx.x == 0 && blockIdx.x == 0)
    finalize_into(res->own_q_lo, res->own_q_hi, (uint32_t)res->overflow, fa, res);
}

// Thread t of workgroup b = b0 + blockIdx.x owns quads (b*Q + u)*T + t, u < Q.
__global__ __launch_bounds__(ZK_K2_THREADS) void k2_adam(
    const float* __restrict__ grad, float* __restrict__ master, float* __restrict__ mom,
    float* __restrict__ var, uint16_t* __restrict__ slot, int64_t shard, AdamScalars sc,
    const zero_step_result_t* __restrict__ res, int64_t b0) {
  if (res->skip) return;
  const float c = res->clip_coef;
  const int64_t b = b0 + blockIdx.x;
#pragma unroll
  for (int u = 0; u < ZK_K2_QUADS; ++u) {
    const int64_t qd = (b * ZK_K2_QUADS + u) * ZK_K2_THREADS + threadIdx.x;
    adam_quad(grad, master, mom, var, slot, shard, qd, c, sc);
  }
}

// K12 (single pass, steps without clipping): K1's reduce and partial plus
// the update with clip coefficient 1, from the `in` state into the distinct
// `out` state and slot.  KF then finalizes as after K1.
__global__ __launch_bounds__(ZK_K12_THREADS) void k12_reduce_adam(
    ContribTable ct, int32_t n, int64_t shard, float inv32, StatePair st, AdamScalars sc,
    Partial* __restrict__ partials, uint32_t* __restrict__ ticket, int64_t b0) {
  const int64_t b = b0 + blockIdx.x;
  if (b == 0 && threadIdx.x == 0) *ticket = 0u;
  uint64_t qlo = 0, qhi = 0;
  uint32_t bad = 0;
  const int64_t qd = b * ZK_K12_THREADS + threadIdx.x;
  reduce_adam_quad(ct, n, shard, qd, inv32, st, sc, qlo, qhi, bad);
  block_reduce<ZK_K12_THREADS>(qlo, qhi, bad);
  if (threadIdx.x == 0) partials[b] = make_partial(qlo, qhi, bad);
}

// --- bf16 path -------------------------------------------------------------
__global__ __launch_bounds__(ZK_K1_THREADS) void k1_reduce_check_bf16(
    ContribTable ct, int32_t n, int64_t shard, float inv32, float* __restrict__ grad,
    Partial* __restrict__ partials, uint32_t* __restrict__ ticket, int64_t b0) {
  const int64_t b = b0 + blockIdx.x;
  if (b == 0 && threadIdx.x == 0) *ticket = 0u;  // arm the tree kernel's ticket
  const int64_t q_first = b * ZK_K1_THREADS;
  const Partial pt = reduce_block_bf16(ct, n, shard, q_first, inv32, grad);
  if (threadIdx.x == 0) partials[b] = pt;
}

// K12 in bf16: the single pass with the bf16 tree partial of K1's bf16 form.
__global__ __launch_bounds__(ZK_K1_THREADS) void k12_reduce_adam_bf16(
    ContribTable ct, int32_t n, int64_t shard, float inv32, StatePair st, AdamScalars sc,
    Partial* __restrict__ partials, uint32_t* __restrict__ ticket, int64_t b0) {
  const int64_t b = b0 + blockIdx.x;
  if (b == 0 && threadIdx.x == 0) *ticket = 0u;
  uint32_t bad = 0;
  const int64_t qd = b * ZK_K1_THREADS + threadIdx.x;
  double x = reduce_adam_quad_bf16(ct, n, shard, qd, inv32, st, sc, bad);
  block_tree<ZK_K1_THREADS>(x, bad);
  if (threadIdx.x == 0)
    partials[b] = Partial{(uint64_t)__double_as_longlong(x), (uint64_t)(bad ? 1u : 0u) << 63};
}

__global__ __launch_bounds__(kThreads) void kt_tree_finalize_bf16(
    const Partial* __restrict__ partials, int64_t n_partials, int chunk,
    Partial* __restrict__ level2, uint32_t* __restrict__ ticket, FinalizeArgs fa,
    zero_step_result_t* __restrict__ res) {
  tree_partials_and_finalize_bf16(partials, n_partials, chunk, level2, ticket, fa, res);
}

__global__ void k_finalize_bf16(FinalizeArgs fa, zero_step_result_t* res) {
  // re-finalize from the stored own share (own_sq) with new other-rank values
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    const double own = res->own_sq;
    const uint32_t bad = (uint32_t)res->overflow;
    const double tot = own + fa.other_sq;
    const double norm = __builtin_sqrt(tot);
    double coef = 1.0;
    if (fa.max_norm > 0.0) {
      const double c = fa.max_norm / (norm + 1e-6);
      coef = (c < 1.0) ? c : 1.0;
    }
    res->total_sq = tot;
    res->norm = norm;
    res->clip_coef = (float)coef;
    res->skip = (bad || fa.other_overflow) ? 1 : 0;
  }
}

__global__ __launch_bounds__(ZK_K2_THREADS) void k2_adam_bf16(
    const float* __restrict__ grad, float* __restrict__ master, float* __restrict__ mom,
    float* __restrict__ var, uint16_t* __restrict__ slot, int64_t shard, AdamScalars sc,
    const zero_step_result_t* __restrict__ res, int64_t b0) {
  if (res->skip) return;
  const float c = res->clip_coef;
  const int64_t b = b0 + blockIdx.x;
#pragma unroll
  for (int u = 0; u < ZK_K2_QUADS; ++u) {
    const int64_t qd = (b * ZK_K2_QUADS + u) * ZK_K2_THREADS + threadIdx.x;
    adam_quad<Fmt::BF16>(grad, master, mom, var, slot, shard, qd, c, sc);
  }
}

// Slot restore after a skipped single pass that wrote the live slot: the
// slot is the 16-bit cast of the master, so recasting the unchanged master
// gives back its content before the step.  A no-op unless res->skip; a small
// grid-stride grid, so that the common no-op costs one short launch.
template <Fmt F>
__global__ __launch_bounds__(kThreads) void k_slot_restore(const float* __restrict__ master,
                                                           uint16_t* __restrict__ slot,
                                                           int64_t shard,
                                                           const zero_step_result_t* __restrict__ res) {
  if (!res->skip) return;
  for (int64_t j = (int64_t)blockIdx.x * kThreads + threadIdx.x; j < shard;
       j += (int64_t)gridDim.x * kThreads)
    slot[j] = (uint16_t)from_f32<F>(master[j]);
}

}  // namespace

int64_t k1_blocks_bf16(int64_t shard) {
  const int64_t quads = (shard + 3) >> 2;
  const int64_t b = (quads + ZK_K1_THREADS - 1) / ZK_K1_THREADS;
  return b < 1 ? 1 : b;
}

int64_t k1_blocks(int64_t shard) {
  const int64_t units = (shard + 3) >> 2;  // quads, the ragged one included
  const int64_t per = (int64_t)ZK_K1_THREADS * ZK_K1_QUADS;
  const int64_t b = (units + per - 1) / per;
  return b < 1 ? 1 : b;
}

int64_t k1_blocks_deferred(int64_t shard) {
  const int64_t units = (shard + 3) >> 2;  // quads, the ragged one included
  const int64_t per = (int64_t)ZK_K1_THREADS * ZK_K1_DEFER;
  const int64_t b = (units + per - 1) / per;
  return b < 1 ? 1 : b;
}

int64_t k12_blocks(int64_t shard) {  // one quad per thread
  const int64_t quads = (shard + 3) >> 2;
  const int64_t b = (quads + ZK_K12_THREADS - 1) / ZK_K12_THREADS;
  return b < 1 ? 1 : b;
}

int64_t k2_blocks(int64_t shard) {
  const int64_t quads = (shard + 3) >> 2;
  const int64_t per = (int64_t)ZK_K2_THREADS * ZK_K2_QUADS;
  const int64_t b = (quads + per - 1) / per;
  return b < 1 ? 1 : b;
}

size_t workspace_bytes_for_blocks(int64_t reduce_blocks) {
  return kTicketBytes + (size_t)kFinBlocks * kPartialBytes + (size_t)reduce_blocks * kPartialBytes;
}

size_t workspace_bytes(int64_t shard) {
  int64_t a = k1_blocks(shard);
  const int64_t b = k1_blocks_bf16(shard), c = k12_blocks(shard);
  if (b > a) a = b;
  if (c > a) a = c;
  return workspace_bytes_for_blocks(a);
}

void* workspace_partials(void* workspace) {
  return (char*)workspace + kTicketBytes + (size_t)kFinBlocks * kPartialBytes;
}

int launch_partials_finalize(void* workspace, int64_t n_partials, const FinalizeArgs& fa,
                             zero_step_result_t* res, hipStream_t stream) {
  uint32_t* ticket = (uint32_t*)workspace;
  Partial* level2 = (Partial*)((char*)workspace + kTicketBytes);
  Partial* partials = level2 + kFinBlocks;
  int64_t fb = (n_partials + kThreads * 4 - 1) / (kThreads * 4);
  if (fb > kFinBlocks) fb = kFinBlocks;
  if (fb < 1) fb = 1;
  hipLaunchKernelGGL(kf_reduce_finalize, dim3((uint32_t)fb), dim3(kThreads), 0, stream, partials,
                     n_partials, level2, ticket, fa, res);
  return (int)hipGetLastError();
}

int launch_reduce_check(const uint16_t* const* contrib, int n, int64_t shard, float inv32,
                        float* grad, void* workspace, const FinalizeArgs& fa,
                        zero_step_result_t* res, hipStream_t stream) {
  ContribTable ct;
  for (int r = 0; r < ZERO_MAX_RANKS; ++r) ct.p[r] = r < n ? contrib[r] : nullptr;
  const bool deferred = n > 8;
  const int64_t blocks = deferred ? k1_blocks_deferred(shard) : k1_blocks(shard);
  Partial* partials = (Partial*)workspace_partials(workspace);
  uint32_t* ticket = (uint32_t*)workspace;
  int e;
  if (deferred)
    e = launch_segments(blocks, ZK_K1_DEFER_SEG_ELEMS / (4 * ZK_K1_THREADS * ZK_K1_DEFER),
                        [&](int64_t b0, int64_t nb) {
                          hipLaunchKernelGGL(k1_reduce_check_deferred, dim3((uint32_t)nb),
                                             dim3(ZK_K1_THREADS), ZK_K1_DEFER_LDS, stream, ct, n,
                                             shard, inv32, grad, partials, ticket, b0);
                        });
  else
    e = launch_segments(blocks, ZK_K1_SEG_ELEMS / (4 * ZK_K1_THREADS * ZK_K1_QUADS),
                        [&](int64_t b0, int64_t nb) {
                          hipLaunchKernelGGL(k1_reduce_check, dim3((uint32_t)nb),
                                             dim3(ZK_K1_THREADS), k1_lds(n), stream, ct, n, shard,
                                             inv32, grad, partials, ticket, b0);
                        });
  if (e != hipSuccess) return e;
  return launch_partials_finalize(workspace, blocks, fa, res, stream);
}

__global__ void k_finalize_empty(FinalizeArgs fa, zero_step_result_t* res) {
  if (threadIdx.x == 0 && blockIdx.x == 0) finalize_into(0ull, 0ull, 0u, fa, res);
}

int launch_finalize_empty(const FinalizeArgs& fa, zero_step_result_t* res, hipStream_t stream) {
  hipLaunchKernelGGL(k_finalize_empty, dim3(1), dim3(64), 0, stream, fa, res);
  return (int)hipGetLastError();
}

int launch_finalize(const FinalizeArgs& fa, zero_step_result_t* res, hipStream_t stream) {
  hipLaunchKernelGGL(k_finalize, dim3(1), dim3(64), 0, stream, fa, res);
  return (int)hipGetLastError();
}

int launch_reduce_adam_1pass(const uint16_t* const* contrib, int n, int64_t shard, float inv32,
                             const float* master_in, const float* m_in, const float* v_in,
                             float* master_out, float* m_out, float* v_out, uint16_t* slot_out,
                             const AdamScalars& sc, void* workspace, const FinalizeArgs& fa,
                             zero_step_result_t* res, hipStream_t stream) {
  ContribTable ct;
  for (int r = 0; r < ZERO_MAX_RANKS; ++r) ct.p[r] = r < n ? contrib[r] : nullptr;
  const StatePair st{master_in, m_in, v_in, master_out, m_out, v_out, slot_out};
  const int64_t blocks = k12_blocks(shard);
  Partial* partials = (Partial*)workspace_partials(workspace);
  uint32_t* ticket = (uint32_t*)workspace;
  const int e = launch_segments(blocks, k12_seg_elems(n) / (4 * ZK_K12_THREADS),
                                [&](int64_t b0, int64_t nb) {
                                  hipLaunchKernelGGL(k12_reduce_adam, dim3((uint32_t)nb),
                                                     dim3(ZK_K12_THREADS), k12_lds(n), stream, ct,
                                                     n, shard, inv32, st, sc, partials, ticket,
                                                     b0);
                                });
  if (e != hipSuccess) return e;
  return launch_partials_finalize(workspace, blocks, fa, res, stream);
}

// The bf16 tree kernel over `blocks` workgroup partials: power-of-two chunks
// with at most kFinBlocks workgroups, the last one finalizing.
static int launch_tree_finalize_bf16(void* workspace, int64_t blocks, const FinalizeArgs& fa,
                                     zero_step_result_t* res, hipStream_t stream) {
  uint32_t* ticket = (uint32_t*)workspace;
  Partial* level2 = (Partial*)((char*)workspace + kTicketBytes);
  Partial* partials = (Partial*)workspace_partials(workspace);
  int64_t per = (blocks + kFinBlocks - 1) / kFinBlocks;
  int64_t chunk = 1;
  while (chunk < per) chunk <<= 1;
  if (chunk > kTreeChunk) return (int)hipErrorInvalidValue;
  const int64_t fb = (blocks + chunk - 1) / chunk;
  hipLaunchKernelGGL(kt_tree_finalize_bf16, dim3((uint32_t)fb), dim3(kThreads), 0, stream,
                     partials, blocks, (int)chunk, level2, ticket, fa, res);
  return (int)hipGetLastError();
}

int launch_reduce_check_bf16(const uint16_t* const* contrib, int n, int64_t shard, float inv32,
                             float* grad, void* workspace, const FinalizeArgs& fa,
                             zero_step_result_t* res, hipStream_t stream) {
  ContribTable ct;
  for (int r = 0; r < ZERO_MAX_RANKS; ++r) ct.p[r] = r < n ? contrib[r] : nullptr;
  const int64_t blocks = k1_blocks_bf16(shard);
  uint32_t* ticket = (uint32_t*)workspace;
  Partial* partials = (Partial*)workspace_partials(workspace);
  const int e = launch_segments(blocks, ZK_K1_SEG_ELEMS / (4 * ZK_K1_THREADS),
                                [&](int64_t b0, int64_t nb) {
                                  hipLaunchKernelGGL(k1_reduce_check_bf16, dim3((uint32_t)nb),
                                                     dim3(ZK_K1_THREADS), ZK_K1B_LDS, stream, ct,
                                                     n, shard, inv32, grad, partials, ticket, b0);
                                });
  if (e != hipSuccess) return e;
  return launch_tree_finalize_bf16(workspace, blocks, fa, res, stream);
}

int launch_reduce_adam_1pass_bf16(const uint16_t* const* contrib, int n, int64_t shard,
                                  float inv32, const float* master_in, const float* m_in,
                                  const float* v_in, float* master_out, float* m_out,
                                  float* v_out, uint16_t* slot_out, const AdamScalars& sc,
                                  void* workspace, const FinalizeArgs& fa,
                                  zero_step_result_t* res, hipStream_t stream) {
  ContribTable ct;
  for (int r = 0; r < ZERO_MAX_RANKS; ++r) ct.p[r] = r < n ? contrib[r] : nullptr;
  const StatePair st{master_in, m_in, v_in, master_out, m_out, v_out, slot_out};
  const int64_t blocks = k1_blocks_bf16(shard);
  Partial* partials = (Partial*)workspace_partials(workspace);
  uint32_t* ticket = (uint32_t*)workspace;
  const int e = launch_segments(blocks, k12_seg_elems(n) / (4 * ZK_K1_THREADS),
                                [&](int64_t b0, int64_t nb) {
                                  hipLaunchKernelGGL(k12_reduce_adam_bf16, dim3((uint32_t)nb),
                                                     dim3(ZK_K1_THREADS), ZK_K12B_LDS, stream, ct,
                                                     n, shard, inv32, st, sc, partials, ticket,
                                                     b0);
                                });
  if (e != hipSuccess) return e;
  return launch_tree_finalize_bf16(workspace, blocks, fa, res, stream);
}

int launch_slot_restore(const float* master, uint16_t* slot, int64_t shard, bool bf16,
                        const zero_step_result_t* res, hipStream_t stream) {
  int64_t blocks = (shard + kThreads - 1) / kThreads;
  if (blocks > kRestoreBlocks) blocks = kRestoreBlocks;
  if (blocks < 1) blocks = 1;
  if (bf16)
    hipLaunchKernelGGL(k_slot_restore<Fmt::BF16>, dim3((uint32_t)blocks), dim3(kThreads), 0,
                       stream, master, slot, shard, res);
  else
    hipLaunchKernelGGL(k_slot_restore<Fmt::F16>, dim3((uint32_t)blocks), dim3(kThreads), 0,
                       stream, master, slot, shard, res);
  return (int)hipGetLastError();
}

int launch_finalize_bf16(const FinalizeArgs& fa, zero_step_result_t* res, hipStream_t stream) {
  hipLaunchKernelGGL(k_finalize_bf16, dim3(1), dim3(64), 0, stream, fa, res);
  return (int)hipGetLastError();
}

constexpr int64_t kK2SegBlocks = ZK_K2_SEG_ELEMS / (4 * ZK_K2_THREADS * ZK_K2_QUADS);

int launch_adam_bf16(const float* grad, float* master, float* m, float* v, uint16_t* slot,
                     int64_t shard, const AdamScalars& sc, const zero_step_result_t* res,
                     hipStream_t stream) {
  return launch_segments(k2_blocks(shard), kK2SegBlocks, [&](int64_t b0, int64_t nb) {
    hipLaunchKernelGGL(k2_adam_bf16, dim3((uint32_t)nb), dim3(ZK_K2_THREADS), ZK_K2_LDS, stream,
                       grad, master, m, v, slot, shard, sc, res, b0);
  });
}

int launch_adam(const float* grad, float* master, float* m, float* v, uint16_t* slot,
                int64_t shard, const AdamScalars& sc, const zero_step_result_t* res,
                hipStream_t stream) {
  return launch_segments(k2_blocks(shard), kK2SegBlocks, [&](int64_t b0, int64_t nb) {
    hipLaunchKernelGGL(k2_adam, dim3((uint32_t)nb), dim3(ZK_K2_THREADS), ZK_K2_LDS, stream,
                       grad, master, m, v, slot, shard, sc, res, b0);
  });
}

}  // namespace zk
