// Multi-unit form of the shard step (ZeRO-3 / FSDP): one grid of the reduce
// and one of the Adam kernel (each issued as consecutive launches when it is
// long, see launch_segments) update every unit a rank holds.
//
// Pages: "10.6 ZeRO 与 FSDP" §10.6.4 (stage 3: each GPU updates its 1/N of
// the parameters from its 1/N of the optimizer state and of the gradient) and
// §10.6.7 (FSDP units: one unit's parameters are flattened and sharded
// together, e.g. one transformer block per unit).  Each unit has its own
// buffers, described by a zero_unit_buffers_t in a device table; workgroups
// are dealt out unit by unit (zero_units_prepare records each unit's first
// workgroup), so a workgroup finds its unit by a binary search and then runs
// the same per-quad bodies as the flat kernels.  The squared norm and the
// overflow flag cover all units together; the clip and skip are global.  The
// single pass over all units (steps without clipping) reads a second table
// whose state buffers receive the update.
#include <stddef.h>

#include "zero_device.h"

namespace zk {
namespace {

using namespace dev;

// The unit table as the kernels read it: the same layout as
// zero_unit_buffers_t, with the buffer pointers typed as global memory.  The
// table's plain pointers would otherwise be generic (flat) addresses, and
// every access to the unit's buffers would become a FLAT instruction that
// waits on both memory counters.
template <typename T>
using gptr = __attribute__((address_space(1))) T*;
struct UnitBuffersGlobal {
  gptr<const uint16_t> contrib;
  int64_t ld;
  gptr<float> grad, master, m, v;
  gptr<uint16_t> param16;
  int64_t shard, reduce_block, adam_block;
};
static_assert(sizeof(UnitBuffersGlobal) == sizeof(zero_unit_buffers_t), "table layout");
static_assert(offsetof(UnitBuffersGlobal, ld) == offsetof(zero_unit_buffers_t, ld), "ld");
static_assert(offsetof(UnitBuffersGlobal, param16) == offsetof(zero_unit_buffers_t, param16),
              "param16");
static_assert(offsetof(UnitBuffersGlobal, adam_block) ==
                  offsetof(zero_unit_buffers_t, adam_block), "adam_block");

struct StridedRows {
  const uint16_t* base;
  int64_t ld;
  __device__ __forceinline__ const uint16_t* row(int r) const { return base + (int64_t)r * ld; }
};

// Largest unit index u with first(u) <= b (units with no workgroups are
// skipped because the next unit starts at the same workgroup).
template <typename First>
__device__ __forceinline__ int32_t find_unit(int32_t n_units, int64_t b, First first) {
  int32_t lo = 0, hi = n_units - 1;
  while (lo < hi) {
    const int32_t mid = (lo + hi + 1) >> 1;
    if (first(mid) <= b) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// b0: the first workgroup of this launch (see launch_segments).
__global__ __launch_bounds__(ZK_K1_THREADS) void k1u_reduce_check(
    const zero_unit_buffers_t* __restrict__ units, int32_t n_units, int32_t n, float inv32,
    Partial* __restrict__ partials, uint32_t* __restrict__ ticket, int64_t b0) {
  const int64_t b = b0 + blockIdx.x;
  if (b == 0 && threadIdx.x == 0) *ticket = 0u;  // arm the finalize kernel's ticket
  const int32_t u = find_unit(n_units, b, [&](int32_t i) { return units[i].reduce_block; });
  const UnitBuffersGlobal& ub = ((const UnitBuffersGlobal*)units)[u];
  const StridedRows rows{(const uint16_t*)ub.contrib, ub.ld};
  const int64_t q_first = (b - ub.reduce_block) * ZK_K1_THREADS * ZK_K1_QUADS;
  const Partial pt = reduce_block(rows, n, ub.shard, q_first, inv32, (float*)ub.grad);
  if (threadIdx.x == 0) partials[b] = pt;
}

// The deferred form above N = 8 (see reduce_block_deferred): workgroup b
// takes the ZK_K1_DEFER consecutive workgroups bK .. bK + K - 1 of the
// one-chunk numbering that zero_units_prepare recorded, so its chunks may lie
// in different units.  Each chunk's g quad stays in registers until every
// chunk is summed; the chunk's g address and its count of whole-quad threads
// are workgroup-uniform.  Each unit's ragged tail is summed and stored where
// it is met.  The values and the norm are those of the one-chunk kernel; the
// partials are fewer (one per workgroup).
static_assert(ZK_K1_QUADS == 1, "a chunk is one one-quad workgroup");
__global__ __launch_bounds__(ZK_K1_THREADS) void k1u_reduce_check_deferred(
    const zero_unit_buffers_t* __restrict__ units, int32_t n_units, int64_t chunks, int32_t n,
    float inv32, Partial* __restrict__ partials, uint32_t* __restrict__ ticket, int64_t b0) {
  constexpr int K = ZK_K1_DEFER;
  const int64_t b = b0 + blockIdx.x;
  if (b == 0 && threadIdx.x == 0) *ticket = 0u;
  uint64_t qlo = 0, qhi = 0;
  uint32_t bad = 0;
  f32x4 g[K];
  float* gbase[K];  // the chunk's first quad in its unit's g
  int32_t whole[K];  // threads of the chunk that own a whole quad
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int64_t c = b * K + k;
    whole[k] = 0;
    gbase[k] = nullptr;
    if (c < chunks) {
      const int32_t u = find_unit(n_units, c, [&](int32_t i) { return units[i].reduce_block; });
      const UnitBuffersGlobal& ub = ((const UnitBuffersGlobal*)units)[u];
      const StridedRows rows{(const uint16_t*)ub.contrib, ub.ld};
      const int64_t q_first = (c - ub.reduce_block) * ZK_K1_THREADS;
      const int64_t full = ub.shard >> 2, rel = full - q_first;
      whole[k] = rel <= 0 ? 0 : rel >= ZK_K1_THREADS ? ZK_K1_THREADS : (int32_t)rel;
      gbase[k] = (float*)ub.grad + q_first * 4;
      if ((int32_t)threadIdx.x < whole[k]) {
        float acc[4];
        sum_rows_quad(rows, n, (q_first + threadIdx.x) * 4, acc);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          g[k][e] = acc[e] * inv32;
          uint64_t lo, hi;
          sq_units(acc[e], lo, hi, bad);
          add128(qlo, qhi, lo, hi);
        }
      }
      // the thread that would own quad `full` takes the unit's ragged tail
      if (rel >= 0 && rel < ZK_K1_THREADS && (int64_t)threadIdx.x == rel)
        reduce_tail(rows, n, full * 4, ub.shard, inv32, (float*)ub.grad, qlo, qhi, bad);
    }
  }
#pragma unroll
  for (int k = 0; k < K; ++k)
    if ((int32_t)threadIdx.x < whole[k])
      vstore<ZK_K1_NT_STORE>(g[k], (f32x4*)(gbase[k] + threadIdx.x * 4));
  block_reduce<ZK_K1_THREADS>(qlo, qhi, bad);
  if (threadIdx.x == 0) partials[b] = make_partial(qlo, qhi, bad);
}

__global__ __launch_bounds__(ZK_K2_THREADS) void k2u_adam(
    const zero_unit_buffers_t* __restrict__ units, int32_t n_units, AdamScalars sc,
    const zero_step_result_t* __restrict__ res, int64_t b0) {
  if (res->skip) return;
  const float c = res->clip_coef;
  const int64_t b = b0 + blockIdx.x;
  const int32_t u = find_unit(n_units, b, [&](int32_t i) { return units[i].adam_block; });
  const UnitBuffersGlobal& ub = ((const UnitBuffersGlobal*)units)[u];
#pragma unroll
  for (int k = 0; k < ZK_K2_QUADS; ++k) {
    const int64_t qd = ((b - ub.adam_block) * ZK_K2_QUADS + k) * ZK_K2_THREADS + threadIdx.x;
    adam_quad((const float*)ub.grad, (float*)ub.master, (float*)ub.m, (float*)ub.v,
              (uint16_t*)ub.param16, ub.shard, qd, c, sc);
  }
}

// Single pass over all units (steps without clipping): `units` gives the
// rows and the current state, `outs` (same shards, same workgroup columns)
// the set that receives the new state and slot.
static_assert(ZK_K1_QUADS == 1, "the unit single pass reuses the reduce's one-quad workgroups");
__global__ __launch_bounds__(ZK_K1_THREADS) void k12u_reduce_adam(
    const zero_unit_buffers_t* __restrict__ units, const zero_unit_buffers_t* __restrict__ outs,
    int32_t n_units, int32_t n, float inv32, AdamScalars sc, Partial* __restrict__ partials,
    uint32_t* __restrict__ ticket, int64_t b0) {
  const int64_t b = b0 + blockIdx.x;
  if (b == 0 && threadIdx.x == 0) *ticket = 0u;
  const int32_t u = find_unit(n_units, b, [&](int32_t i) { return units[i].reduce_block; });
  const UnitBuffersGlobal& ub = ((const UnitBuffersGlobal*)units)[u];
  const UnitBuffersGlobal& ob = ((const UnitBuffersGlobal*)outs)[u];
  const StridedRows rows{(const uint16_t*)ub.contrib, ub.ld};
  const StatePair st{(const float*)ub.master, (const float*)ub.m, (const float*)ub.v,
                     (float*)ob.master,       (float*)ob.m,       (float*)ob.v,
                     (uint16_t*)ob.param16};
  uint64_t qlo = 0, qhi = 0;
  uint32_t bad = 0;
  const int64_t qd = (b - ub.reduce_block) * ZK_K1_THREADS + threadIdx.x;
  reduce_adam_quad(rows, n, ub.shard, qd, inv32, st, sc, qlo, qhi, bad);
  block_reduce<ZK_K1_THREADS>(qlo, qhi, bad);
  if (threadIdx.x == 0) partials[b] = make_partial(qlo, qhi, bad);
}

// Slot restore over all units (see the flat k_slot_restore): a no-op unless
// the step was skipped; then every unit's slot is recast from its master.
__global__ __launch_bounds__(kThreads) void k_units_slot_restore(
    const zero_unit_buffers_t* __restrict__ units, int32_t n_units,
    const zero_step_result_t* __restrict__ res) {
  if (!res->skip) return;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int32_t u = 0; u < n_units; ++u) {
    const UnitBuffersGlobal& ub = ((const UnitBuffersGlobal*)units)[u];
    const float* master = (const float*)ub.master;
    uint16_t* slot = (uint16_t*)ub.param16;
    for (int64_t j = (int64_t)blockIdx.x * kThreads + threadIdx.x; j < ub.shard; j += stride)
      slot[j] = (uint16_t)f2h(master[j]);
  }
}

// The unit table, written by value: kTableChunk entries travel in the kernel
// arguments (48 * 80 B fits the 4 KiB argument segment) and one workgroup
// stores them as 8-byte words.
constexpr int kTableChunk = 48;
struct TableChunk {
  zero_unit_buffers_t u[kTableChunk];
};
constexpr int kTableWords = (int)(sizeof(zero_unit_buffers_t) / 8);
static_assert(sizeof(zero_unit_buffers_t) % 8 == 0, "whole 8-byte words");

__global__ __launch_bounds__(kThreads) void k_store_table(TableChunk c, int32_t n,
                                                           zero_unit_buffers_t* __restrict__ dst) {
  const uint64_t* src = (const uint64_t*)&c.u[0];
  uint64_t* out = (uint64_t*)dst;
  for (int i = threadIdx.x; i < n * kTableWords; i += kThreads) out[i] = src[i];
}

}  // namespace

int launch_store_table(const zero_unit_buffers_t* units_host, int32_t n_units,
                       zero_unit_buffers_t* units_dev, hipStream_t stream) {
  for (int32_t u0 = 0; u0 < n_units; u0 += kTableChunk) {
    const int32_t n = n_units - u0 < kTableChunk ? n_units - u0 : kTableChunk;
    TableChunk c;
    for (int32_t i = 0; i < n; ++i) c.u[i] = units_host[u0 + i];
    for (int32_t i = n; i < kTableChunk; ++i) c.u[i] = zero_unit_buffers_t{};
    hipLaunchKernelGGL(k_store_table, dim3(1), dim3(kThreads), 0, stream, c, n, units_dev + u0);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
  }
  return (int)hipSuccess;
}

int launch_units_slot_restore(const zero_unit_buffers_t* units_dev, int32_t n_units,
                              int64_t max_shard, const zero_step_result_t* res,
                              hipStream_t stream) {
  int64_t blocks = (max_shard + kThreads - 1) / kThreads;
  if (blocks > kRestoreBlocks) blocks = kRestoreBlocks;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(k_units_slot_restore, dim3((uint32_t)blocks), dim3(kThreads), 0, stream,
                     units_dev, n_units, res);
  return (int)hipGetLastError();
}

int launch_units_reduce_adam_1pass(const zero_unit_buffers_t* units_dev,
                                   const zero_unit_buffers_t* outs_dev, int32_t n_units,
                                   int64_t blocks, int n, float inv32, const AdamScalars& sc,
                                   void* workspace, hipStream_t stream) {
  Partial* partials = (Partial*)workspace_partials(workspace);
  uint32_t* ticket = (uint32_t*)workspace;
  return launch_segments(blocks, k12_seg_elems(n) / (4 * ZK_K1_THREADS),
                         [&](int64_t b0, int64_t nb) {
                           hipLaunchKernelGGL(k12u_reduce_adam, dim3((uint32_t)nb),
                                              dim3(ZK_K1_THREADS), ZK_K12U_LDS, stream, units_dev,
                                              outs_dev, n_units, n, inv32, sc, partials, ticket,
                                              b0);
                         });
}

int launch_units_reduce(const zero_unit_buffers_t* units_dev, int32_t n_units, int64_t blocks,
                        int n, float inv32, void* workspace, int64_t* n_partials,
                        hipStream_t stream) {
  Partial* partials = (Partial*)workspace_partials(workspace);
  uint32_t* ticket = (uint32_t*)workspace;
  if (n > 8) {
    const int64_t wg = (blocks + ZK_K1_DEFER - 1) / ZK_K1_DEFER;
    *n_partials = wg;
    return launch_segments(wg, ZK_K1_DEFER_SEG_ELEMS / (4 * ZK_K1_THREADS * ZK_K1_DEFER),
                           [&](int64_t b0, int64_t nb) {
                             hipLaunchKernelGGL(k1u_reduce_check_deferred, dim3((uint32_t)nb),
                                                dim3(ZK_K1_THREADS), ZK_K1_DEFER_LDS, stream,
                                                units_dev, n_units, blocks, n, inv32, partials,
                                                ticket, b0);
                           });
  }
  *n_partials = blocks;
  return launch_segments(blocks, ZK_K1_SEG_ELEMS / (4 * ZK_K1_THREADS * ZK_K1_QUADS),
                         [&](int64_t b0, int64_t nb) {
                           hipLaunchKernelGGL(k1u_reduce_check, dim3((uint32_t)nb),
                                              dim3(ZK_K1_THREADS), k1_lds(n), stream, units_dev,
                                              n_units, n, inv32, partials, ticket, b0);
                         });
}

int launch_units_adam(const zero_unit_buffers_t* units_dev, int32_t n_units, int64_t blocks,
                      const AdamScalars& sc, const zero_step_result_t* res, hipStream_t stream) {
  return launch_segments(blocks, ZK_K2_SEG_ELEMS / (4 * ZK_K2_THREADS * ZK_K2_QUADS),
                         [&](int64_t b0, int64_t nb) {
                           hipLaunchKernelGGL(k2u_adam, dim3((uint32_t)nb), dim3(ZK_K2_THREADS),
                                              ZK_K2_LDS, stream, units_dev, n_units, sc, res, b0);
                         });
}

}  // namespace zk
