// Device kernels of the ZeRO shard step for CDNA4 (gfx950).
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
//
// K1 and K2 stream every element once and use one-shot grids: each thread
// owns a fixed piece of the shard (no grid-stride loop), so workgroups are
// dispatched in address order and retire as they finish; on MI355X this
// streams measurably faster than persistent grids.  Loads and stores are 16
// bytes per lane, so a 64-wide wave moves 1 KiB per instruction.  Nothing here
// is a dense contraction, so no matrix cores are used; HBM bandwidth bounds
// K1 and K2.
//
// Floating point: every fp32 operation is rounded on its own (contraction is
// off here and in the build flags); division and square root are correctly
// rounded; denormals are kept.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "zero_internal.h"

#pragma clang fp contract(off)

// Launch shape and cache hints (compile-time; measured on MI355X).
#ifndef ZK_K1_QUADS
#define ZK_K1_QUADS 1  // 4-element quads per K1 thread
#endif
#ifndef ZK_K2_QUADS
#define ZK_K2_QUADS 1  // 4-element quads per K2 thread
#endif
#ifndef ZK_K1_THREADS
#define ZK_K1_THREADS 512  // threads per K1 workgroup (a multiple of 64)
#endif
#ifndef ZK_K2_THREADS
#define ZK_K2_THREADS 64  // threads per K2 workgroup
#endif
#ifndef ZK_K1_NT_LOAD
#define ZK_K1_NT_LOAD 1
#endif
#ifndef ZK_K1_NT_STORE
#define ZK_K1_NT_STORE 1
#endif
#ifndef ZK_K2_NT_LOAD
#define ZK_K2_NT_LOAD 1
#endif
#ifndef ZK_K2_NT_STORE
#define ZK_K2_NT_STORE 1
#endif

namespace zk {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct ContribTable {
  const uint16_t* p[ZERO_MAX_RANKS];
};

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// A 128-bit partial sum; bit 63 of hi carries the overflow flag.
struct Partial {
  uint64_t lo, hi;
};
static_assert(sizeof(Partial) == kPartialBytes, "partial layout");

constexpr int kRankBatch = 8;  // contribution rows loaded before they are summed

template <bool NT, typename T>
__device__ __forceinline__ T vload(const T* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

template <bool NT, typename T>
__device__ __forceinline__ void vstore(T v, T* p) {
  if constexpr (NT) __builtin_nontemporal_store(v, p);
  else *p = v;
}

__device__ __forceinline__ float h2f(uint32_t bits) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

__device__ __forceinline__ uint32_t f2h(float x) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x);
}

// acc^2 in units of 2^-48 as a 128-bit integer (lo, hi); sets bad for a
// non-finite acc, which contributes nothing.  With m the 24-bit significand
// and e the biased exponent, acc^2 = m^2 * 2^(2e - 300) = m^2 * 2^(2e - 252)
// units.  Sums of fp16 values are multiples of 2^-24, so a right shift here
// only drops zero bits.
__device__ __forceinline__ void sq_units(float acc, uint64_t& lo, uint64_t& hi, uint32_t& bad) {
  const uint32_t bits = __float_as_uint(acc) & 0x7FFFFFFFu;
  const uint32_t e = bits >> 23;
  const bool fin = e != 0xFFu;
  bad |= fin ? 0u : 1u;
  uint32_t mant = (bits & 0x7FFFFFu) | (e ? 0x800000u : 0u);
  mant = fin ? mant : 0u;
  const int sh = 2 * (int)(e ? e : 1u) - 252;
  const uint64_t sq = (uint64_t)mant * (uint64_t)mant;  // < 2^48
  const uint32_t s = (uint32_t)(sh < 0 ? -sh : sh);
  const uint64_t l_lo = s < 64 ? (sq << (s & 63)) : 0ull;
  const uint64_t l_hi = s == 0 ? 0ull
                        : s < 64 ? (sq >> ((64 - s) & 63))
                        : s < 128 ? (sq << ((s - 64) & 63))
                        : 0ull;
  const uint64_t r_lo = s < 64 ? (sq >> (s & 63)) : 0ull;
  lo = sh >= 0 ? l_lo : r_lo;
  hi = sh >= 0 ? l_hi : 0ull;
}

__device__ __forceinline__ void add128(uint64_t& alo, uint64_t& ahi, uint64_t blo, uint64_t bhi) {
  alo += blo;
  ahi += bhi + (alo < blo ? 1ull : 0ull);
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t x, int mask) {
  return (uint64_t)__shfl_xor((long long)x, mask);
}

__device__ __forceinline__ uint64_t shfl_down_u64(uint64_t x, unsigned int delta) {
  const uint32_t lo = (uint32_t)__shfl_down((int)(uint32_t)x, delta);
  const uint32_t hi = (uint32_t)__shfl_down((int)(uint32_t)(x >> 32), delta);
  return ((uint64_t)hi << 32) | lo;
}

// Sum (lo, hi, bad) over a workgroup of T threads; valid in thread 0.
template <int T>
__device__ void block_reduce(uint64_t& lo, uint64_t& hi, uint32_t& bad) {
  static_assert(T % 64 == 0, "whole waves");
  for (int off = 32; off > 0; off >>= 1) {
    add128(lo, hi, shfl_xor_u64(lo, off), shfl_xor_u64(hi, off));
    bad |= (uint32_t)__shfl_xor((int)bad, off);
  }
  if constexpr (T == 64) return;
  __shared__ uint64_t s_lo[T / 64], s_hi[T / 64];
  __shared__ uint32_t s_bad[T / 64];
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    s_lo[wave] = lo;
    s_hi[wave] = hi;
    s_bad[wave] = bad;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < T / 64; ++w) {
      add128(lo, hi, s_lo[w], s_hi[w]);
      bad |= s_bad[w];
    }
  }
}

// Round a nonnegative integer c*2^128 + hi*2^64 + lo (c in {0,1}) to the
// nearest fp64, ties to even.
__device__ double u129_to_f64(uint32_t c, uint64_t hi, uint64_t lo) {
  if (!c && !hi) return (double)lo;  // uint64 -> fp64 rounds once
  uint64_t top, scale_exp;
  bool sticky;
  if (c) {
    top = 0x8000000000000000ull | (hi >> 1);
    sticky = (hi & 1ull) || lo;
    scale_exp = 65;
  } else {
    const int lz = __clzll((long long)hi);
    top = lz ? ((hi << lz) | (lo >> (64 - lz))) : hi;
    sticky = (lz ? (lo << lz) : lo) != 0;
    scale_exp = 64 - lz;
  }
  uint64_t keep = top >> 11;
  const uint64_t rb = top & 0x7FFull;
  if (rb > 0x400ull || (rb == 0x400ull && (sticky || (keep & 1ull)))) keep += 1;
  return __builtin_ldexp((double)keep, (int)scale_exp + 11);
}

__device__ void finalize_into(uint64_t qlo, uint64_t qhi, uint32_t bad, const FinalizeArgs& fa,
                              zero_step_result_t* res) {
  // (qhi:qlo) + (other_hi:other_lo) as a 129-bit value (carry:thi:tlo)
  const uint64_t tlo = qlo + fa.other_lo;
  const uint64_t c0 = tlo < qlo ? 1ull : 0ull;
  const uint64_t t1 = qhi + fa.other_hi;
  const uint64_t thi = t1 + c0;
  const uint32_t carry = ((t1 < qhi) || (thi < t1)) ? 1u : 0u;
  const double own = ((u129_to_f64(0, qhi, qlo) * 0x1p-48) * fa.inv64) * fa.inv64;
  const double tot = ((u129_to_f64(carry, thi, tlo) * 0x1p-48) * fa.inv64) * fa.inv64 + fa.other_sq;
  const double norm = __builtin_sqrt(tot);
  double coef = 1.0;
  if (fa.max_norm > 0.0) {
    const double c = fa.max_norm / (norm + 1e-6);
    coef = (c < 1.0) ? c : 1.0;
  }
  res->own_q_lo = qlo;
  res->own_q_hi = qhi;
  res->own_sq = own;
  res->total_sq = tot;
  res->norm = norm;
  res->clip_coef = (float)coef;
  res->overflow = bad ? 1 : 0;
  res->skip = (bad || fa.other_overflow || carry) ? 1 : 0;
  res->reserved = 0;
}

// ---------------------------------------------------------------------------
// K1: reduce, unscale, overflow flag, exact squared norm, one partial per
// workgroup.  Thread t of workgroup b owns quads (b*Q + u)*T + t, u < Q: each
// loads 8 bytes from every row, so a wave's row load covers 512 contiguous
// bytes and its gradient store 1 KiB.
__device__ __forceinline__ void reduce_quad(const ContribTable& ct, int32_t n, int64_t qd,
                                            float inv32, float* __restrict__ grad,
                                            uint64_t& qlo, uint64_t& qhi, uint32_t& bad) {
  const int64_t off = qd * 4;
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int r0 = 0; r0 < n; r0 += kRankBatch) {
    u32x2 d[kRankBatch];
#pragma unroll
    for (int b = 0; b < kRankBatch; ++b)
      if (r0 + b < n) d[b] = vload<ZK_K1_NT_LOAD>((const u32x2*)(ct.p[r0 + b] + off));
#pragma unroll
    for (int b = 0; b < kRankBatch; ++b) {
      if (r0 + b < n) {
#pragma unroll
        for (int w = 0; w < 2; ++w) {
          acc[2 * w] = acc[2 * w] + h2f(d[b][w] & 0xFFFFu);
          acc[2 * w + 1] = acc[2 * w + 1] + h2f(d[b][w] >> 16);
        }
      }
    }
  }
  f32x4 g;
#pragma unroll
  for (int e = 0; e < 4; ++e) g[e] = acc[e] * inv32;
  vstore<ZK_K1_NT_STORE>(g, (f32x4*)(grad + off));
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    uint64_t lo, hi;
    sq_units(acc[e], lo, hi, bad);
    add128(qlo, qhi, lo, hi);
  }
}

__global__ __launch_bounds__(ZK_K1_THREADS) void k1_reduce_check(ContribTable ct, int32_t n,
                                                            int64_t shard, float inv32,
                                                            float* __restrict__ grad,
                                                            Partial* __restrict__ partials) {
  uint64_t qlo = 0, qhi = 0;
  uint32_t bad = 0;
  const int64_t full = shard >> 2;
#pragma unroll
  for (int u = 0; u < ZK_K1_QUADS; ++u) {
    const int64_t qd = ((int64_t)blockIdx.x * ZK_K1_QUADS + u) * ZK_K1_THREADS + threadIdx.x;
    if (qd < full) reduce_quad(ct, n, qd, inv32, grad, qlo, qhi, bad);
  }
  // the thread that would own quad `full` takes the ragged tail
  const int64_t tail_from = full * 4;
  const int64_t per = (int64_t)ZK_K1_THREADS * ZK_K1_QUADS;
  const bool tail_owner = (int64_t)blockIdx.x == full / per &&
                          (int64_t)threadIdx.x == (full % per) % ZK_K1_THREADS;
  if (tail_owner) {
    // ragged tail: the last shard % 4 elements
    for (int64_t j = tail_from; j < shard; ++j) {
      float a = 0.0f;
      for (int r = 0; r < n; ++r) a = a + h2f(ct.p[r][j]);
      grad[j] = a * inv32;
      uint64_t lo, hi;
      sq_units(a, lo, hi, bad);
      add128(qlo, qhi, lo, hi);
    }
  }
  block_reduce<ZK_K1_THREADS>(qlo, qhi, bad);
  if (threadIdx.x == 0) partials[blockIdx.x] = Partial{qlo, qhi | ((uint64_t)(bad ? 1u : 0u) << 63)};
}

// ---------------------------------------------------------------------------
// KF: sum the K1 partials, then the last workgroup finalizes.  A block
// partial is below 2^105, so bit 63 of its high word is free for the flag.
__global__ __launch_bounds__(kThreads) void kf_reduce_finalize(
    const Partial* __restrict__ partials, int64_t n_partials, Partial* __restrict__ level2,
    uint32_t* __restrict__ ticket, FinalizeArgs fa, zero_step_result_t* __restrict__ res) {
  uint64_t lo = 0, hi = 0;
  uint32_t bad = 0;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n_partials;
       i += (int64_t)gridDim.x * kThreads) {
    const Partial pt = partials[i];
    bad |= (uint32_t)(pt.hi >> 63);
    add128(lo, hi, pt.lo, pt.hi & 0x7FFFFFFFFFFFFFFFull);
  }
  block_reduce<kThreads>(lo, hi, bad);
  __shared__ uint32_t s_last;
  if (threadIdx.x == 0) {
    level2[blockIdx.x] = Partial{lo, hi | ((uint64_t)(bad ? 1u : 0u) << 63)};
    __threadfence();
    const uint32_t prev = atomicAdd(ticket, 1u);
    s_last = (prev == gridDim.x - 1) ? 1u : 0u;
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  lo = hi = 0;
  bad = 0;
  for (uint32_t i = threadIdx.x; i < gridDim.x; i += kThreads) {
    const Partial pt = level2[i];
    bad |= (uint32_t)(pt.hi >> 63);
    add128(lo, hi, pt.lo, pt.hi & 0x7FFFFFFFFFFFFFFFull);
  }
  block_reduce<kThreads>(lo, hi, bad);
  if (threadIdx.x == 0) {
    finalize_into(lo, hi, bad, fa, res);
    *ticket = 0u;  // ready for the next call
  }
}

__global__ void k_finalize(FinalizeArgs fa, zero_step_result_t* res) {
  if (threadIdx.x == 0 && blockIdx.x == 0)
    finalize_into(res->own_q_lo, res->own_q_hi, (uint32_t)res->overflow, fa, res);
}

// ---------------------------------------------------------------------------
// K2: AdamW on the shard and the fp16 cast into the slot.  Thread t of
// workgroup b owns quads (4 elements) (b*Q + u)*T + t, u < Q, so every
// fp32 load and store instruction of a wave covers 1 KiB and every slot store
// 512 bytes.
__device__ __forceinline__ void adam1(float g, float c, const AdamScalars& sc, float& p, float& m,
                                      float& v) {
  const float gc = g * c;
  m = sc.b1 * m + sc.omb1 * gc;
  v = sc.b2 * v + sc.omb2 * (gc * gc);
  const float den = __builtin_sqrtf(v) / sc.sqrt_bc2 + sc.eps;
  const float u = (m / den) * sc.step_size;
  p = p * sc.decay - u;
}

__global__ __launch_bounds__(ZK_K2_THREADS) void k2_adam(
    const float* __restrict__ grad, float* __restrict__ master, float* __restrict__ mom,
    float* __restrict__ var, uint16_t* __restrict__ slot, int64_t shard, AdamScalars sc,
    const zero_step_result_t* __restrict__ res) {
  if (res->skip) return;
  const float c = res->clip_coef;
  // slot misalignment in elements relative to 8-byte words (the slot may sit
  // at any element offset of the flat buffer)
  const uint32_t me = (uint32_t)(((uintptr_t)slot >> 1) & 3u);
  const uint32_t lane = threadIdx.x & 63u;
  const int64_t full = shard >> 2;
  f32x4 g[ZK_K2_QUADS], p[ZK_K2_QUADS], m[ZK_K2_QUADS], v[ZK_K2_QUADS];
  int64_t qd[ZK_K2_QUADS];
#pragma unroll
  for (int u = 0; u < ZK_K2_QUADS; ++u) {
    qd[u] = ((int64_t)blockIdx.x * ZK_K2_QUADS + u) * ZK_K2_THREADS + threadIdx.x;
    if (qd[u] < full) {
      const int64_t off = qd[u] * 4;
      g[u] = vload<ZK_K2_NT_LOAD>((const f32x4*)(grad + off));
      p[u] = vload<ZK_K2_NT_LOAD>((const f32x4*)(master + off));
      m[u] = vload<ZK_K2_NT_LOAD>((const f32x4*)(mom + off));
      v[u] = vload<ZK_K2_NT_LOAD>((const f32x4*)(var + off));
    }
  }
#pragma unroll
  for (int u = 0; u < ZK_K2_QUADS; ++u) {
    const bool valid = qd[u] < full;
    const int64_t off = qd[u] * 4;
    uint64_t h = 0;  // the quad's four fp16 results, element e in bits 16e..16e+15
    if (valid) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float pp = p[u][e], mm = m[u][e], vv = v[u][e];
        adam1(g[u][e], c, sc, pp, mm, vv);
        p[u][e] = pp;
        m[u][e] = mm;
        v[u][e] = vv;
        h |= (uint64_t)f2h(pp) << (16 * e);
      }
      vstore<ZK_K2_NT_STORE>(p[u], (f32x4*)(master + off));
      vstore<ZK_K2_NT_STORE>(m[u], (f32x4*)(mom + off));
      vstore<ZK_K2_NT_STORE>(v[u], (f32x4*)(var + off));
    }
    if (me == 0) {
      if (valid) vstore<ZK_K2_NT_STORE>(h, (uint64_t*)(slot + off));
    } else {
      // Realign through the neighbour lane: lane i writes the aligned 8-byte
      // word holding its last `me` results and lane i+1's first 4 - me.
      // The pieces at a wave's edges or at the shard's end go out as 2-byte
      // stores.  Every lane of the wave takes part in the shuffle.
      const uint64_t hn = shfl_down_u64(h, 1);
      const bool right = lane < 63u && qd[u] + 1 < full;
      if (valid) {
        if (lane == 0u) {
          for (uint32_t e = 0; e < 4u - me; ++e) slot[off + e] = (uint16_t)(h >> (16 * e));
        }
        if (right) {
          vstore<ZK_K2_NT_STORE>((h >> (16 * (4u - me))) | (hn << (16 * me)),
                                 (uint64_t*)(slot + off + 4 - me));
        } else {
          for (uint32_t e = 4u - me; e < 4u; ++e) slot[off + e] = (uint16_t)(h >> (16 * e));
        }
      }
    }
    if (qd[u] == full) {
      for (int64_t j = full * 4; j < shard; ++j) {
        float pp = master[j], mm = mom[j], vv = var[j];
        adam1(grad[j], c, sc, pp, mm, vv);
        master[j] = pp;
        mom[j] = mm;
        var[j] = vv;
        slot[j] = (uint16_t)f2h(pp);
      }
    }
  }
}

}  // namespace

int64_t k1_blocks(int64_t shard) {
  const int64_t units = (shard + 3) >> 2;  // quads, the ragged one included
  const int64_t per = (int64_t)ZK_K1_THREADS * ZK_K1_QUADS;
  const int64_t b = (units + per - 1) / per;
  return b < 1 ? 1 : b;
}

size_t workspace_bytes(int64_t shard) {
  return kTicketBytes + (size_t)kFinBlocks * sizeof(Partial) +
         (size_t)k1_blocks(shard) * sizeof(Partial);
}

int launch_reduce_check(const uint16_t* const* contrib, int n, int64_t shard, float inv32,
                        float* grad, void* workspace, const FinalizeArgs& fa,
                        zero_step_result_t* res, hipStream_t stream) {
  ContribTable ct;
  for (int r = 0; r < ZERO_MAX_RANKS; ++r) ct.p[r] = r < n ? contrib[r] : nullptr;
  uint32_t* ticket = (uint32_t*)workspace;
  Partial* level2 = (Partial*)((char*)workspace + kTicketBytes);
  Partial* partials = level2 + kFinBlocks;
  const int64_t blocks = k1_blocks(shard);
  hipLaunchKernelGGL(k1_reduce_check, dim3((uint32_t)blocks), dim3(ZK_K1_THREADS), 0, stream, ct, n,
                     shard, inv32, grad, partials);
  int e = (int)hipGetLastError();
  if (e != hipSuccess) return e;
  int64_t fb = (blocks + kThreads * 4 - 1) / (kThreads * 4);
  if (fb > kFinBlocks) fb = kFinBlocks;
  if (fb < 1) fb = 1;
  hipLaunchKernelGGL(kf_reduce_finalize, dim3((uint32_t)fb), dim3(kThreads), 0, stream, partials,
                     blocks, level2, ticket, fa, res);
  return (int)hipGetLastError();
}

int launch_finalize(const FinalizeArgs& fa, zero_step_result_t* res, hipStream_t stream) {
  hipLaunchKernelGGL(k_finalize, dim3(1), dim3(64), 0, stream, fa, res);
  return (int)hipGetLastError();
}

int launch_adam(const float* grad, float* master, float* m, float* v, uint16_t* slot,
                int64_t shard, const AdamScalars& sc, const zero_step_result_t* res,
                hipStream_t stream) {
  const int64_t quads = (shard + 3) >> 2;
  const int64_t per = (int64_t)ZK_K2_THREADS * ZK_K2_QUADS;
  int64_t blocks = (quads + per - 1) / per;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(k2_adam, dim3((uint32_t)blocks), dim3(ZK_K2_THREADS), 0, stream, grad, master, m,
                     v, slot, shard, sc, res);
  return (int)hipGetLastError();
}

}  // namespace zk
