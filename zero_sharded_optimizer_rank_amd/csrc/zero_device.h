// Device building blocks shared by the flat-shard kernels (zero_kernels.hip)
// and the multi-unit kernels (zero_units.hip): vector types, cache-hinted
// 16-byte access, fp16 conversion, the exact squared-norm arithmetic, the
// 128-bit workgroup reduction, the fp64 finalize, and the per-quad bodies of
// the reduce and of the Adam update.
//
// Floating point: every fp32 operation is rounded on its own (contraction is
// off here and in the build flags); division and square root are correctly
// rounded; denormals are kept.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "zero_internal.h"

#pragma clang fp contract(off)

// Launch shape and cache hints (compile-time; measured on MI355X).
#ifndef ZK_K1_QUADS
#define ZK_K1_QUADS 1  // 4-element quads per reduce thread
#endif
#ifndef ZK_K2_QUADS
#define ZK_K2_QUADS 1  // 4-element quads per Adam thread
#endif
#ifndef ZK_K1_THREADS
#define ZK_K1_THREADS 128  // threads per reduce workgroup (a multiple of 64)
#endif
#ifndef ZK_K2_THREADS
#define ZK_K2_THREADS 64  // threads per Adam workgroup
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
#ifndef ZK_K12_THREADS
#define ZK_K12_THREADS 64  // threads per single-pass workgroup (a multiple of 64)
#endif
#ifndef ZK_K12_BATCH
#define ZK_K12_BATCH 4  // contribution rows the single pass loads before summing
#endif
#ifndef ZK_K12_NT_LOAD
#define ZK_K12_NT_LOAD 1
#endif
#ifndef ZK_K12_NT_STORE
#define ZK_K12_NT_STORE 1
#endif
// LDS the Adam kernels reserve and never touch, to cap how many of their
// one-wave workgroups a CU holds: 160 KiB / 14848 B = 11.  With the default
// 32 waves per CU the eight streams of the update thrash the memory system;
// measured on the Llama-3-8B shard: 32 waves 5.90 TB/s, 16 waves 6.35,
// 12 waves 6.44, 11 waves 6.53, 10 waves 6.43, 8 waves 6.21.  Other shapes,
// interleaved with this one on the same shard (6.55-6.57 TB/s): two quads per
// thread at 6 / 8 / 11 / 14 workgroups per CU 5.64 / 6.42 / 6.07 / 5.77;
// two-wave workgroups at 5 / 6 / 7 per CU 5.94 / 6.27 / 6.12; one quad at
// 9 / 10 / 12 per CU 6.18 / 6.45 / 6.48.
#ifndef ZK_K2_LDS
#define ZK_K2_LDS 14848
#endif
// The reduce kernel is capped the same way, by N: with 128-thread (two-wave)
// workgroups, 16 per CU for N <= 8 and 10 per CU beyond (10240 and 16384 B
// of reserved LDS).  Measured reduce rates, cap 10 / 12 / 14 / 16 / none:
// N = 8:  5.65 / 6.24 / 6.51 / 6.51 / 6.05 TB/s;  N = 16: 6.21 / 6.39 /
// 6.21 / 6.20 / 6.09;  N = 32: 6.20 / 6.22 / 6.03 / 6.01 / 5.93;  N = 64:
// 6.26 / 6.20 / 5.99 / 6.00 / 5.94 (the earlier 512-thread, 8-row-batch
// form: 6.23, 5.66, 5.56, 5.77).  A finer interleaved sweep at N = 64, caps
// 9 / 10 / 11 / 12 / 13 / 14 / 16: flat 7.5B shard 6.12 / 6.26 / 6.27 / 6.23
// / 6.14 / 5.99 / 5.99 TB/s, GPT-2 shard 6.09 / 6.17 / 6.15 / 6.09 / 6.05 /
// 5.94 / 5.92; at N = 8, caps 13 / 14 / 16 / 18 / 20: 6.37 / 6.50 / 6.50 /
// 6.05 / 6.05.
#ifndef ZK_K1_LDS_SMALL_N
#define ZK_K1_LDS_SMALL_N 10240
#endif
#ifndef ZK_K1_LDS
#define ZK_K1_LDS 16384
#endif
// Above N = 8 the reduce defers its gradient stores: each workgroup sums
// ZK_K1_DEFER consecutive 512-element chunks one after the other, holding
// the chunks' g quads in registers, and stores them all at the end.  With 64
// rows the rows are 97% of the bytes, and the small g stream spread evenly
// among them slows the reads far more than its own size: on the flat 7.5B
// shard's geometry, reading the 64 rows alone took 2.12 ms, with the g
// stores after every chunk 2.46-2.48 ms, with 8 or 16 chunks' stores
// deferred 2.35 and 2.30 ms (no-arithmetic probes, 8 workgroups per CU); 8
// chunks per workgroup without the deferral ran at 2.71 ms.  In one launch
// over the whole shard the deferral only paid up to about 2^27 elements (S =
// 24 M 0.480 against 0.524 ms, 117 M 2.415 / 2.466, but 250 M 5.63 / 5.38,
// 1.08 G 24.4 / 23.3); issued in launches of ZK_K1_DEFER_SEG_ELEMS elements
// (see launch_segments) it pays at every length.  At N = 8 it did not pay
// (3.17-3.42 against 3.08-3.10 ms on Llama-3-8B, deferring 2, 4 or 8 chunks).
#ifndef ZK_K1_DEFER
#define ZK_K1_DEFER 8
#endif
#ifndef ZK_K1_DEFER_LDS
#define ZK_K1_DEFER_LDS 18176
#endif
// Elements per launch of the streaming kernels.  A one-shot grid streams
// more slowly the longer it runs; the same workgroups issued as several
// launches back to back on the stream (launch_segments) run faster.  First
// measured through windows of one shard (interleaved, same buffers): the
// deferred reduce at N = 64 in launches of 2^25 elements against one
// launch: Llama-2-70B 22.02 against 23.27 ms (one-chunk form), S = 250 M
// 4.96 / 5.30, the flat 7.5B shard 2.26 / 2.41 (2^24: 2.25, 2^26: 2.31);
// built into the kernels, 2^26 / 2^25 / 2^24 / 2^23 per launch took 22.39 /
// 21.90 / 21.68 / 21.64 ms on Llama-2-70B and 2.30 / 2.25 / 2.22 / 2.22 on
// the flat 7.5B shard.  The one-chunk reduce at N = 8 in launches of 2^28:
// 3.08 against 3.16 ms (2^27: 3.12, 2^26: 3.18; shorter ones lose to the
// launch gaps); the update in launches of 2^26-2^28: 4.55 against 4.60 ms.
// A plain copy gains nothing from it (6.73 against 6.71 TB/s in two
// launches, less in more).
#ifndef ZK_K1_SEG_ELEMS
#define ZK_K1_SEG_ELEMS ((int64_t)1 << 28)
#endif
#ifndef ZK_K1_DEFER_SEG_ELEMS
#define ZK_K1_DEFER_SEG_ELEMS ((int64_t)1 << 24)
#endif
#ifndef ZK_K2_SEG_ELEMS
#define ZK_K2_SEG_ELEMS ((int64_t)1 << 27)
#endif
// The single pass: 2^26 elements per launch for N <= 8, 2^23 beyond (flat
// 7.5B at N = 64: one launch 3.15 ms, 2^24 2.98, 2^23 2.94, 2^22 2.93;
// Llama-3-8B: 2^28 6.67, 2^26 6.63, 2^24 6.82).
#ifndef ZK_K12_SEG_ELEMS
#define ZK_K12_SEG_ELEMS ((int64_t)1 << 26)
#endif
#ifndef ZK_K12_SEG_ELEMS_LARGE_N
#define ZK_K12_SEG_ELEMS_LARGE_N ((int64_t)1 << 23)
#endif
// The single-pass kernel (reduce and update in one pass, steps without
// clipping) streams N + 3 inputs and 4 outputs.  One-wave workgroups, 16 per
// CU for N <= 8 and 20 beyond (10240 and 8192 B of reserved LDS).  Measured
// (step ms, clipping off; Llama-3-8B N = 8 / GPT-2 N = 64 / flat 7.5B
// N = 64): one wave, cap 16: 6.73 / 0.657 / 3.14; cap 20: 6.81 / 0.651 /
// 3.15; cap 24: 6.95 / 0.658 / 3.21; two waves, cap 8: 6.88 / 0.677 / 3.11;
// four waves, cap 5: 6.98 / 0.669 / 3.11; two waves with 2 or 8 rows per
// load batch: 6.80-7.20 / 0.68-0.81 / 3.15-3.77.  Two-wave caps from none to
// 3 per CU at N = 8 ran at 5.43 (none) to 6.13 TB/s (8 per CU), then fell
// to 2.98 at 3 per CU.
#ifndef ZK_K12_LDS_SMALL_N
#define ZK_K12_LDS_SMALL_N 10240
#endif
#ifndef ZK_K12_LDS
#define ZK_K12_LDS 8192
#endif
// The unit single pass keeps the unit reduce's two-wave workgroups (one
// workgroup column for both) at the two-wave single pass's best cap.
#ifndef ZK_K12U_LDS
#define ZK_K12U_LDS 20480
#endif
// The bf16 single pass keeps two-wave workgroups (one tree partial per 512
// elements, so the largest shard stays within the tree kernel's chunk) and
// the two-wave single pass's best cap, 8 per CU.
#ifndef ZK_K12B_LDS
#define ZK_K12B_LDS 20480
#endif
// The bf16 reduce kernel (longer-lived waves: fp64 squares and a shuffle
// tree per quad) runs best at 12 workgroups per CU for every N; at N = 8,
// cap 8 / 10 / 11 / 12 / 13 / 14 / 16 / none: 5.31 / 6.06 / 6.35 / 6.61 /
// 6.38 / 6.07 / 6.07 / 5.97 TB/s.
#ifndef ZK_K1B_LDS
#define ZK_K1B_LDS 13312
#endif

namespace zk {
namespace dev {

// Reserved LDS of a reduce launch over n contribution rows.
inline unsigned k1_lds(int n) { return n <= 8 ? ZK_K1_LDS_SMALL_N : ZK_K1_LDS; }
inline unsigned k12_lds(int n) { return n <= 8 ? ZK_K12_LDS_SMALL_N : ZK_K12_LDS; }

// Issue a one-shot grid of `blocks` workgroups as launches of at most `seg`
// workgroups each, in order on one stream: launch(b0, nb) launches
// workgroups b0 .. b0 + nb - 1 (the kernels add b0 to blockIdx.x).  A grid
// of up to two segments goes out whole: on short shards the gaps between
// launches cost more than the split gains (GPT-2's 24 M elements at N = 64:
// deferred reduce in one launch 0.497 ms, in launches of 2^24 0.512).
inline int64_t k12_seg_elems(int n) { return n > 8 ? ZK_K12_SEG_ELEMS_LARGE_N : ZK_K12_SEG_ELEMS; }

template <typename Launch>
inline int launch_segments(int64_t blocks, int64_t seg, Launch launch) {
  if (seg < 1) seg = 1;
  if (blocks <= 2 * seg) seg = blocks > 0 ? blocks : 1;
  for (int64_t b0 = 0; b0 < blocks; b0 += seg) {
    launch(b0, blocks - b0 < seg ? blocks - b0 : seg);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
  }
  return (int)hipSuccess;
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// A 128-bit partial sum; bit 63 of hi carries the overflow flag (a workgroup
// partial is below 2^105, so the bit is free).
struct Partial {
  uint64_t lo, hi;
};
static_assert(sizeof(Partial) == kPartialBytes, "partial layout");

constexpr int kRankBatch = 4;  // contribution rows loaded before they are summed

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

// bfloat16 <-> fp32: bf16 is the top half of fp32 (widening is exact);
// narrowing rounds to nearest even, and a NaN stays a quiet NaN (its top
// half with the quiet bit set).  The narrowing is gfx950's conversion
// instruction (v_cvt_pk_bf16_f32), which gives exactly that rule --
// (u + 0x7FFF + bit 16 of u) >> 16, and (u >> 16) | 0x40 for a NaN -- for
// every one of the 2^32 fp32 bit patterns (checked exhaustively on the
// device, with these compile flags); it replaced the same rule written out
// in integer operations.
__device__ __forceinline__ float bf2f(uint32_t bits) { return __uint_as_float(bits << 16); }

__device__ __forceinline__ uint32_t f2bf(float x) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x);
}

enum class Fmt { F16, BF16 };

template <Fmt F>
__device__ __forceinline__ float to_f32(uint32_t bits) {
  if constexpr (F == Fmt::BF16) return bf2f(bits);
  else return h2f(bits);
}

template <Fmt F>
__device__ __forceinline__ uint32_t from_f32(float x) {
  if constexpr (F == Fmt::BF16) return f2bf(x);
  else return f2h(x);
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

__device__ __forceinline__ Partial make_partial(uint64_t lo, uint64_t hi, uint32_t bad) {
  return Partial{lo, hi | ((uint64_t)(bad ? 1u : 0u) << 63)};
}

// Round a nonnegative integer c*2^128 + hi*2^64 + lo (c in {0,1}) to the
// nearest fp64, ties to even.
__device__ inline double u129_to_f64(uint32_t c, uint64_t hi, uint64_t lo) {
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

// The norm, clip coefficient and skip decision from this rank's exact Q and
// the other ranks' share (see zero_step_result_t in zero_shard.h).
__device__ inline void finalize_into(uint64_t qlo, uint64_t qhi, uint32_t bad,
                                     const FinalizeArgs& fa, zero_step_result_t* res) {
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
// Reduce side, per 4-element quad: load 8 bytes from each of the n rows and
// sum them in rank order from +0.  Rows gives row(r), a pointer to rank r's
// fp16 values.
template <int B = kRankBatch, typename Rows>
__device__ __forceinline__ void sum_rows_quad(const Rows& rows, int32_t n, int64_t off,
                                              float (&acc)[4]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) acc[e] = 0.0f;
  for (int r0 = 0; r0 < n; r0 += B) {
    u32x2 d[B];
#pragma unroll
    for (int b = 0; b < B; ++b)
      if (r0 + b < n) d[b] = vload<ZK_K1_NT_LOAD>((const u32x2*)(rows.row(r0 + b) + off));
#pragma unroll
    for (int b = 0; b < B; ++b) {
      if (r0 + b < n) {
#pragma unroll
        for (int w = 0; w < 2; ++w) {
          acc[2 * w] = acc[2 * w] + h2f(d[b][w] & 0xFFFFu);
          acc[2 * w + 1] = acc[2 * w + 1] + h2f(d[b][w] >> 16);
        }
      }
    }
  }
}

// The reduce kernel's quad: the row sum, the quad of g (16 bytes) and the
// exact squares.
template <typename Rows>
__device__ __forceinline__ void reduce_quad(const Rows& rows, int32_t n, int64_t qd, float inv32,
                                            float* __restrict__ grad, uint64_t& qlo,
                                            uint64_t& qhi, uint32_t& bad) {
  const int64_t off = qd * 4;
  float acc[4];
  sum_rows_quad(rows, n, off, acc);
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

// The last shard % 4 elements, one by one.
template <typename Rows>
__device__ inline void reduce_tail(const Rows& rows, int32_t n, int64_t from, int64_t shard,
                                   float inv32, float* __restrict__ grad, uint64_t& qlo,
                                   uint64_t& qhi, uint32_t& bad) {
  for (int64_t j = from; j < shard; ++j) {
    float a = 0.0f;
    for (int r = 0; r < n; ++r) a = a + h2f(rows.row(r)[j]);
    grad[j] = a * inv32;
    uint64_t lo, hi;
    sq_units(a, lo, hi, bad);
    add128(qlo, qhi, lo, hi);
  }
}

// Reduce kernel body for one workgroup covering quads [q_first, q_first + T*Q)
// of a segment of `shard` elements: thread t owns quads q_first + u*T + t.
// Returns the workgroup partial in thread 0.
template <typename Rows>
__device__ inline Partial reduce_block(const Rows& rows, int32_t n, int64_t shard, int64_t q_first,
                                       float inv32, float* __restrict__ grad) {
  uint64_t qlo = 0, qhi = 0;
  uint32_t bad = 0;
  const int64_t full = shard >> 2;
#pragma unroll
  for (int u = 0; u < ZK_K1_QUADS; ++u) {
    const int64_t qd = q_first + (int64_t)u * ZK_K1_THREADS + threadIdx.x;
    if (qd < full) reduce_quad(rows, n, qd, inv32, grad, qlo, qhi, bad);
  }
  // the thread that would own quad `full` takes the ragged tail
  const int64_t rel = full - q_first;
  if (rel >= 0 && rel < (int64_t)ZK_K1_THREADS * ZK_K1_QUADS &&
      (int64_t)threadIdx.x == rel % ZK_K1_THREADS)
    reduce_tail(rows, n, full * 4, shard, inv32, grad, qlo, qhi, bad);
  block_reduce<ZK_K1_THREADS>(qlo, qhi, bad);
  return make_partial(qlo, qhi, bad);
}

// The deferred form of reduce_block: the workgroup covers K chunks of
// ZK_K1_THREADS quads, [q_first, q_first + K*T); thread t sums its quad of
// chunk k (q_first + k*T + t) in the same rank order and keeps its g quad in
// registers until every chunk is summed, then stores them.  The values and
// the partial are those of K reduce_block workgroups.
template <int K, typename Rows>
__device__ inline Partial reduce_block_deferred(const Rows& rows, int32_t n, int64_t shard,
                                                int64_t q_first, float inv32,
                                                float* __restrict__ grad) {
  uint64_t qlo = 0, qhi = 0;
  uint32_t bad = 0;
  const int64_t full = shard >> 2;
  f32x4 g[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int64_t qd = q_first + (int64_t)k * ZK_K1_THREADS + threadIdx.x;
    if (qd < full) {
      float acc[4];
      sum_rows_quad(rows, n, qd * 4, acc);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        g[k][e] = acc[e] * inv32;
        uint64_t lo, hi;
        sq_units(acc[e], lo, hi, bad);
        add128(qlo, qhi, lo, hi);
      }
    }
  }
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int64_t qd = q_first + (int64_t)k * ZK_K1_THREADS + threadIdx.x;
    if (qd < full) vstore<ZK_K1_NT_STORE>(g[k], (f32x4*)(grad + qd * 4));
  }
  const int64_t rel = full - q_first;  // the thread that would own quad `full`: the tail
  if (rel >= 0 && rel < (int64_t)ZK_K1_THREADS * K && (int64_t)threadIdx.x == rel % ZK_K1_THREADS)
    reduce_tail(rows, n, full * 4, shard, inv32, grad, qlo, qhi, bad);
  block_reduce<ZK_K1_THREADS>(qlo, qhi, bad);
  return make_partial(qlo, qhi, bad);
}

// ---------------------------------------------------------------------------
// Adam, per element: one rounding per operation, in this order.
__device__ __forceinline__ void adam1(float g, float c, const AdamScalars& sc, float& p, float& m,
                                      float& v) {
  const float gc = g * c;
  m = sc.b1 * m + sc.omb1 * gc;
  v = sc.b2 * v + sc.omb2 * (gc * gc);
  const float den = __builtin_sqrtf(v) / sc.sqrt_bc2 + sc.eps;
  const float u = (m / den) * sc.step_size;
  p = p * sc.decay - u;
}

// The fp16 (or bf16) results of one wave-contiguous quad (element e in bits
// 16e..16e+15 of h) go to slot[] with aligned 8-byte stores at any slot
// alignment: when the slot is not 8-byte aligned, lane i writes the word
// holding its last `me` results and lane i+1's first 4 - me (through a shuffle
// every lane of the wave takes part in); the pieces at a wave's edges or the
// segment's end go out as 2-byte stores.  Every lane of the wave must call
// this; `valid` says whether the lane's quad is a whole quad of the segment.
__device__ __forceinline__ void store_slot_quad(uint16_t* __restrict__ slot, uint64_t h,
                                                bool valid, int64_t qd, int64_t full) {
  const uint32_t me = (uint32_t)(((uintptr_t)slot >> 1) & 3u);
  const uint32_t lane = threadIdx.x & 63u;
  const int64_t off = qd * 4;
  if (me == 0) {
    if (valid) vstore<ZK_K2_NT_STORE>(h, (uint64_t*)(slot + off));
  } else {
    const uint64_t hn = shfl_down_u64(h, 1);
    const bool right = lane < 63u && qd + 1 < full;
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
}

// Adam body for one wave-contiguous quad of a segment: thread's quad qd of a
// segment with `shard` elements (full = shard / 4 whole quads).  The quads of
// a wave must be consecutive.
template <Fmt F = Fmt::F16>
__device__ inline void adam_quad(const float* __restrict__ grad, float* __restrict__ master,
                                 float* __restrict__ mom, float* __restrict__ var,
                                 uint16_t* __restrict__ slot, int64_t shard, int64_t qd, float c,
                                 const AdamScalars& sc) {
  const int64_t full = shard >> 2;
  const bool valid = qd < full;
  const int64_t off = qd * 4;
  uint64_t h = 0;  // the quad's four fp16 results, element e in bits 16e..16e+15
  if (valid) {
    f32x4 g = vload<ZK_K2_NT_LOAD>((const f32x4*)(grad + off));
    f32x4 p = vload<ZK_K2_NT_LOAD>((const f32x4*)(master + off));
    f32x4 m = vload<ZK_K2_NT_LOAD>((const f32x4*)(mom + off));
    f32x4 v = vload<ZK_K2_NT_LOAD>((const f32x4*)(var + off));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float pp = p[e], mm = m[e], vv = v[e];
      adam1(g[e], c, sc, pp, mm, vv);
      p[e] = pp;
      m[e] = mm;
      v[e] = vv;
      h |= (uint64_t)from_f32<F>(pp) << (16 * e);
    }
    vstore<ZK_K2_NT_STORE>(p, (f32x4*)(master + off));
    vstore<ZK_K2_NT_STORE>(m, (f32x4*)(mom + off));
    vstore<ZK_K2_NT_STORE>(v, (f32x4*)(var + off));
  }
  store_slot_quad(slot, h, valid, qd, full);
  if (qd == full) {
    // the ragged tail: the last shard % 4 elements, one by one
    for (int64_t j = full * 4; j < shard; ++j) {
      float pp = master[j], mm = mom[j], vv = var[j];
      adam1(grad[j], c, sc, pp, mm, vv);
      master[j] = pp;
      mom[j] = mm;
      var[j] = vv;
      slot[j] = (uint16_t)from_f32<F>(pp);
    }
  }
}

// ---------------------------------------------------------------------------
// Single pass for a step without clipping: the update needs no global value
// but the skip decision, so one pass can reduce a quad, add its exact squares
// and apply Adam (clip coefficient 1) from the `in` state to a second,
// distinct `out` state and slot.  The partial goes out as in the reduce
// kernel; the caller adopts `out` only if the finalized step is not skipped,
// so `in` survives a skip untouched.  No gradient is written.
struct StatePair {
  const float* __restrict__ p_in;
  const float* __restrict__ m_in;
  const float* __restrict__ v_in;
  float* __restrict__ p_out;
  float* __restrict__ m_out;
  float* __restrict__ v_out;
  uint16_t* __restrict__ slot_out;
};

template <typename Rows>
__device__ inline void reduce_adam_quad(const Rows& rows, int32_t n, int64_t shard, int64_t qd,
                                        float inv32, const StatePair& st, const AdamScalars& sc,
                                        uint64_t& qlo, uint64_t& qhi, uint32_t& bad) {
  const int64_t full = shard >> 2;
  const bool valid = qd < full;
  const int64_t off = qd * 4;
  uint64_t h = 0;
  if (valid) {
    f32x4 p = vload<ZK_K12_NT_LOAD>((const f32x4*)(st.p_in + off));
    f32x4 m = vload<ZK_K12_NT_LOAD>((const f32x4*)(st.m_in + off));
    f32x4 v = vload<ZK_K12_NT_LOAD>((const f32x4*)(st.v_in + off));
    float acc[4];
    sum_rows_quad<ZK_K12_BATCH>(rows, n, off, acc);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      uint64_t lo, hi;
      sq_units(acc[e], lo, hi, bad);
      add128(qlo, qhi, lo, hi);
      float pp = p[e], mm = m[e], vv = v[e];
      adam1(acc[e] * inv32, 1.0f, sc, pp, mm, vv);
      p[e] = pp;
      m[e] = mm;
      v[e] = vv;
      h |= (uint64_t)f2h(pp) << (16 * e);
    }
    vstore<ZK_K12_NT_STORE>(p, (f32x4*)(st.p_out + off));
    vstore<ZK_K12_NT_STORE>(m, (f32x4*)(st.m_out + off));
    vstore<ZK_K12_NT_STORE>(v, (f32x4*)(st.v_out + off));
  }
  store_slot_quad(st.slot_out, h, valid, qd, full);
  if (qd == full) {
    for (int64_t j = full * 4; j < shard; ++j) {
      float a = 0.0f;
      for (int r = 0; r < n; ++r) a = a + h2f(rows.row(r)[j]);
      uint64_t lo, hi;
      sq_units(a, lo, hi, bad);
      add128(qlo, qhi, lo, hi);
      float pp = st.p_in[j], mm = st.m_in[j], vv = st.v_in[j];
      adam1(a * inv32, 1.0f, sc, pp, mm, vv);
      st.p_out[j] = pp;
      st.m_out[j] = mm;
      st.v_out[j] = vv;
      st.slot_out[j] = (uint16_t)f2h(pp);
    }
  }
}

// Partial-sum kernel body: sum `n_partials` partials with grid-stride
// threads, publish one second-level partial per workgroup, and let the last
// workgroup (ticket) sum those and finalize.  The ticket is left at zero.
__device__ inline void reduce_partials_and_finalize(const Partial* __restrict__ partials,
                                                    int64_t n_partials,
                                                    Partial* __restrict__ level2,
                                                    uint32_t* __restrict__ ticket,
                                                    const FinalizeArgs& fa,
                                                    zero_step_result_t* __restrict__ res) {
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
    level2[blockIdx.x] = make_partial(lo, hi, bad);
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


// ---------------------------------------------------------------------------
// bf16 path: the shard's squared norm is the balanced pairwise tree, in fp64,
// of the exact squares acc_j^2 over element indices zero-padded to a power of
// two.  Every level below is a contiguous power-of-two-aligned subtree of that
// one tree, so the result does not depend on the launch shape.

__device__ __forceinline__ uint64_t shfl_down_bits(uint64_t x, unsigned int d) {
  return shfl_down_u64(x, d);
}

__device__ __forceinline__ double sq_or_zero(float acc, uint32_t& bad) {
  const bool fin = (__float_as_uint(acc) & 0x7F800000u) != 0x7F800000u;
  bad |= fin ? 0u : 1u;
  const double a = fin ? (double)acc : 0.0;
  return a * a;  // exact: at most 48 significant bits, exponent in range
}

// One quad's tree node: (s0 + s1) + (s2 + s3); elements past the shard are +0.
template <typename Rows>
__device__ __forceinline__ double reduce_quad_bf16(const Rows& rows, int32_t n, int64_t qd,
                                                   int64_t shard, float inv32,
                                                   float* __restrict__ grad, uint32_t& bad) {
  const int64_t full = shard >> 2;
  const int64_t off = qd * 4;
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if (qd < full) {
    for (int r0 = 0; r0 < n; r0 += kRankBatch) {
      u32x2 d[kRankBatch];
#pragma unroll
      for (int b = 0; b < kRankBatch; ++b)
        if (r0 + b < n) d[b] = vload<ZK_K1_NT_LOAD>((const u32x2*)(rows.row(r0 + b) + off));
#pragma unroll
      for (int b = 0; b < kRankBatch; ++b) {
        if (r0 + b < n) {
#pragma unroll
          for (int w = 0; w < 2; ++w) {
            acc[2 * w] = acc[2 * w] + bf2f(d[b][w] & 0xFFFFu);
            acc[2 * w + 1] = acc[2 * w + 1] + bf2f(d[b][w] >> 16);
          }
        }
      }
    }
    f32x4 g;
#pragma unroll
    for (int e = 0; e < 4; ++e) g[e] = acc[e] * inv32;
    vstore<ZK_K1_NT_STORE>(g, (f32x4*)(grad + off));
  } else if (qd == full) {
    for (int64_t j = off; j < shard; ++j) {
      float a = 0.0f;
      for (int r = 0; r < n; ++r) a = a + bf2f(rows.row(r)[j]);
      acc[j - off] = a;
      grad[j] = a * inv32;
    }
  } else {
    return 0.0;
  }
  return (sq_or_zero(acc[0], bad) + sq_or_zero(acc[1], bad)) +
         (sq_or_zero(acc[2], bad) + sq_or_zero(acc[3], bad));
}

// Tree over the T quad nodes of a workgroup (wave shuffles, then LDS across
// waves); the subtree and the OR of the flags land in thread 0.
template <int T>
__device__ inline void block_tree(double& x, uint32_t& bad) {
  static_assert(T % 64 == 0 && (T & (T - 1)) == 0, "a power-of-two number of whole waves");
  const uint32_t lane = threadIdx.x & 63u;
  for (unsigned int d = 1; d < 64; d <<= 1) {
    const double y = __longlong_as_double((long long)shfl_down_bits(
        (uint64_t)__double_as_longlong(x), d));
    if ((lane & (2 * d - 1)) == 0) x = x + y;  // left child + right child
    bad |= (uint32_t)__shfl_xor((int)bad, (int)d);
  }
  if constexpr (T == 64) return;
  __shared__ double s_x[T / 64];
  __shared__ uint32_t s_bad[T / 64];
  const int wave = threadIdx.x >> 6;
  if (lane == 0) {
    s_x[wave] = x;
    s_bad[wave] = bad;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < T / 64; w <<= 1)
      for (int i = 0; i < T / 64; i += 2 * w) s_x[i] = s_x[i] + s_x[i + w];
    x = s_x[0];
    for (int w = 1; w < T / 64; ++w) bad |= s_bad[w];
  }
}

// Reduce kernel body (bf16): workgroup covers quads [q_first, q_first + T),
// one quad per thread; returns the subtree partial (value bits in lo, flag in
// bit 63 of hi) in thread 0.
template <typename Rows>
__device__ inline Partial reduce_block_bf16(const Rows& rows, int32_t n, int64_t shard,
                                            int64_t q_first, float inv32,
                                            float* __restrict__ grad) {
  uint32_t bad = 0;
  double x = reduce_quad_bf16(rows, n, q_first + threadIdx.x, shard, inv32, grad, bad);
  block_tree<ZK_K1_THREADS>(x, bad);
  return Partial{(uint64_t)__double_as_longlong(x), (uint64_t)(bad ? 1u : 0u) << 63};
}

// Single pass, bf16: the quad's row sum, its tree node (as reduce_quad_bf16)
// and the update with coefficient 1 from the `in` state into the `out`
// state and bf16 slot.  Returns the quad's node; elements past the shard
// count +0.
template <typename Rows>
__device__ inline double reduce_adam_quad_bf16(const Rows& rows, int32_t n, int64_t shard,
                                               int64_t qd, float inv32, const StatePair& st,
                                               const AdamScalars& sc, uint32_t& bad) {
  const int64_t full = shard >> 2;
  const bool valid = qd < full;
  const int64_t off = qd * 4;
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  uint64_t h = 0;
  if (valid) {
    f32x4 p = vload<ZK_K12_NT_LOAD>((const f32x4*)(st.p_in + off));
    f32x4 m = vload<ZK_K12_NT_LOAD>((const f32x4*)(st.m_in + off));
    f32x4 v = vload<ZK_K12_NT_LOAD>((const f32x4*)(st.v_in + off));
    for (int r0 = 0; r0 < n; r0 += kRankBatch) {
      u32x2 d[kRankBatch];
#pragma unroll
      for (int b = 0; b < kRankBatch; ++b)
        if (r0 + b < n) d[b] = vload<ZK_K1_NT_LOAD>((const u32x2*)(rows.row(r0 + b) + off));
#pragma unroll
      for (int b = 0; b < kRankBatch; ++b) {
        if (r0 + b < n) {
#pragma unroll
          for (int w = 0; w < 2; ++w) {
            acc[2 * w] = acc[2 * w] + bf2f(d[b][w] & 0xFFFFu);
            acc[2 * w + 1] = acc[2 * w + 1] + bf2f(d[b][w] >> 16);
          }
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float pp = p[e], mm = m[e], vv = v[e];
      adam1(acc[e] * inv32, 1.0f, sc, pp, mm, vv);
      p[e] = pp;
      m[e] = mm;
      v[e] = vv;
      h |= (uint64_t)f2bf(pp) << (16 * e);
    }
    vstore<ZK_K12_NT_STORE>(p, (f32x4*)(st.p_out + off));
    vstore<ZK_K12_NT_STORE>(m, (f32x4*)(st.m_out + off));
    vstore<ZK_K12_NT_STORE>(v, (f32x4*)(st.v_out + off));
  }
  store_slot_quad(st.slot_out, h, valid, qd, full);
  if (qd == full) {
    for (int64_t j = off; j < shard; ++j) {
      float a = 0.0f;
      for (int r = 0; r < n; ++r) a = a + bf2f(rows.row(r)[j]);
      acc[j - off] = a;
      float pp = st.p_in[j], mm = st.m_in[j], vv = st.v_in[j];
      adam1(a * inv32, 1.0f, sc, pp, mm, vv);
      st.p_out[j] = pp;
      st.m_out[j] = mm;
      st.v_out[j] = vv;
      st.slot_out[j] = (uint16_t)f2bf(pp);
    }
  } else if (!valid) {
    return 0.0;
  }
  return (sq_or_zero(acc[0], bad) + sq_or_zero(acc[1], bad)) +
         (sq_or_zero(acc[2], bad) + sq_or_zero(acc[3], bad));
}

__device__ inline void finalize_bf16_into(double tree, uint32_t bad, const FinalizeArgs& fa,
                                          zero_step_result_t* res) {
  const double own = (tree * fa.inv64) * fa.inv64;
  const double tot = own + fa.other_sq;
  const double norm = __builtin_sqrt(tot);
  double coef = 1.0;
  if (fa.max_norm > 0.0) {
    const double c = fa.max_norm / (norm + 1e-6);
    coef = (c < 1.0) ? c : 1.0;
  }
  res->own_q_lo = 0;
  res->own_q_hi = 0;
  res->own_sq = own;
  res->total_sq = tot;
  res->norm = norm;
  res->clip_coef = (float)coef;
  res->overflow = bad ? 1 : 0;
  res->skip = (bad || fa.other_overflow) ? 1 : 0;
  res->reserved = 0;
}

constexpr int kTreeChunk = 16384;  // most partials one workgroup of the tree kernel sums

// LDS tree over `count` values (count a power of two, <= kTreeChunk) held in
// s[0..count); the result lands in s[0].
__device__ inline void lds_tree(double* s, int count) {
  for (int w = 1; w < count; w <<= 1) {
    __syncthreads();
    for (int i = (int)threadIdx.x * 2 * w; i < count; i += kThreads * 2 * w) s[i] = s[i] + s[i + w];
  }
  __syncthreads();
}

// Tree kernel body (bf16): workgroup j sums partials [j*chunk, (j+1)*chunk)
// (chunk a power of two; partials past n_partials count +0) into a level-2
// node; the last workgroup (ticket) sums the level-2 nodes, zero-padded to a
// power of two, and finalizes.
__device__ inline void tree_partials_and_finalize_bf16(const Partial* __restrict__ partials,
                                                       int64_t n_partials, int chunk,
                                                       Partial* __restrict__ level2,
                                                       uint32_t* __restrict__ ticket,
                                                       const FinalizeArgs& fa,
                                                       zero_step_result_t* __restrict__ res) {
  __shared__ double s[kTreeChunk];
  __shared__ uint32_t s_bad;
  __shared__ uint32_t s_last;
  if (threadIdx.x == 0) s_bad = 0u;
  __syncthreads();
  uint32_t bad = 0;
  const int64_t base = (int64_t)blockIdx.x * chunk;
  for (int i = threadIdx.x; i < chunk; i += kThreads) {
    double v = 0.0;
    if (base + i < n_partials) {
      const Partial pt = partials[base + i];
      v = __longlong_as_double((long long)pt.lo);
      bad |= (uint32_t)(pt.hi >> 63);
    }
    s[i] = v;
  }
  if (bad) atomicOr(&s_bad, 1u);
  lds_tree(s, chunk);
  if (threadIdx.x == 0) {
    level2[blockIdx.x] = Partial{(uint64_t)__double_as_longlong(s[0]),
                                 (uint64_t)(s_bad ? 1u : 0u) << 63};
    __threadfence();
    const uint32_t prev = atomicAdd(ticket, 1u);
    s_last = (prev == gridDim.x - 1) ? 1u : 0u;
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  int count = 1;
  while (count < (int)gridDim.x) count <<= 1;
  bad = 0;
  for (int i = threadIdx.x; i < count; i += kThreads) {
    double v = 0.0;
    if (i < (int)gridDim.x) {
      const Partial pt = level2[i];
      v = __longlong_as_double((long long)pt.lo);
      bad |= (uint32_t)(pt.hi >> 63);
    }
    s[i] = v;
  }
  if (threadIdx.x == 0) s_bad = 0u;
  __syncthreads();
  if (bad) atomicOr(&s_bad, 1u);
  lds_tree(s, count);
  if (threadIdx.x == 0) {
    finalize_bf16_into(s[0], s_bad, fa, res);
    *ticket = 0u;
  }
}

}  // namespace dev
}  // namespace zk
