/*
 * CPU oracle, C form of the reduce-side statistics: TEST INFRASTRUCTURE ONLY
 * (used by tests/ at full workload sizes, where numpy would take minutes).
 * It states the same definition as zero_oracle.py, written out plainly:
 *
 *   acc_j = (...((+0 + c_0j) + c_1j) + ...) + c_(N-1)j   in IEEE fp32,
 *           ranks in order 0..N-1 (page "10.6 ZeRO 与 FSDP", §10.6.1:
 *           reduce-scatter = reduce, then each GPU keeps its 1/N slice);
 *   bad   = some acc_j is +inf, -inf or NaN;
 *   Q     = sum over finite acc_j of (acc_j * 2^24)^2, an exact integer.
 *
 * fp16 -> fp32 is done by bit manipulation (exact); fp32 adds are single IEEE
 * operations (build with -ffp-contract=off, no fast-math); Q uses unsigned
 * __int128, exact because every term is below 2^92 and a chunk holds far
 * fewer than 2^36 elements.  Threads split the element range; their partial
 * Q are integers, so the order of the final sum does not matter.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static float half_to_float(uint16_t h) {
  uint32_t s = (uint32_t)(h >> 15) << 31, e = (h >> 10) & 0x1F, f = h & 0x3FF, bits;
  if (e == 0x1F) {
    bits = s | 0x7F800000u | (f << 13); /* inf or NaN */
  } else if (e == 0) {
    if (f == 0) {
      bits = s; /* signed zero */
    } else {
      float x = (float)f * 0x1p-24f; /* subnormal: exact (f < 2^10) */
      memcpy(&bits, &x, 4);
      bits |= s;
    }
  } else {
    bits = s | ((e + 112) << 23) | (f << 13);
  }
  float out;
  memcpy(&out, &bits, 4);
  return out;
}

/*
 * rows: host [n] pointers, each to `count` fp16 bit patterns.
 * Outputs Q as (q_lo, q_hi) and the overflow flag.  Returns 0, or -1 if an
 * |acc| reaches 2^24 (outside the exact-integer range).
 */
int oracle_reduce_stats(const uint16_t* const* rows, int n, int64_t count, uint64_t* q_lo,
                        uint64_t* q_hi, int32_t* bad_out) {
  unsigned __int128 total = 0;
  int bad = 0, range_err = 0;
#pragma omp parallel
  {
    unsigned __int128 q = 0;
    int b = 0, re = 0;
#pragma omp for schedule(static)
    for (int64_t j = 0; j < count; ++j) {
      float acc = 0.0f;
      for (int r = 0; r < n; ++r) acc = acc + half_to_float(rows[r][j]);
      if (!isfinite(acc)) {
        b = 1;
        continue;
      }
      double k = fabs((double)acc) * 16777216.0; /* exact */
      if (k >= 281474976710656.0) { /* 2^48 */
        re = 1;
        continue;
      }
      uint64_t ki = (uint64_t)k;
      q += (unsigned __int128)ki * ki;
    }
#pragma omp critical
    {
      total += q;
      bad |= b;
      range_err |= re;
    }
  }
  *q_lo = (uint64_t)total;
  *q_hi = (uint64_t)(total >> 64);
  *bad_out = bad;
  return range_err ? -1 : 0;
}

/*
 * bf16 path.  acc_j as above with bf16 inputs (bf16 -> fp32 is exact: the
 * pattern is the top half of the fp32 one); sq_j = acc_j^2 in fp64 (exact),
 * +0 for a non-finite acc_j, and +0 for j >= count up to `width`, a power of
 * two >= count.  The result is the balanced pairwise tree over sq_0 ..
 * sq_(width-1): level by level, node = left + right.  Written out with a
 * scratch array of `width` doubles.  Returns 0, or -1 on a bad width or no
 * memory.
 */
int oracle_reduce_tree_bf16(const uint16_t* const* rows, int n, int64_t count, int64_t width,
                            double* tree, int32_t* bad_out) {
  if (width < 1 || (width & (width - 1)) || width < count) return -1;
  double* y = (double*)malloc((size_t)width * sizeof(double));
  if (!y) return -1;
  int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
  for (int64_t j = 0; j < width; ++j) {
    double sq = 0.0;
    if (j < count) {
      float acc = 0.0f;
      for (int r = 0; r < n; ++r) {
        uint32_t bits = (uint32_t)rows[r][j] << 16;
        float x;
        memcpy(&x, &bits, 4);
        acc = acc + x;
      }
      if (isfinite(acc)) {
        sq = (double)acc * (double)acc;
      } else {
        bad = 1;
      }
    }
    y[j] = sq;
  }
  /* in place, one thread: y[i] is written only after y[2i] and y[2i+1] were read */
  for (int64_t half = width / 2; half >= 1; half /= 2)
    for (int64_t i = 0; i < half; ++i) y[i] = y[2 * i] + y[2 * i + 1];
  *tree = y[0];
  *bad_out = bad;
  free(y);
  return 0;
}
