/*
 * CPU oracle, C form of the reduce-side statistics and of the update:
 * TEST INFRASTRUCTURE ONLY (used by tests/ at full workload sizes, where
 * numpy would take minutes).  It states the same definitions as
 * zero_oracle.py, written out plainly:
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

/* ------------------------------------------------------------------------ */
/*
 * The rest of the step, element by element, for whole-shard comparisons at
 * full workload sizes.  Same definitions as zero_oracle.py (unscale,
 * adam_apply and the 16-bit cast), written out plainly; each fp32 operation
 * is one IEEE single-precision operation rounded to nearest even (x86-64 SSE
 * arithmetic, built with -ffp-contract=off, no fast-math; sqrtf is correctly
 * rounded).
 */

/* IEEE binary16 from fp32, round to nearest even (binary16: sign, 5 exponent
 * bits biased by 15, 10 fraction bits; normal numbers from 2^-14, subnormal
 * multiples of 2^-24 below it; largest finite 65504).  Overflow gives +-inf;
 * a NaN gives a NaN of the same sign. */
static uint16_t float_to_half(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  const uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return (uint16_t)(sign | 0x7E00u); /* NaN */
  const int e = (int)(a >> 23) - 127;                     /* unbiased exponent */
  if (e > 15) return (uint16_t)(sign | 0x7C00u);          /* >= 2^16, or inf */
  if (a == 0) return sign;
  /* significand with the implicit bit (fp32 subnormals are far below 2^-25) */
  const uint32_t sig = (a & 0x7FFFFFu) | (a >= 0x00800000u ? 0x800000u : 0u);
  uint32_t keep, rest, half;
  int drop; /* low bits of sig that do not fit */
  if (e >= -14) {
    drop = 13; /* normal binary16: 10 fraction bits of the 23 */
  } else {
    drop = 13 + (-14 - e); /* subnormal binary16: quantum 2^-24 */
    if (drop > 25) return sign; /* below 2^-25: rounds to zero */
  }
  keep = sig >> drop;
  rest = sig & ((1u << drop) - 1u);
  half = 1u << (drop - 1);
  uint32_t h;
  if (e >= -14)
    h = ((uint32_t)(e + 15) << 10) | (keep & 0x3FFu);
  else
    h = keep; /* subnormal: exponent field 0 */
  if (rest > half || (rest == half && (h & 1u))) h += 1u; /* carries into the exponent */
  return (uint16_t)(sign | h);                            /* 0x7C00 after a carry is inf */
}

/* bfloat16 from fp32, round to nearest even: the upper 16 bits of the fp32
 * pattern, rounded on the lower 16; a NaN stays a quiet NaN of the same sign. */
static uint16_t float_to_bf16(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  uint32_t upper = u >> 16;
  const uint32_t lower = u & 0xFFFFu;
  if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) upper += 1u;
  return (uint16_t)upper;
}

static float bf16_to_float(uint16_t b) {
  uint32_t bits = (uint32_t)b << 16;
  float x;
  memcpy(&x, &bits, 4);
  return x;
}

void oracle_cast16(const float* x, uint16_t* out, int64_t count, int bf16) {
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < count; ++j) out[j] = bf16 ? float_to_bf16(x[j]) : float_to_half(x[j]);
}

/*
 * g_j = f32(acc_j * inv32) with acc_j the rank-ordered fp32 sum from +0 of
 * the N rows (fp16 or, with bf16, bfloat16 bit patterns): the oracle's
 * reduce_contributions then unscale.
 */
void oracle_reduce_unscale(const uint16_t* const* rows, int n, int64_t count, int bf16,
                           float inv32, float* g) {
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < count; ++j) {
    float acc = 0.0f;
    for (int r = 0; r < n; ++r)
      acc = acc + (bf16 ? bf16_to_float(rows[r][j]) : half_to_float(rows[r][j]));
    g[j] = acc * inv32;
  }
}

/*
 * The oracle's adam_apply on `count` elements, in place on p, m, v, and the
 * 16-bit cast of the new p into slot.  sc = {b1, 1-b1, b2, 1-b2, eps,
 * lr/(1-b1^t), sqrt(1-b2^t), 1-lr*wd} as fp32 values rounded once on the
 * host (zero_oracle.step_scalars).  Per element, one rounding per operation:
 *   gc = g*c;  m = b1*m + (1-b1)*gc;  v = b2*v + (1-b2)*(gc*gc);
 *   den = sqrt(v)/sqrt_bc2 + eps;  u = (m/den)*step_size;  p = p*decay - u
 */
void oracle_adam_update(const float* g, float* p, float* m, float* v, uint16_t* slot,
                        int64_t count, const float* sc, float coef, int bf16) {
  const float b1 = sc[0], omb1 = sc[1], b2 = sc[2], omb2 = sc[3], eps = sc[4];
  const float step_size = sc[5], sqrt_bc2 = sc[6], decay = sc[7];
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < count; ++j) {
    const float gc = g[j] * coef;
    const float mt = b1 * m[j] + omb1 * gc;
    const float gsq = gc * gc;
    const float vt = b2 * v[j] + omb2 * gsq;
    const float den = sqrtf(vt) / sqrt_bc2 + eps;
    const float u = (mt / den) * step_size;
    const float pt = p[j] * decay - u;
    m[j] = mt;
    v[j] = vt;
    p[j] = pt;
    slot[j] = bf16 ? float_to_bf16(pt) : float_to_half(pt);
  }
}

/* Number of positions where two arrays of `count` words of `width` bytes
 * (2 or 4) differ bitwise; -1 for another width. */
int64_t oracle_count_unequal(const void* a, const void* b, int64_t count, int width) {
  if (width != 2 && width != 4) return -1;
  int64_t bad = 0;
  if (width == 4) {
    const uint32_t *x = (const uint32_t*)a, *y = (const uint32_t*)b;
#pragma omp parallel for schedule(static) reduction(+ : bad)
    for (int64_t j = 0; j < count; ++j) bad += x[j] != y[j];
  } else {
    const uint16_t *x = (const uint16_t*)a, *y = (const uint16_t*)b;
#pragma omp parallel for schedule(static) reduction(+ : bad)
    for (int64_t j = 0; j < count; ++j) bad += x[j] != y[j];
  }
  return bad;
}
