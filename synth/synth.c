/*
 * Seeded, counter-addressable synthetic inputs for the ZeRO shard step.
 *
 * This file holds input generation only: no step of the optimizer, the
 * reduction or the norm lives here.  Both the CPU oracle and the GPU feeder
 * call these functions, so the two sides always see bit-identical inputs.
 *
 * Random bits: Philox4x32 with 10 rounds, from J. K. Salmon, M. A. Moraes,
 * R. O. Dror, D. E. Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3"
 * (SC'11), section 3 (the Philox S-box: two 32x32->64 multiplies per round,
 * a Weyl-sequence key schedule).  Element e of a stream takes 32-bit word
 * (e mod 4) of the block at counter e/4, so any element range can be
 * regenerated on its own.
 *
 * Gradient contributions are fp16 (or bf16) values drawn from the normal
 * distribution N(0, std^2) discretised onto the format's grid: each finite value h gets
 * the probability mass of the real interval that rounds to h under
 * round-to-nearest-even, resolved to 2^-32 (one 32-bit word per element) and
 * drawn by inversion with a guide table (Chen and Asau, 1974).  Master
 * weights are fp32 values f32(sigma * z) with z from the Box-Muller
 * transform (Box and Muller, 1958) on two 32-bit words.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

static inline void philox_round(uint32_t c[4], const uint32_t k[2]) {
  uint64_t p0 = (uint64_t)PHILOX_M0 * c[0];
  uint64_t p1 = (uint64_t)PHILOX_M1 * c[2];
  uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
  uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
  uint32_t n0 = hi1 ^ c[1] ^ k[0];
  uint32_t n2 = hi0 ^ c[3] ^ k[1];
  c[0] = n0;
  c[1] = lo1;
  c[2] = n2;
  c[3] = lo0;
}

void synth_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  uint32_t c[4] = {ctr[0], ctr[1], ctr[2], ctr[3]};
  uint32_t k[2] = {key[0], key[1]};
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k[0] += PHILOX_W0;
      k[1] += PHILOX_W1;
    }
    philox_round(c, k);
  }
  memcpy(out, c, sizeof c);
}

/* ------------------------------------------------------------------------ */
/* fp16 grid helpers (bit patterns <-> exact real values)                    */

static double half_bits_to_double(uint16_t h) {
  int s = h >> 15, e = (h >> 10) & 0x1F, f = h & 0x3FF;
  double x;
  if (e == 0)
    x = ldexp((double)f, -24);
  else
    x = ldexp((double)(f | 0x400), e - 25);
  return s ? -x : x;
}

/* fp16: 31744 finite non-negative patterns (0x0000..0x7BFF) and as many
 * negative ones; bf16: 32640 (0x0000..0x7F7F) and as many negative ones. */
#define SYNTH_FP16_TABLE_N 63488
#define SYNTH_BF16_TABLE_N 65280
#define SYNTH_GUIDE_N 65536

int64_t synth_fp16_table_size(void) { return SYNTH_FP16_TABLE_N; }
int64_t synth_table_size(int fmt) { return fmt == 1 ? SYNTH_BF16_TABLE_N : SYNTH_FP16_TABLE_N; }

static double bf16_bits_to_double(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

static double normal_cdf(double x) { return 0.5 * erfc(-x / sqrt(2.0)); }

/*
 * Build the inversion table for N(0, std^2) on the grid of a 16-bit format
 * (fmt 0: IEEE binary16, fmt 1: bfloat16).
 * thr[k] = floor(2^32 * Phi(b_k / std)), where b_k is the upper edge of the
 * round-to-nearest interval of the k-th finite value in ascending order
 * (-0 is its own value, just below +0).  val[k] is that bit pattern.
 * guide[i] = smallest k with thr[k] > i * 2^16.
 * Returns 0, or -1 on bad arguments.
 */
int synth_normal_table(int fmt, double std, uint64_t* thr, uint16_t* val, uint32_t* guide) {
  if (!(std > 0.0) || !thr || !val || !guide || (fmt != 0 && fmt != 1)) return -1;
  double (*value)(uint16_t) = fmt == 1 ? bf16_bits_to_double : half_bits_to_double;
  const int maxmag = fmt == 1 ? 0x7F7F : 0x7BFF; /* largest finite magnitude pattern */
  const int64_t n = synth_table_size(fmt);
  int64_t k = 0;
  /* negative values, ascending: -max ... -smallest subnormal */
  for (int mb = maxmag; mb >= 1; --mb) {
    double a = value((uint16_t)mb);
    double b = value((uint16_t)(mb - 1));
    double edge = -0.5 * (a + b); /* midpoint toward zero */
    val[k] = (uint16_t)(0x8000 | mb);
    thr[k++] = (uint64_t)floor(normal_cdf(edge / std) * 4294967296.0);
  }
  /* -0 takes [-half the smallest subnormal, 0) */
  val[k] = 0x8000;
  thr[k++] = (uint64_t)floor(normal_cdf(0.0) * 4294967296.0);
  /* +0 .. +max */
  for (int b = 0; b <= maxmag; ++b) {
    val[k] = (uint16_t)b;
    if (b == maxmag) {
      thr[k++] = 4294967296ull;
    } else {
      double edge = 0.5 * (value((uint16_t)b) + value((uint16_t)(b + 1)));
      thr[k++] = (uint64_t)floor(normal_cdf(edge / std) * 4294967296.0);
    }
  }
  if (k != n) return -1;
  /* monotone by construction of Phi; enforce against libm wobble */
  for (int64_t i = 1; i < k; ++i)
    if (thr[i] < thr[i - 1]) thr[i] = thr[i - 1];
  int64_t j = 0;
  for (int64_t i = 0; i < SYNTH_GUIDE_N; ++i) {
    uint64_t lo = (uint64_t)i << 16;
    while (thr[j] <= lo) ++j;
    guide[i] = (uint32_t)j;
  }
  return 0;
}

int synth_fp16_normal_table(double std, uint64_t* thr, uint16_t* val, uint32_t* guide) {
  return synth_normal_table(0, std, thr, val, guide);
}

static inline uint16_t table_draw(uint32_t u, const uint64_t* thr, const uint16_t* val,
                                  const uint32_t* guide) {
  uint32_t j = guide[u >> 16];
  while (thr[j] <= u) ++j;
  return val[j];
}

/*
 * Fill out[0..count) with fp16 draws for stream (key, word2, word3) at
 * element indexes begin..begin+count-1.  Elements at index >= limit are +0
 * (padding).  Parallel over 4-element counter blocks.
 */
void synth_fp16_normal(uint32_t key0, uint32_t key1, uint32_t word2, uint32_t word3, int64_t begin,
                       int64_t count, int64_t limit, const uint64_t* thr, const uint16_t* val,
                       const uint32_t* guide, uint16_t* out) {
  if (count <= 0) return;
  const uint32_t key[2] = {key0, key1};
  int64_t first_blk = begin >> 2;
  int64_t last_blk = (begin + count - 1) >> 2;
#pragma omp parallel for schedule(static)
  for (int64_t blk = first_blk; blk <= last_blk; ++blk) {
    uint32_t ctr[4] = {(uint32_t)blk, (uint32_t)((uint64_t)blk >> 32), word2, word3};
    uint32_t w[4];
    synth_philox4x32_10(ctr, key, w);
    for (int q = 0; q < 4; ++q) {
      int64_t e = blk * 4 + q;
      if (e < begin || e >= begin + count) continue;
      out[e - begin] = (e < limit) ? table_draw(w[q], thr, val, guide) : (uint16_t)0;
    }
  }
}

/*
 * fp32 normal draws: out[i] = f32(sigma * z), z standard normal via
 * Box-Muller.  Element e uses the word pair (2p, 2p+1), p = (e/2) mod 2, of
 * the block at counter e/4: even e takes the cosine branch, odd e the sine.
 * Elements at index >= limit are +0.
 */
void synth_f32_normal(uint32_t key0, uint32_t key1, uint32_t word2, uint32_t word3, int64_t begin,
                      int64_t count, int64_t limit, double sigma, float* out) {
  if (count <= 0) return;
  const uint32_t key[2] = {key0, key1};
  const double two_pi = 6.283185307179586476925286766559;
  int64_t first_blk = begin >> 2;
  int64_t last_blk = (begin + count - 1) >> 2;
#pragma omp parallel for schedule(static)
  for (int64_t blk = first_blk; blk <= last_blk; ++blk) {
    uint32_t ctr[4] = {(uint32_t)blk, (uint32_t)((uint64_t)blk >> 32), word2, word3};
    uint32_t w[4];
    synth_philox4x32_10(ctr, key, w);
    for (int pr = 0; pr < 2; ++pr) {
      double u1 = ((double)w[2 * pr] + 1.0) * (1.0 / 4294967296.0); /* (0, 1] */
      double u2 = (double)w[2 * pr + 1] * (1.0 / 4294967296.0);     /* [0, 1) */
      double r = sqrt(-2.0 * log(u1));
      double th = two_pi * u2;
      double z[2] = {r * cos(th), r * sin(th)};
      for (int q = 0; q < 2; ++q) {
        int64_t e = blk * 4 + 2 * pr + q;
        if (e < begin || e >= begin + count) continue;
        out[e - begin] = (e < limit) ? (float)(sigma * z[q]) : 0.0f;
      }
    }
  }
}

/* Raw words, for tests and for seeded choices (e.g. an injection site). */
void synth_words(uint32_t key0, uint32_t key1, uint32_t word2, uint32_t word3, int64_t begin,
                 int64_t count, uint32_t* out) {
  const uint32_t key[2] = {key0, key1};
  for (int64_t i = 0; i < count; ++i) {
    int64_t e = begin + i;
    int64_t blk = e >> 2;
    uint32_t ctr[4] = {(uint32_t)blk, (uint32_t)((uint64_t)blk >> 32), word2, word3};
    uint32_t w[4];
    synth_philox4x32_10(ctr, key, w);
    out[i] = w[e & 3];
  }
}
