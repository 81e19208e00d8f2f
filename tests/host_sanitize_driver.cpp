// Host-only exercise of the C ABI for sanitizer builds (AddressSanitizer with
// UndefinedBehaviorSanitizer, and ThreadSanitizer): the planner, the unit
// planner and table preparation, the model-state bytes, the loss scaler, the
// argument checks of the device calls (each rejected before anything is
// launched), and the host Adam of the offload form with 1..16 worker threads
// at every vector width, every result compared bit for bit with one thread of
// scalar code.  No GPU is touched.  Exit status 0 when every check holds.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <vector>

#include "zero_shard.h"

namespace {

int g_fail = 0;

#define CHECK(cond)                                                        \
  do {                                                                     \
    if (!(cond)) {                                                         \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond);   \
      ++g_fail;                                                            \
    }                                                                      \
  } while (0)

struct Rng {  // xorshift64*
  uint64_t s;
  uint64_t next() {
    s ^= s >> 12;
    s ^= s << 25;
    s ^= s >> 27;
    return s * 0x2545F4914F6CDD1Dull;
  }
  int64_t below(int64_t n) { return (int64_t)(next() % (uint64_t)n); }
  float normal() {  // sum of uniforms: enough spread for the update
    double a = 0;
    for (int i = 0; i < 12; ++i) a += (double)(next() >> 11) * 0x1p-53;
    return (float)(a - 6.0);
  }
};

void planner(Rng& rng) {
  for (int it = 0; it < 2000; ++it) {
    const int nt = (int)rng.below(9);
    std::vector<int64_t> numels(nt > 0 ? nt : 1), offs(nt > 0 ? nt : 1);
    for (int i = 0; i < nt; ++i) numels[i] = rng.below(200);
    const int n = 1 + (int)rng.below(17), align = (int)(1 + rng.below(8));
    zero_plan_t p;
    CHECK(zero_plan(numels.data(), nt, n, align, &p, offs.data()) == ZERO_OK);
    int64_t covered = 0;
    for (int r = 0; r < n; ++r) {
      const int64_t real = zero_plan_real(&p, r);
      CHECK(real >= 0 && real <= p.shard);
      covered += real;
      int32_t cnt = -1;
      std::vector<zero_segment_t> seg(2);
      const int rc = zero_plan_segments(&p, numels.data(), offs.data(), nt, r, seg.data(), 2, &cnt);
      CHECK(rc == ZERO_OK || (rc == ZERO_ENOSPC && cnt > 2));
      if (cnt > 2) {
        seg.resize(cnt);
        CHECK(zero_plan_segments(&p, numels.data(), offs.data(), nt, r, seg.data(), cnt, &cnt) ==
              ZERO_OK);
      }
      int64_t len = 0;
      for (int k = 0; k < cnt; ++k) len += seg[k].length;
      CHECK(len == real);
    }
    CHECK(covered == p.psi);
  }
  // overflow and bad arguments are refused
  zero_plan_t p;
  const int64_t big[2] = {INT64_MAX / 2, INT64_MAX / 2};
  CHECK(zero_plan(big, 2, 1, 1, &p, nullptr) == ZERO_EINVAL);
  const int64_t neg[1] = {-1};
  CHECK(zero_plan(neg, 1, 1, 1, &p, nullptr) == ZERO_EINVAL);
  CHECK(zero_plan(nullptr, 1, 1, 1, &p, nullptr) == ZERO_EINVAL);
  CHECK(zero_plan(nullptr, 0, 0, 1, &p, nullptr) == ZERO_EINVAL);
  const int64_t huge[1] = {INT64_MAX / 2};
  CHECK(zero_plan(huge, 1, 0x7FFFFFFF, 0x7FFFFFFF, &p, nullptr) == ZERO_OK);
  CHECK(p.psi_padded >= p.psi && p.psi_padded / p.world_size == p.shard);
  CHECK(zero_plan(huge, 1, 1, 0, &p, nullptr) == ZERO_EINVAL);
  CHECK(strlen(zero_last_error()) > 0);
  CHECK(zero_plan_real(nullptr, 0) == -1);
}

void units(Rng& rng) {
  for (int it = 0; it < 500; ++it) {
    const int nt = 1 + (int)rng.below(10);
    std::vector<int64_t> numels(nt);
    std::vector<int32_t> uot(nt);
    int32_t u = 0;
    for (int i = 0; i < nt; ++i) {
      numels[i] = rng.below(5000);
      if (i > 0 && rng.below(2)) ++u;
      uot[i] = u;
    }
    const int n = 1 + (int)rng.below(16);
    zero_unit_plan_t up;
    std::vector<zero_unit_info_t> info(nt);
    const int cap = (int)rng.below(nt + 1);
    const int rc = zero_plan_units(numels.data(), nt, uot.data(), n, 1, &up, info.data(), cap);
    CHECK(rc == (up.n_units > cap ? ZERO_ENOSPC : ZERO_OK));
    if (rc) continue;
    // a table of made-up, well-aligned device addresses (never dereferenced)
    std::vector<zero_unit_buffers_t> tab(up.n_units);
    uintptr_t base = (uintptr_t)1 << 40;
    for (int64_t k = 0; k < up.n_units; ++k) {
      zero_unit_buffers_t& b = tab[k];
      const int64_t s = info[k].shard;
      b.contrib = (const uint16_t*)(base);
      b.ld = (s + 7) / 8 * 8;
      b.grad = (float*)(base + (1 << 24));
      b.master = (float*)(base + (2 << 24));
      b.m = (float*)(base + (3 << 24));
      b.v = (float*)(base + (4 << 24));
      b.param16 = (uint16_t*)(base + (5 << 24) + 2 * rng.below(4));
      b.shard = s;
      base += (uintptr_t)1 << 28;
    }
    int64_t b1 = -1, b2 = -1;
    CHECK(zero_units_prepare(tab.data(), (int32_t)up.n_units, &b1, &b2) == ZERO_OK);
    CHECK(b1 >= up.n_units && b2 >= 0);
    CHECK(zero_units_workspace_bytes(tab.data(), (int32_t)up.n_units) > 0);
    if (up.n_units > 1) {
      tab[1].reduce_block += 1;  // stale table: refused
      CHECK(zero_units_workspace_bytes(tab.data(), (int32_t)up.n_units) == 0);
      zero_step_args_t a = {};
      a.lr = 1e-3; a.beta1 = 0.9; a.beta2 = 0.999; a.eps = 1e-8; a.loss_scale = 1; a.step = 1;
      CHECK(zero_units_adam_apply(tab.data(), nullptr, (int32_t)up.n_units, &a, nullptr, 0) ==
            ZERO_EINVAL);
    }
  }
}

zero_step_args_t good_args() {
  zero_step_args_t a = {};
  a.lr = 1e-3; a.beta1 = 0.9; a.beta2 = 0.999; a.eps = 1e-8; a.weight_decay = 0.01;
  a.max_grad_norm = 1.0; a.loss_scale = 1024; a.step = 1;
  return a;
}

void device_call_checks() {
  // every call below fails an argument check before any launch
  zero_plan_t p = {1000, 2, 1, 500, 1000};
  zero_step_args_t a = good_args();
  const uintptr_t base = (uintptr_t)1 << 40;
  const uint16_t* rows[2] = {(const uint16_t*)base, (const uint16_t*)(base + 4096)};
  float* f = (float*)(base + (1 << 20));
  uint16_t* slot = (uint16_t*)(base + (2 << 20));
  zero_step_result_t* res = (zero_step_result_t*)(base + (3 << 20));
  void* ws = (void*)(base + (4 << 20));
  const size_t wsb = zero_workspace_bytes(&p);
  CHECK(wsb > 0);
  CHECK(zero_reduce_adam_step(nullptr, 0, rows, f, f, f, slot, f, ws, wsb, &a, res, 0) ==
        ZERO_EINVAL);
  CHECK(zero_reduce_adam_step(&p, 2, rows, f, f, f, slot, f, ws, wsb, &a, res, 0) == ZERO_EINVAL);
  CHECK(zero_reduce_adam_step(&p, 0, rows, f, f, f, slot, f, ws, 16, &a, res, 0) == ZERO_ENOSPC);
  CHECK(zero_reduce_adam_step(&p, 0, rows, f, f, f, slot + 1, f, ws, wsb, &a, nullptr, 0) ==
        ZERO_EINVAL);
  zero_step_args_t bad = a;
  bad.loss_scale = 0;
  CHECK(zero_reduce_check(&p, 0, rows, &bad, f, ws, wsb, res, 0) == ZERO_EINVAL);
  bad = a;
  bad.beta1 = 1.0;
  CHECK(zero_adam_apply(&p, 0, f, f, f, f, slot, &bad, res, 0) == ZERO_EINVAL);
  CHECK(zero_reduce_adam_step_1pass(&p, 0, rows, f, f, f, f, f, f, slot, ws, wsb, &a, res, 0) ==
        ZERO_EINVAL);  // clipping requested
  zero_plan_t big = {2 * (ZERO_NOALLOC_MAX_SHARD + 8), 2, 1, ZERO_NOALLOC_MAX_SHARD + 8,
                     2 * (ZERO_NOALLOC_MAX_SHARD + 8)};
  CHECK(zero_reduce_adam_step_noalloc(&big, 0, rows, f, f, f, slot, f, &a, res, 0) == ZERO_ENOSPC);
  CHECK(zero_slot_restore(&p, 0, f, (uint16_t*)f, res, 0) == ZERO_EINVAL);
  CHECK(zero_state_bytes(4, 1, 1, 12) == -1.0 && zero_state_bytes(3, 1e9, 8, 12) == 2e9);
  zero_scaler_t s = {65536, 2, 0.5, 1, 2, 0, 0};
  for (int i = 0; i < 40; ++i) CHECK(zero_scaler_update(&s, i % 3 == 0) == ZERO_OK);
  CHECK(s.scale >= 1.0 && s.t > 0);
  CHECK(zero_scaler_update(nullptr, 0) == ZERO_EINVAL);
}

void host_adam(Rng& rng) {
  const zero_step_args_t a = good_args();
  const int widths[4] = {0, 1, 8, 16};
  const int64_t lens[6] = {0, 1, 63, 64, 1000, 70001};
  for (int64_t len : lens) {
    std::vector<float> g(len + 1), p0(len + 1), m0(len + 1), v0(len + 1);
    for (int64_t j = 0; j < len; ++j) {
      g[j] = rng.normal() * 1e-3f;
      p0[j] = rng.normal() * 0.02f;
      m0[j] = rng.normal() * 1e-4f;
      v0[j] = fabsf(rng.normal()) * 1e-7f;
    }
    std::vector<float> rp = p0, rm = m0, rv = v0;
    std::vector<uint16_t> rh(len + 1);
    CHECK(zero_host_adam_apply(g.data(), rp.data(), rm.data(), rv.data(), rh.data(), len, &a,
                               0.5f, 1, 1) == ZERO_OK);
    for (int w : widths) {
      for (int t = 1; t <= 16; ++t) {
        std::vector<float> pp = p0, mm = m0, vv = v0;
        std::vector<uint16_t> hh(len + 1);
        const int rc = zero_host_adam_apply(g.data(), pp.data(), mm.data(), vv.data(), hh.data(),
                                            len, &a, 0.5f, t, w);
        if (rc == ZERO_EINVAL && w >= 8) continue;  // the CPU lacks that width
        CHECK(rc == ZERO_OK);
        CHECK(memcmp(pp.data(), rp.data(), 4 * len) == 0);
        CHECK(memcmp(mm.data(), rm.data(), 4 * len) == 0);
        CHECK(memcmp(vv.data(), rv.data(), 4 * len) == 0);
        CHECK(memcmp(hh.data(), rh.data(), 2 * len) == 0);
      }
    }
  }
  std::vector<float> x(8);
  std::vector<uint16_t> h(8);
  CHECK(zero_host_adam_apply(x.data(), x.data(), x.data(), x.data(), h.data(), 8, &a, 0.5f, 0,
                             0) == ZERO_EINVAL);
  CHECK(zero_host_adam_apply(x.data(), x.data(), x.data(), x.data(), h.data(), 8, &a, 1.5f, 1,
                             0) == ZERO_EINVAL);
  CHECK(zero_offload_staging_bytes(64) == 64 * 2 * 6 && zero_offload_staging_bytes(65) == 0);
}

}  // namespace

int main() {
  Rng rng{0x9E3779B97F4A7C15ull};
  planner(rng);
  units(rng);
  device_call_checks();
  host_adam(rng);
  printf("host sanitize driver: %s (%d failed checks)\n", g_fail ? "FAILED" : "ok", g_fail);
  return g_fail ? 1 : 0;
}
