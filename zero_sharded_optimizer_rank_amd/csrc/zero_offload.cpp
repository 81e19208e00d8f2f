// ZeRO-Offload form of the shard step's update: the reduce, unscale, overflow
// check and norm stay on the GPU (K1), the fp32 optimizer state lives in host
// memory, the reduced gradient crosses PCIe to the host, the host runs Adam on
// it, and the fp16 parameters cross back into the rank's slot of the flat
// buffer ("10.6 ZeRO 与 FSDP" §10.6.6: forward and backward stay on the GPU,
// gradients go to the CPU over PCIe, the CPU updates the parameters and sends
// them back; its DeepSpeed configuration sets offload_optimizer to the CPU).
//
// The update is the same separately rounded fp32 sequence as the GPU kernel,
// element for element, so both forms give identical bits:
//   gc = g*c; m = b1*m + omb1*gc; v = b2*v + omb2*(gc*gc);
//   den = sqrt(v)/sqrt_bc2 + eps; u = (m/den)*step_size; p = p*decay - u
// x86 SSE/AVX arithmetic is IEEE single precision with one rounding per
// instruction; this file is built with -ffp-contract=off (no FMA), division
// and square root are the correctly rounded vdivps / vsqrtps, and every
// worker thread runs with the default MXCSR (round to nearest even,
// denormals neither flushed nor treated as zero).
#include <immintrin.h>
#include <stdint.h>
#include <string.h>

#include <condition_variable>
#include <exception>
#include <functional>
#include <memory>
#include <mutex>
#include <thread>
#include <vector>

#include <hip/hip_runtime_api.h>

#include "host_internal.h"
#include "zero_shard.h"

using namespace zk::host;

namespace {

struct Coefs {
  float c, b1, omb1, b2, omb2, eps, step_size, sqrt_bc2, decay;
};

// fp32 -> IEEE binary16 bit pattern, round to nearest even; overflow gives
// infinity, a NaN stays a quiet NaN with the top payload bits.
inline uint16_t f32_to_f16(float f) {
  uint32_t x;
  memcpy(&x, &f, 4);
  const uint32_t sign = (x >> 16) & 0x8000u;
  uint32_t ax = x & 0x7FFFFFFFu;
  if (ax >= 0x7F800000u)  // inf or NaN
    return (uint16_t)(sign | 0x7C00u | (ax > 0x7F800000u ? 0x200u | ((ax >> 13) & 0x3FFu) : 0u));
  if (ax >= 0x477FF000u) return (uint16_t)(sign | 0x7C00u);  // at or above 65520: infinity
  if (ax >= 0x38800000u) {                                    // 2^-14 and up: normal binary16
    ax += 0xFFFu + ((ax >> 13) & 1u);                         // round at bit 13, ties to even
    return (uint16_t)(sign | ((ax - 0x38000000u) >> 13));     // rebias 127 -> 15
  }
  // subnormal binary16 (or zero): the count of 2^-24 units, rounded to the
  // nearest even integer by adding and removing 2^23 under the default mode
  float t;
  memcpy(&t, &ax, 4);
  volatile float big = 8388608.0f;
  const float r = (t * 16777216.0f + big) - big;
  return (uint16_t)(sign | (uint32_t)r);
}

inline void adam_scalar(const float* g, float* p, float* m, float* v, uint16_t* h, int64_t n,
                        const Coefs& k) {
  for (int64_t i = 0; i < n; ++i) {
    const float gc = g[i] * k.c;
    const float mi = k.b1 * m[i] + k.omb1 * gc;
    const float vi = k.b2 * v[i] + k.omb2 * (gc * gc);
    const float den = __builtin_sqrtf(vi) / k.sqrt_bc2 + k.eps;
    const float u = (mi / den) * k.step_size;
    const float pi = p[i] * k.decay - u;
    m[i] = mi;
    v[i] = vi;
    p[i] = pi;
    h[i] = f32_to_f16(pi);
  }
}

__attribute__((target("avx512f"))) void adam_avx512(const float* g, float* p, float* m, float* v,
                                                     uint16_t* h, int64_t n, const Coefs& k) {
  const __m512 c = _mm512_set1_ps(k.c), b1 = _mm512_set1_ps(k.b1),
               omb1 = _mm512_set1_ps(k.omb1), b2 = _mm512_set1_ps(k.b2),
               omb2 = _mm512_set1_ps(k.omb2), eps = _mm512_set1_ps(k.eps),
               ss = _mm512_set1_ps(k.step_size), sb2 = _mm512_set1_ps(k.sqrt_bc2),
               decay = _mm512_set1_ps(k.decay);
  // the fp16 output goes to pinned staging that only the DMA engine reads
  // back: stream it past the caches when it is 32-byte aligned
  const bool stream_h = ((uintptr_t)h & 31) == 0;
  int64_t i = 0;
  for (; i + 16 <= n; i += 16) {
    const __m512 gc = _mm512_mul_ps(_mm512_loadu_ps(g + i), c);
    const __m512 mi =
        _mm512_add_ps(_mm512_mul_ps(b1, _mm512_loadu_ps(m + i)), _mm512_mul_ps(omb1, gc));
    const __m512 vi = _mm512_add_ps(_mm512_mul_ps(b2, _mm512_loadu_ps(v + i)),
                                    _mm512_mul_ps(omb2, _mm512_mul_ps(gc, gc)));
    const __m512 den = _mm512_add_ps(_mm512_div_ps(_mm512_sqrt_ps(vi), sb2), eps);
    const __m512 u = _mm512_mul_ps(_mm512_div_ps(mi, den), ss);
    const __m512 pi = _mm512_sub_ps(_mm512_mul_ps(_mm512_loadu_ps(p + i), decay), u);
    _mm512_storeu_ps(m + i, mi);
    _mm512_storeu_ps(v + i, vi);
    _mm512_storeu_ps(p + i, pi);
    const __m256i hv = _mm512_cvtps_ph(pi, _MM_FROUND_TO_NEAREST_INT | _MM_FROUND_NO_EXC);
    if (stream_h)
      _mm256_stream_si256((__m256i*)(h + i), hv);
    else
      _mm256_storeu_si256((__m256i*)(h + i), hv);
  }
  if (stream_h) _mm_sfence();  // order the streaming stores before the caller signals completion
  adam_scalar(g + i, p + i, m + i, v + i, h + i, n - i, k);
}

__attribute__((target("avx2,f16c"))) void adam_avx2(const float* g, float* p, float* m, float* v,
                                                    uint16_t* h, int64_t n, const Coefs& k) {
  const __m256 c = _mm256_set1_ps(k.c), b1 = _mm256_set1_ps(k.b1),
               omb1 = _mm256_set1_ps(k.omb1), b2 = _mm256_set1_ps(k.b2),
               omb2 = _mm256_set1_ps(k.omb2), eps = _mm256_set1_ps(k.eps),
               ss = _mm256_set1_ps(k.step_size), sb2 = _mm256_set1_ps(k.sqrt_bc2),
               decay = _mm256_set1_ps(k.decay);
  int64_t i = 0;
  for (; i + 8 <= n; i += 8) {
    const __m256 gc = _mm256_mul_ps(_mm256_loadu_ps(g + i), c);
    const __m256 mi =
        _mm256_add_ps(_mm256_mul_ps(b1, _mm256_loadu_ps(m + i)), _mm256_mul_ps(omb1, gc));
    const __m256 vi = _mm256_add_ps(_mm256_mul_ps(b2, _mm256_loadu_ps(v + i)),
                                    _mm256_mul_ps(omb2, _mm256_mul_ps(gc, gc)));
    const __m256 den = _mm256_add_ps(_mm256_div_ps(_mm256_sqrt_ps(vi), sb2), eps);
    const __m256 u = _mm256_mul_ps(_mm256_div_ps(mi, den), ss);
    const __m256 pi = _mm256_sub_ps(_mm256_mul_ps(_mm256_loadu_ps(p + i), decay), u);
    _mm256_storeu_ps(m + i, mi);
    _mm256_storeu_ps(v + i, vi);
    _mm256_storeu_ps(p + i, pi);
    _mm_storeu_si128((__m128i*)(h + i),
                     _mm256_cvtps_ph(pi, _MM_FROUND_TO_NEAREST_INT | _MM_FROUND_NO_EXC));
  }
  adam_scalar(g + i, p + i, m + i, v + i, h + i, n - i, k);
}

typedef void (*AdamFn)(const float*, float*, float*, float*, uint16_t*, int64_t, const Coefs&);

// vector_width: 0 = widest the CPU has, 1 = scalar, 8 = AVX2 + F16C, 16 = AVX-512F.
AdamFn pick(int32_t vector_width) {
  const bool has512 = __builtin_cpu_supports("avx512f");
  const bool has256 = __builtin_cpu_supports("avx2") && __builtin_cpu_supports("f16c");
  switch (vector_width) {
    case 0: return has512 ? adam_avx512 : has256 ? adam_avx2 : adam_scalar;
    case 1: return adam_scalar;
    case 8: return has256 ? adam_avx2 : nullptr;
    case 16: return has512 ? adam_avx512 : nullptr;
    default: return nullptr;
  }
}

// A fixed team of worker threads for one call; run() splits [0, n) into
// contiguous 64-element-aligned slices and returns when all are done.
class Team {
 public:
  explicit Team(int threads) : n_threads_(threads) {
    try {
      for (int t = 1; t < threads; ++t) workers_.emplace_back([this, t] { loop(t); });
    } catch (...) {
      // a thread failed to start: stop and join the ones that did before the
      // exception leaves (a joinable std::thread must not be destroyed)
      stop();
      throw;
    }
  }
  ~Team() { stop(); }
  void run(int64_t n, const std::function<void(int64_t, int64_t)>& fn) {
    {
      std::lock_guard<std::mutex> lk(mu_);
      fn_ = &fn;
      n_ = n;
      pending_ = n_threads_ - 1;
      ++gen_;
    }
    cv_.notify_all();
    slice(0);
    std::unique_lock<std::mutex> lk(mu_);
    done_.wait(lk, [this] { return pending_ == 0; });
  }

 private:
  void stop() {
    {
      std::lock_guard<std::mutex> lk(mu_);
      quit_ = true;
      ++gen_;
    }
    cv_.notify_all();
    for (auto& w : workers_)
      if (w.joinable()) w.join();
    workers_.clear();
  }
  void slice(int t) {
    const int64_t per = ((n_ + n_threads_ - 1) / n_threads_ + 63) / 64 * 64;
    const int64_t a = per * t;
    const int64_t b = a + per < n_ ? a + per : n_;
    if (a < b) (*fn_)(a, b);
  }
  void loop(int t) {
    const unsigned int saved = _mm_getcsr();
    _mm_setcsr(0x1F80u);  // round to nearest even, no flush to zero, exceptions masked
    uint64_t seen = 0;
    for (;;) {
      {
        std::unique_lock<std::mutex> lk(mu_);
        cv_.wait(lk, [&] { return gen_ != seen; });
        seen = gen_;
        if (quit_) break;
      }
      slice(t);
      {
        std::lock_guard<std::mutex> lk(mu_);
        if (--pending_ == 0) done_.notify_one();
      }
    }
    _mm_setcsr(saved);
  }

  int n_threads_;
  std::vector<std::thread> workers_;
  std::mutex mu_;
  std::condition_variable cv_, done_;
  uint64_t gen_ = 0;
  int pending_ = 0;
  bool quit_ = false;
  int64_t n_ = 0;
  const std::function<void(int64_t, int64_t)>* fn_ = nullptr;
};

// The calling thread also works; give it the default MXCSR for the call.
struct CsrGuard {
  unsigned int saved;
  CsrGuard() : saved(_mm_getcsr()) { _mm_setcsr(0x1F80u); }
  ~CsrGuard() { _mm_setcsr(saved); }
};

Coefs make_coefs(const zero_step_args_t* args, float clip_coef) {
  const zk::AdamScalars s = adam_scalars(args);
  return Coefs{clip_coef, s.b1, s.omb1, s.b2, s.omb2, s.eps, s.step_size, s.sqrt_bc2, s.decay};
}

int check_threads(int32_t threads) {
  if (threads < 1 || threads > ZERO_MAX_HOST_THREADS)
    return fail(ZERO_EINVAL, "threads %d outside 1..%d", threads, ZERO_MAX_HOST_THREADS);
  return ZERO_OK;
}

// Releases the pipeline's events on every exit path.
struct Events {
  hipEvent_t e[4] = {nullptr, nullptr, nullptr, nullptr};
  int create() {
    for (auto& x : e) {
      const int rc = (int)hipEventCreateWithFlags(&x, hipEventDisableTiming);
      if (rc != hipSuccess) return rc;
    }
    return hipSuccess;
  }
  ~Events() {
    for (auto& x : e)
      if (x) (void)hipEventDestroy(x);
  }
};

}  // namespace

extern "C" {

int zero_host_adam_apply(const float* grad, float* master, float* m, float* v,
                         uint16_t* param16, int64_t count, const zero_step_args_t* args,
                         float clip_coef, int32_t threads, int32_t vector_width) {
  g_err[0] = 0;
  int rc = check_adam_args(args);
  if (!rc) rc = check_threads(threads);
  if (rc) return rc;
  if (count < 0) return fail(ZERO_EINVAL, "count < 0");
  if (!(clip_coef > 0.0f) || !(clip_coef <= 1.0f))
    return fail(ZERO_EINVAL, "clip_coef must lie in (0, 1]");
  const AdamFn fn = pick(vector_width);
  if (!fn) return fail(ZERO_EINVAL, "vector width %d not available on this CPU", vector_width);
  if (count == 0) return ZERO_OK;
  if (!grad || !master || !m || !v || !param16) return fail(ZERO_EINVAL, "NULL array");
  const Coefs k = make_coefs(args, clip_coef);
  try {
    CsrGuard csr;
    Team team(threads);
    const std::function<void(int64_t, int64_t)> work = [&](int64_t a, int64_t b) {
      fn(grad + a, master + a, m + a, v + a, param16 + a, b - a, k);
    };
    team.run(count, work);
  } catch (const std::exception& ex) {
    return fail(ZERO_EINVAL, "host threads: %s", ex.what());
  }
  return ZERO_OK;
}

size_t zero_offload_staging_bytes(int64_t chunk) {
  if (chunk < 64 || chunk % 64) return 0;
  return (size_t)chunk * 2 * (sizeof(float) + sizeof(uint16_t));
}

int zero_offload_adam_apply(const zero_plan_t* plan, int32_t rank, const float* grad_dev,
                            float* master_host, float* m_host, float* v_host,
                            uint16_t* param16_slot_dev, const zero_step_args_t* args,
                            const zero_step_result_t* dev_result,
                            const zero_offload_staging_t* staging, int32_t threads,
                            zero_step_result_t* result_out, hipStream_t stream) {
  g_err[0] = 0;
  int rc = check_plan_rank(plan, rank);
  if (!rc) rc = check_adam_args(args);
  if (!rc) rc = check_threads(threads);
  if (rc) return rc;
  if (!dev_result) return fail(ZERO_EINVAL, "dev_result is NULL");
  if (!aligned(dev_result, 8)) return fail(ZERO_EALIGN, "dev_result not 8-byte aligned");
  if (!staging || !staging->grad_pinned || !staging->param16_pinned)
    return fail(ZERO_EINVAL, "staging buffers are NULL");
  if (staging->chunk < 64 || staging->chunk % 64)
    return fail(ZERO_EINVAL, "staging chunk %lld is not a positive multiple of 64",
                (long long)staging->chunk);
  const int64_t S = plan->shard;
  if (S > 0 && (!grad_dev || !master_host || !m_host || !v_host || !param16_slot_dev))
    return fail(ZERO_EINVAL, "NULL state pointer");
  if (S > 0 && !aligned(param16_slot_dev, 2))
    return fail(ZERO_EALIGN, "param16_slot not 2-byte aligned");
  const AdamFn fn = pick(0);
  hipStream_t up = staging->upload_stream ? staging->upload_stream : stream;

  zero_step_result_t res;
  rc = hip_status(hipMemcpyAsync(&res, dev_result, sizeof res, hipMemcpyDeviceToHost, stream),
                  "result copy");
  if (!rc) rc = hip_status(hipStreamSynchronize(stream), "result copy");
  if (rc) return rc;
  if (result_out) *result_out = res;
  if (res.skip || S == 0) return ZERO_OK;

  const Coefs k = make_coefs(args, res.clip_coef);
  const int64_t chunk = staging->chunk;
  const int64_t n_chunks = (S + chunk - 1) / chunk;
  float* gbuf[2] = {staging->grad_pinned, staging->grad_pinned + chunk};
  uint16_t* hbuf[2] = {staging->param16_pinned, staging->param16_pinned + chunk};
  // ev.e[0..1]: gradient chunk arrived (on `stream`); ev.e[2..3]: slot chunk
  // sent (on `up`, which may be a second stream so both PCIe directions run
  // at once)
  Events ev;
  rc = hip_status(ev.create(), "event create");
  if (rc) return rc;
  auto d2h = [&](int64_t i) {
    const int64_t len = (i + 1) * chunk <= S ? chunk : S - i * chunk;
    int e = (int)hipMemcpyAsync(gbuf[i & 1], grad_dev + i * chunk, (size_t)len * sizeof(float),
                                hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = (int)hipEventRecord(ev.e[i & 1], stream);
    return e;
  };
  CsrGuard csr;
  std::unique_ptr<Team> team;
  try {
    team.reset(new Team(threads));
  } catch (const std::exception& ex) {
    return fail(ZERO_EINVAL, "host threads: %s", ex.what());
  }
  int e = d2h(0);
  for (int64_t i = 0; i < n_chunks && e == hipSuccess; ++i) {
    const int64_t base = i * chunk;
    const int64_t len = base + chunk <= S ? chunk : S - base;
    if (i + 1 < n_chunks) e = d2h(i + 1);  // its buffer was consumed in iteration i - 1
    if (e == hipSuccess) e = (int)hipEventSynchronize(ev.e[i & 1]);
    if (e == hipSuccess && i >= 2) e = (int)hipEventSynchronize(ev.e[2 + (i & 1)]);
    if (e != hipSuccess) break;
    const float* g = gbuf[i & 1];
    uint16_t* h = hbuf[i & 1];
    const std::function<void(int64_t, int64_t)> work = [&](int64_t a, int64_t b) {
      fn(g + a, master_host + base + a, m_host + base + a, v_host + base + a, h + a, b - a, k);
    };
    team->run(len, work);
    e = (int)hipMemcpyAsync(param16_slot_dev + base, h, (size_t)len * sizeof(uint16_t),
                            hipMemcpyHostToDevice, up);
    if (e == hipSuccess) e = (int)hipEventRecord(ev.e[2 + (i & 1)], up);
  }
  int es = (int)hipStreamSynchronize(stream);
  if (e == hipSuccess) e = es;
  if (up != stream) {
    es = (int)hipStreamSynchronize(up);
    if (e == hipSuccess) e = es;
  }
  return hip_status(e, "offload pipeline");
}

int zero_offload_step(const zero_plan_t* plan, int32_t rank, const uint16_t* const* contrib,
                      float* grad_dev, void* workspace, size_t ws_bytes, float* master_host,
                      float* m_host, float* v_host, uint16_t* param16_slot_dev,
                      const zero_step_args_t* args, zero_step_result_t* dev_result,
                      const zero_offload_staging_t* staging, int32_t threads,
                      zero_step_result_t* result_out, hipStream_t stream) {
  g_err[0] = 0;
  int rc = check_adam_args(args);
  if (!rc) rc = check_threads(threads);
  if (rc) return rc;
  rc = zero_reduce_check(plan, rank, contrib, args, grad_dev, workspace, ws_bytes, dev_result,
                         stream);
  if (rc) return rc;
  return zero_offload_adam_apply(plan, rank, grad_dev, master_host, m_host, v_host,
                                 param16_slot_dev, args, dev_result, staging, threads, result_out,
                                 stream);
}

}  // extern "C"
