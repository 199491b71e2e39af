// Host side of the step: the worker pool, host memory, the CPU AdamW over the
// fp32 master state ("Technical Brief: MegaTrain's Single-GPU 120B-Parameter
// Training Breakthrough", section "Checkpointing, Manual Gradients, and
// CPU-Side Optimizer Steps": the update runs on the CPU where fp32 master
// weights and moments live), and the RoPE table.
#include <immintrin.h>
#include <sched.h>
#include <sys/mman.h>

#include <cmath>
#include <cstring>

#include "mt_ops.h"
#include "runtime.h"

namespace mt {

// ------------------------------------------------------------------ pool ---

Pool::Pool(int n) {
  for (int i = 0; i < n; ++i) workers_.emplace_back([this] { loop(); });
}

Pool::~Pool() {
  {
    std::lock_guard<std::mutex> g(mu_);
    stop_ = true;
  }
  cv_.notify_all();
  for (auto& t : workers_) t.join();
}

void Pool::submit(int64_t n, std::function<void(int64_t)> fn, std::function<void()> done, int64_t priority) {
  if (n <= 0) {
    if (done) done();
    return;
  }
  auto job = std::make_shared<Job>();
  job->fn = std::move(fn);
  job->done = std::move(done);
  job->n = n;
  job->priority = priority;
  {
    std::lock_guard<std::mutex> g(mu_);
    auto it = jobs_.begin();
    while (it != jobs_.end() && (*it)->priority <= priority) ++it;
    jobs_.insert(it, job);
  }
  cv_.notify_all();
}

void Pool::run(int64_t n, const std::function<void(int64_t)>& fn) {
  std::mutex m;
  std::condition_variable cv;
  bool finished = false;
  submit(
      n, fn,
      [&] {
        std::lock_guard<std::mutex> g(m);
        finished = true;
        cv.notify_all();
      },
      INT64_MIN);
  std::unique_lock<std::mutex> lk(m);
  cv.wait(lk, [&] { return finished; });
}

void Pool::loop() {
  for (;;) {
    std::shared_ptr<Job> job;
    int64_t i = -1;
    {
      std::unique_lock<std::mutex> lk(mu_);
      cv_.wait(lk, [&] { return stop_ || !jobs_.empty(); });
      if (stop_ && jobs_.empty()) return;
      // Urgent jobs (run()) first; then a job already under way, so that a
      // started job finishes before the next one starts; then the lowest
      // priority value. The queue is kept in priority order.
      auto pick = jobs_.begin();
      if ((*pick)->priority != INT64_MIN) {
        for (auto it = jobs_.begin(); it != jobs_.end(); ++it)
          if ((*it)->next.load() > 0) { pick = it; break; }
      }
      job = *pick;
      i = job->next.fetch_add(1);
      if (i >= job->n - 1) jobs_.erase(pick);   // the last index takes it off the queue
    }
    job->fn(i);
    if (job->finished.fetch_add(1) + 1 == job->n && job->done) job->done();
  }
}

// ---------------------------------------------------------- host memory ---

void* host_alloc_plain(size_t bytes) {
  if (bytes == 0) bytes = 64;
  void* p = mmap(nullptr, bytes, PROT_READ | PROT_WRITE, MAP_PRIVATE | MAP_ANONYMOUS | MAP_NORESERVE,
                 -1, 0);
  if (p == MAP_FAILED) return nullptr;
  madvise(p, bytes, MADV_HUGEPAGE);
  return p;
}

void host_free_plain(void* p, size_t bytes) {
  if (p) munmap(p, bytes == 0 ? 64 : bytes);
}

// ----------------------------------------------------------------- AdamW ---

AdamConst adam_const(const mt_model_cfg& c, int64_t t) {
  const double bc1 = 1.0 - std::pow(c.beta1, (double)t);
  const double bc2 = 1.0 - std::pow(c.beta2, (double)t);
  AdamConst k;
  k.decay = (float)(1.0 - c.lr * c.weight_decay);
  k.b1 = (float)c.beta1;
  k.omb1 = (float)(1.0 - c.beta1);
  k.b2 = (float)c.beta2;
  k.omb2 = (float)(1.0 - c.beta2);
  k.step_size = (float)(c.lr / bc1);
  k.inv_sqrt_bc2 = (float)(1.0 / std::sqrt(bc2));
  k.eps = (float)c.adam_eps;
  return k;
}

static inline uint16_t bf16_rne(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static inline float bf16_to_f32(uint16_t h) {
  const uint32_t u = (uint32_t)h << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// Gradients as fp32 (G16 false) or as bf16 bit patterns (G16 true, widened
// exactly; with g32 the widened values are also written out).
template <bool G16>
static inline float grad_at(const void* g, int64_t i) {
  if constexpr (G16) return bf16_to_f32(static_cast<const uint16_t*>(g)[i]);
  else return static_cast<const float*>(g)[i];
}

template <bool G16>
static inline void adamw_scalar(float* p, float* m, float* v, const void* g, int64_t i0, int64_t i1,
                                const AdamConst& k, uint16_t* bo, float* fo, float* g32) {
  for (int64_t i = i0; i < i1; ++i) {
    const float gi = grad_at<G16>(g, i);
    if (g32) g32[i] = gi;
    float pi = p[i] * k.decay;
    const float mi = m[i] * k.b1 + k.omb1 * gi;
    const float vi = v[i] * k.b2 + k.omb2 * gi * gi;
    pi -= k.step_size * mi / (std::sqrt(vi) * k.inv_sqrt_bc2 + k.eps);
    p[i] = pi;
    m[i] = mi;
    v[i] = vi;
    if (bo) bo[i] = bf16_rne(pi);
    if (fo) fo[i] = pi;
  }
}

template <bool G16>
__attribute__((target("avx512f,avx512bw,avx512vl"))) static void adamw_avx512(
    float* p, float* m, float* v, const void* g, int64_t n, const AdamConst& k, uint16_t* bo, float* fo,
    float* g32) {
  const __m512 decay = _mm512_set1_ps(k.decay), b1 = _mm512_set1_ps(k.b1),
               omb1 = _mm512_set1_ps(k.omb1), b2 = _mm512_set1_ps(k.b2),
               omb2 = _mm512_set1_ps(k.omb2), ss = _mm512_set1_ps(k.step_size),
               isb = _mm512_set1_ps(k.inv_sqrt_bc2), eps = _mm512_set1_ps(k.eps);
  const __m512i rbias = _mm512_set1_epi32(0x7FFF), one = _mm512_set1_epi32(1);
  // The bf16 image is write-only here and is next read by the DMA engine, so
  // it is written with streaming stores (no read-for-ownership of its lines).
  // Those need 32-byte aligned destinations: a short scalar head gets there.
  int64_t i = 0;
  if (bo) {
    while (i < n && (reinterpret_cast<uintptr_t>(bo + i) & 31)) ++i;
    adamw_scalar<G16>(p, m, v, g, 0, i, k, bo, fo, g32);
  }
  for (; i + 16 <= n; i += 16) {
    __m512 gi;
    if constexpr (G16) {
      const __m256i h = _mm256_loadu_si256(reinterpret_cast<const __m256i*>(static_cast<const uint16_t*>(g) + i));
      gi = _mm512_castsi512_ps(_mm512_slli_epi32(_mm512_cvtepu16_epi32(h), 16));
      if (g32) _mm512_storeu_ps(g32 + i, gi);
    } else {
      gi = _mm512_loadu_ps(static_cast<const float*>(g) + i);
    }
    __m512 pi = _mm512_mul_ps(_mm512_loadu_ps(p + i), decay);
    const __m512 mi = _mm512_add_ps(_mm512_mul_ps(_mm512_loadu_ps(m + i), b1), _mm512_mul_ps(omb1, gi));
    const __m512 vi = _mm512_add_ps(_mm512_mul_ps(_mm512_loadu_ps(v + i), b2),
                                    _mm512_mul_ps(_mm512_mul_ps(omb2, gi), gi));
    const __m512 den = _mm512_add_ps(_mm512_mul_ps(_mm512_sqrt_ps(vi), isb), eps);
    pi = _mm512_sub_ps(pi, _mm512_div_ps(_mm512_mul_ps(ss, mi), den));
    _mm512_storeu_ps(p + i, pi);
    _mm512_storeu_ps(m + i, mi);
    _mm512_storeu_ps(v + i, vi);
    if (bo) {
      const __m512i u = _mm512_castps_si512(pi);
      const __m512i r = _mm512_add_epi32(_mm512_add_epi32(u, rbias),
                                         _mm512_and_si512(_mm512_srli_epi32(u, 16), one));
      _mm256_stream_si256(reinterpret_cast<__m256i*>(bo + i), _mm512_cvtepi32_epi16(_mm512_srli_epi32(r, 16)));
    }
    if (fo) _mm512_storeu_ps(fo + i, pi);
  }
  adamw_scalar<G16>(p, m, v, g, i, n, k, bo, fo, g32);
  // streaming stores are weakly ordered: make them visible before the caller
  // reports the range done
  if (bo) _mm_sfence();
}

static bool have_avx512() {
  static const bool a = __builtin_cpu_supports("avx512f") && __builtin_cpu_supports("avx512bw") &&
                        __builtin_cpu_supports("avx512vl");
  return a;
}

void adamw_range(float* p, float* m, float* v, const float* g, int64_t n, const AdamConst& k,
                 uint16_t* bo, float* fo) {
  if (have_avx512())
    adamw_avx512<false>(p, m, v, g, n, k, bo, fo, nullptr);
  else
    adamw_scalar<false>(p, m, v, g, 0, n, k, bo, fo, nullptr);
}

void adamw_range_g16(float* p, float* m, float* v, const uint16_t* g, int64_t n, const AdamConst& k,
                     uint16_t* bo, float* fo, float* g32) {
  if (have_avx512())
    adamw_avx512<true>(p, m, v, g, n, k, bo, fo, g32);
  else
    adamw_scalar<true>(p, m, v, g, 0, n, k, bo, fo, g32);
}

void to_bf16_range(const float* x, uint16_t* y, int64_t n) {
  for (int64_t i = 0; i < n; ++i) y[i] = bf16_rne(x[i]);
}

static int online_cpus() {
  cpu_set_t s;
  if (sched_getaffinity(0, sizeof(s), &s) == 0) return CPU_COUNT(&s);
  return (int)std::thread::hardware_concurrency();
}

int default_threads(int requested) {
  int n = requested > 0 ? requested : online_cpus();
  if (n < 1) n = 1;
  if (n > 64) n = 64;
  return n;
}

}  // namespace mt

using namespace mt;

extern "C" int mt_adamw_host(float* p, float* m, float* v, const float* g, int64_t n, int64_t t,
                             double lr, double beta1, double beta2, double eps, double weight_decay,
                             uint16_t* bf16_out, int32_t threads) {
  if (!p || !m || !v || !g || n < 0 || t < 1) return MT_EINVAL;
  mt_model_cfg c{};
  c.lr = lr;
  c.beta1 = beta1;
  c.beta2 = beta2;
  c.adam_eps = eps;
  c.weight_decay = weight_decay;
  const AdamConst k = adam_const(c, t);
  const int nt = default_threads(threads);
  const int64_t chunk = 1 << 18;
  const int64_t nch = (n + chunk - 1) / chunk;
  Pool pool(nt);
  pool.run(nch, [&](int64_t i) {
    const int64_t a = i * chunk, b = std::min(n, a + chunk);
    adamw_range(p + a, m + a, v + a, g + a, b - a, k, bf16_out ? bf16_out + a : nullptr, nullptr);
  });
  return MT_OK;
}

extern "C" int mt_adamw_host_g16(float* p, float* m, float* v, const uint16_t* g16, float* g32_out, int64_t n,
                                 int64_t t, double lr, double beta1, double beta2, double eps,
                                 double weight_decay, uint16_t* bf16_out, int32_t threads) {
  if (!p || !m || !v || !g16 || n < 0 || t < 1) return MT_EINVAL;
  mt_model_cfg c{};
  c.lr = lr;
  c.beta1 = beta1;
  c.beta2 = beta2;
  c.adam_eps = eps;
  c.weight_decay = weight_decay;
  const AdamConst k = adam_const(c, t);
  const int64_t chunk = 1 << 18;
  const int64_t nch = (n + chunk - 1) / chunk;
  Pool pool(default_threads(threads));
  pool.run(nch, [&](int64_t i) {
    const int64_t a = i * chunk, b = std::min(n, a + chunk);
    adamw_range_g16(p + a, m + a, v + a, g16 + a, b - a, k, bf16_out ? bf16_out + a : nullptr, nullptr,
                    g32_out ? g32_out + a : nullptr);
  });
  return MT_OK;
}

extern "C" int mt_rope_table(int32_t T, int32_t hd, float base, float* cos_out, float* sin_out) {
  if (T < 0 || hd <= 0 || hd % 2 || !cos_out || !sin_out) return MT_EINVAL;
  const int half = hd / 2;
  for (int i = 0; i < half; ++i) {
    const double inv = std::pow((double)base, -2.0 * i / hd);
    for (int t = 0; t < T; ++t) {
      const double a = (double)t * inv;
      cos_out[(int64_t)t * half + i] = (float)std::cos(a);
      sin_out[(int64_t)t * half + i] = (float)std::sin(a);
    }
  }
  return MT_OK;
}
