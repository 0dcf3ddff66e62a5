#include "host_expert.hpp"

#include <immintrin.h>

#include <algorithm>
#include <chrono>
#include <cmath>
#include <cstring>
#include <exception>

namespace moe {

// ---------------------------------------------------------------- thread pool
// Decode calls come every few hundred microseconds, and waking a sleeping
// thread through the kernel costs tens of microseconds on a virtual machine.
// So workers spin (with pause and yield, leaving the core to any other
// runnable thread) for a while after each job before they sleep on the
// condition variable, and the caller spins for the end of a run.

namespace {
constexpr auto kSpinFor = std::chrono::microseconds(250);

inline void relax(unsigned &i) {
  _mm_pause();
  if ((++i & 63u) == 0) std::this_thread::yield();
}
}  // namespace

ThreadPool::ThreadPool(int n) : n_(std::max(1, n)) {
  for (int i = 1; i < n_; ++i) th_.emplace_back([this, i] { loop(i); });
}

ThreadPool::~ThreadPool() {
  {
    std::lock_guard<std::mutex> g(m_);
    stop_.store(true);
  }
  cv_.notify_all();
  for (auto &t : th_) t.join();
}

void ThreadPool::run(const std::function<void(int)> &f) {
  if (n_ == 1) {
    f(0);
    return;
  }
  {
    std::lock_guard<std::mutex> g(m_);
    job_ = &f;
    pending_.store(n_ - 1, std::memory_order_relaxed);
    gen_.fetch_add(1, std::memory_order_release);
  }
  cv_.notify_all();  // only sleeping workers need it
  std::exception_ptr mine;
  try {
    f(0);
  } catch (...) {
    mine = std::current_exception();
  }
  unsigned i = 0;
  while (pending_.load(std::memory_order_acquire) != 0) relax(i);
  std::exception_ptr e;
  {
    std::lock_guard<std::mutex> g(err_m_);
    e = err_ ? err_ : mine;
    err_ = nullptr;
  }
  if (e) std::rethrow_exception(e);
}

void ThreadPool::loop(int id) {
  uint64_t seen = 0;
  for (;;) {
    auto t0 = std::chrono::steady_clock::now();
    unsigned i = 0;
    while (gen_.load(std::memory_order_acquire) == seen && !stop_.load(std::memory_order_relaxed)) {
      relax(i);
      if ((i & 255u) == 0 && std::chrono::steady_clock::now() - t0 > kSpinFor) {
        std::unique_lock<std::mutex> lk(m_);
        cv_.wait(lk, [&] { return stop_.load() || gen_.load() != seen; });
        t0 = std::chrono::steady_clock::now();
      }
    }
    if (stop_.load()) return;
    seen = gen_.load(std::memory_order_acquire);
    try {
      (*job_)(id);
    } catch (...) {
      std::lock_guard<std::mutex> g(err_m_);
      if (!err_) err_ = std::current_exception();
    }
    pending_.fetch_sub(1, std::memory_order_release);
  }
}

void SpinBarrier::arrive_and_wait() {
  arrived_.fetch_add(1, std::memory_order_acq_rel);
  unsigned i = 0;
  while (arrived_.load(std::memory_order_acquire) < n_) relax(i);
}

// ---------------------------------------------------------------- row dots

static inline float half_to_float(uint16_t h) {
  uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
  uint32_t exp = (h >> 10) & 0x1Fu, mant = h & 0x3FFu, x;
  if (exp == 0) {
    if (mant == 0) {
      x = sign;
    } else {
      exp = 127 - 15 + 1;
      while (!(mant & 0x400u)) {
        mant <<= 1;
        exp--;
      }
      x = sign | (exp << 23) | ((mant & 0x3FFu) << 13);
    }
  } else if (exp == 31) {
    x = sign | 0x7F800000u | (mant << 13);
  } else {
    x = sign | ((exp - 15 + 127) << 23) | (mant << 13);
  }
  float f;
  std::memcpy(&f, &x, 4);
  return f;
}

// sum_b d_b * sum_i (q_i - 8) * x_i over nb blocks of one row (portable).
static float row_dot_scalar(const uint8_t *q, const uint16_t *s, const float *x, int64_t nb) {
  float acc = 0.0f;
  for (int64_t b = 0; b < nb; ++b) {
    const uint8_t *qb = q + 16 * b;
    const float *xb = x + 32 * b;
    float dot = 0.0f;
    for (int j = 0; j < 16; ++j) {
      dot += (float)((int)(qb[j] & 15) - 8) * xb[j];
      dot += (float)((int)(qb[j] >> 4) - 8) * xb[j + 16];
    }
    acc += half_to_float(s[b]) * dot;
  }
  return acc;
}

__attribute__((target("avx2,fma,f16c"))) static float row_dot_avx2(const uint8_t *q,
                                                                    const uint16_t *s,
                                                                    const float *x, int64_t nb) {
  const __m128i m4 = _mm_set1_epi8(0x0F);
  const __m256 eight = _mm256_set1_ps(8.0f);
  __m256 acc = _mm256_setzero_ps();
  for (int64_t b = 0; b < nb; ++b) {
    const __m128i raw = _mm_loadu_si128((const __m128i *)(q + 16 * b));
    const __m128i lo = _mm_and_si128(raw, m4);
    const __m128i hi = _mm_and_si128(_mm_srli_epi16(raw, 4), m4);
    const float *xb = x + 32 * b;
    const __m256 x0 = _mm256_loadu_ps(xb), x1 = _mm256_loadu_ps(xb + 8);
    const __m256 x2 = _mm256_loadu_ps(xb + 16), x3 = _mm256_loadu_ps(xb + 24);
    const __m256 q0 = _mm256_cvtepi32_ps(_mm256_cvtepu8_epi32(lo));
    const __m256 q1 = _mm256_cvtepi32_ps(_mm256_cvtepu8_epi32(_mm_srli_si128(lo, 8)));
    const __m256 q2 = _mm256_cvtepi32_ps(_mm256_cvtepu8_epi32(hi));
    const __m256 q3 = _mm256_cvtepi32_ps(_mm256_cvtepu8_epi32(_mm_srli_si128(hi, 8)));
    __m256 dot = _mm256_mul_ps(q0, x0);
    dot = _mm256_fmadd_ps(q1, x1, dot);
    dot = _mm256_fmadd_ps(q2, x2, dot);
    dot = _mm256_fmadd_ps(q3, x3, dot);
    const __m256 xs = _mm256_add_ps(_mm256_add_ps(x0, x1), _mm256_add_ps(x2, x3));
    dot = _mm256_fnmadd_ps(eight, xs, dot);
    const __m256 d = _mm256_cvtph_ps(_mm_set1_epi16((short)s[b]));
    acc = _mm256_fmadd_ps(d, dot, acc);
  }
  __m128 a = _mm_add_ps(_mm256_castps256_ps128(acc), _mm256_extractf128_ps(acc, 1));
  a = _mm_add_ps(a, _mm_movehl_ps(a, a));
  a = _mm_add_ss(a, _mm_shuffle_ps(a, a, 0x55));
  return _mm_cvtss_f32(a);
}

// 512-bit form: the 32 nibbles become signed bytes q - 8, sign-extended to two
// vectors of 16 int32 and converted; two multiply-adds per block, then the
// block scale in one more.  No correction term is needed.
__attribute__((target("avx512f"))) static float row_dot_avx512(const uint8_t *q,
                                                                const uint16_t *s,
                                                                const float *x, int64_t nb) {
  const __m128i m4 = _mm_set1_epi8(0x0F), b8 = _mm_set1_epi8(8);
  __m512 acc0 = _mm512_setzero_ps(), acc1 = _mm512_setzero_ps();
  int64_t b = 0;
  for (; b + 1 < nb; b += 2) {
    // two blocks per iteration, independent chains
    const __m128i r0 = _mm_loadu_si128((const __m128i *)(q + 16 * b));
    const __m128i r1 = _mm_loadu_si128((const __m128i *)(q + 16 * b + 16));
    const __m128i lo0 = _mm_sub_epi8(_mm_and_si128(r0, m4), b8);
    const __m128i hi0 = _mm_sub_epi8(_mm_and_si128(_mm_srli_epi16(r0, 4), m4), b8);
    const __m128i lo1 = _mm_sub_epi8(_mm_and_si128(r1, m4), b8);
    const __m128i hi1 = _mm_sub_epi8(_mm_and_si128(_mm_srli_epi16(r1, 4), m4), b8);
    const float *xb = x + 32 * b;
    __m512 d0 = _mm512_mul_ps(_mm512_cvtepi32_ps(_mm512_cvtepi8_epi32(lo0)), _mm512_loadu_ps(xb));
    d0 = _mm512_fmadd_ps(_mm512_cvtepi32_ps(_mm512_cvtepi8_epi32(hi0)), _mm512_loadu_ps(xb + 16), d0);
    __m512 d1 = _mm512_mul_ps(_mm512_cvtepi32_ps(_mm512_cvtepi8_epi32(lo1)), _mm512_loadu_ps(xb + 32));
    d1 = _mm512_fmadd_ps(_mm512_cvtepi32_ps(_mm512_cvtepi8_epi32(hi1)), _mm512_loadu_ps(xb + 48), d1);
    const __m512 s0 = _mm512_cvtph_ps(_mm256_set1_epi16((short)s[b]));
    const __m512 s1 = _mm512_cvtph_ps(_mm256_set1_epi16((short)s[b + 1]));
    acc0 = _mm512_fmadd_ps(s0, d0, acc0);
    acc1 = _mm512_fmadd_ps(s1, d1, acc1);
  }
  for (; b < nb; ++b) {
    const __m128i r0 = _mm_loadu_si128((const __m128i *)(q + 16 * b));
    const __m128i lo0 = _mm_sub_epi8(_mm_and_si128(r0, m4), b8);
    const __m128i hi0 = _mm_sub_epi8(_mm_and_si128(_mm_srli_epi16(r0, 4), m4), b8);
    const float *xb = x + 32 * b;
    __m512 d0 = _mm512_mul_ps(_mm512_cvtepi32_ps(_mm512_cvtepi8_epi32(lo0)), _mm512_loadu_ps(xb));
    d0 = _mm512_fmadd_ps(_mm512_cvtepi32_ps(_mm512_cvtepi8_epi32(hi0)), _mm512_loadu_ps(xb + 16), d0);
    acc0 = _mm512_fmadd_ps(_mm512_cvtph_ps(_mm256_set1_epi16((short)s[b])), d0, acc0);
  }
  return _mm512_reduce_add_ps(_mm512_add_ps(acc0, acc1));
}

static bool have_avx2() {
  static const bool v = __builtin_cpu_supports("avx2") && __builtin_cpu_supports("fma") &&
                        __builtin_cpu_supports("f16c");
  return v;
}

static bool have_avx512() {
  static const bool v = __builtin_cpu_supports("avx512f");
  return v;
}

static inline float row_dot(const uint8_t *q, const uint16_t *s, const float *x, int64_t nb) {
  if (have_avx512()) return row_dot_avx512(q, s, x, nb);
  return have_avx2() ? row_dot_avx2(q, s, x, nb) : row_dot_scalar(q, s, x, nb);
}

static inline float silu(float v) { return v / (1.0f + std::exp(-v)); }

// ---------------------------------------------------------------- layer part

static constexpr int64_t kRowChunk = 32;

void host_moe_partial(ThreadPool &pool, const RecordLayout &L, const std::vector<HostExpertJob> &jobs,
                      const int32_t *rank_job, const float *weights, int32_t T, int32_t k,
                      const float *x, float *partial, std::vector<float> &h,
                      const std::function<void()> *caller_first) {
  const int64_t d = L.d, f = L.f;
  // h rows: one per (job, token) in job order
  std::vector<int64_t> h_base(jobs.size() + 1, 0);
  for (size_t i = 0; i < jobs.size(); ++i) h_base[i + 1] = h_base[i] + (int64_t)jobs[i].tokens.size();
  h.resize((size_t)(h_base.back() * f));
  // token t, rank j -> row of h (or -1)
  std::vector<int64_t> pair_row((size_t)T * k, -1);
  for (int32_t t = 0; t < T; ++t)
    for (int32_t j = 0; j < k; ++j) {
      const int32_t jb = rank_job[t * k + j];
      if (jb < 0) continue;
      const auto &tk = jobs[jb].tokens;
      const int64_t pos = std::lower_bound(tk.begin(), tk.end(), t) - tk.begin();
      pair_row[(size_t)t * k + j] = h_base[jb] + pos;
    }

  // One run of the pool: gate/up rows (chunks of kRowChunk rows of one job),
  // a barrier (down needs every row of h), then down rows; every output
  // element summed in rank order.
  const int64_t chunks_f = (f + kRowChunk - 1) / kRowChunk;
  const int64_t total1 = chunks_f * (int64_t)jobs.size();
  const int64_t chunks_d = (d + kRowChunk - 1) / kRowChunk;
  std::atomic<int64_t> next1{0}, next2{0};
  SpinBarrier h_done(pool.size());
  std::mutex err_m;
  std::exception_ptr first_err;
  auto keep = [&](std::exception_ptr e) {
    std::lock_guard<std::mutex> g(err_m);
    if (!first_err) first_err = e;
  };
  pool.run([&](int tid) {
    if (tid == 0 && caller_first) {
      try {
        (*caller_first)();
      } catch (...) {
        keep(std::current_exception());
      }
    }
    try {
      for (;;) {
        const int64_t u = next1.fetch_add(1);
        if (u >= total1) break;
        const int64_t jb = u / chunks_f, r0 = (u % chunks_f) * kRowChunk;
        const int64_t r1 = std::min(f, r0 + kRowChunk);
        const uint8_t *rec = jobs[jb].record;
        const auto &toks = jobs[jb].tokens;
        for (int64_t r = r0; r < r1; ++r) {
          const uint8_t *gq = rec + L.off_gq + r * L.nb_gu * 16;
          const uint8_t *uq = rec + L.off_uq + r * L.nb_gu * 16;
          const uint16_t *gs = (const uint16_t *)(rec + L.off_gs) + r * L.nb_gu;
          const uint16_t *us = (const uint16_t *)(rec + L.off_us) + r * L.nb_gu;
          for (size_t ti = 0; ti < toks.size(); ++ti) {
            const float *xt = x + (int64_t)toks[ti] * d;
            const float g = row_dot(gq, gs, xt, L.nb_gu);
            const float uu = row_dot(uq, us, xt, L.nb_gu);
            h[(size_t)((h_base[jb] + (int64_t)ti) * f + r)] = silu(g) * uu;
          }
        }
      }
    } catch (...) {
      keep(std::current_exception());
    }
    h_done.arrive_and_wait();
    try {
      std::vector<float> dots((size_t)h_base.back());
      for (;;) {
        const int64_t u = next2.fetch_add(1);
        if (u >= chunks_d) break;
        const int64_t i0 = u * kRowChunk, i1 = std::min(d, i0 + kRowChunk);
        for (int64_t i = i0; i < i1; ++i) {
          for (size_t jb = 0; jb < jobs.size(); ++jb) {
            const uint8_t *rec = jobs[jb].record;
            const uint8_t *dq = rec + L.off_dq + i * L.nb_dn * 16;
            const uint16_t *ds = (const uint16_t *)(rec + L.off_ds) + i * L.nb_dn;
            for (int64_t r = h_base[jb]; r < h_base[jb + 1]; ++r)
              dots[(size_t)r] = row_dot(dq, ds, h.data() + r * f, L.nb_dn);
          }
          for (int32_t t = 0; t < T; ++t) {
            float acc = 0.0f;
            for (int32_t j = 0; j < k; ++j) {
              const int64_t r = pair_row[(size_t)t * k + j];
              if (r >= 0) acc += weights[t * k + j] * dots[(size_t)r];
            }
            partial[(int64_t)t * d + i] = acc;
          }
        }
      }
    } catch (...) {
      keep(std::current_exception());
    }
  });
  if (first_err) std::rethrow_exception(first_err);
}

void host_expert_forward(ThreadPool &pool, const RecordLayout &L, const uint8_t *record,
                         const float *x, int32_t T, float *y) {
  std::vector<HostExpertJob> jobs(1);
  jobs[0].record = record;
  for (int32_t t = 0; t < T; ++t) jobs[0].tokens.push_back(t);
  std::vector<int32_t> rank_job((size_t)T, 0);
  std::vector<float> w((size_t)T, 1.0f);
  std::vector<float> h;
  host_moe_partial(pool, L, jobs, rank_job.data(), w.data(), T, 1, x, y, h);
}

}  // namespace moe
