// Drives the host-only runtime (the slot planner and the host-miss experts)
// through many random calls, for a build under AddressSanitizer and
// UndefinedBehaviorSanitizer.  Checks the planner's invariants after every
// call (slot_of and expert_in inverse, every selected expert placed exactly
// once, fills only into slots the call does not hold protected) and the
// host-miss partial sum against a plain scalar evaluation of the same bytes.
// Also drives the thread pool (every worker runs each job once, a spin barrier
// orders the workers' writes, idle gaps long enough for the workers to fall
// asleep, an exception on any worker reaches the caller of run()), the
// caller's first task of a host partial (runs once; an exception it throws
// surfaces after the run, whose results are complete), and the per-call
// device workspace layout (sizes, alignment, overlaps, the decode decision,
// mixed call orders on one growing arena), and the host's expert selection
// over logits with infinities, NaNs and signed zeros.
// Built under ThreadSanitizer with the argument "threads": the pool and the
// host partial only.  Exit status 0 and "ok" on success.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <functional>
#include <atomic>
#include <chrono>
#include <stdexcept>
#include <string>
#include <thread>
#include <random>
#include <set>
#include <vector>
#include <new>
#include <algorithm>

#include "../../expert_cache_host_amd/csrc/host_expert.hpp"
#include "../../expert_cache_host_amd/csrc/host_routing.hpp"
#include "../../expert_cache_host_amd/csrc/layout.hpp"
#include "../../expert_cache_host_amd/csrc/planner.hpp"
#include "../../expert_cache_host_amd/csrc/workspace.hpp"

#define CHECK(c)                                                   \
  do {                                                             \
    if (!(c)) {                                                    \
      std::fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
      std::exit(1);                                                \
    }                                                              \
  } while (0)

static void planner_runs(std::mt19937_64 &rng) {
  for (int trial = 0; trial < 60; ++trial) {
    const int E = 2 + (int)(rng() % 40), S = 1 + (int)(rng() % E), k = 1 + (int)(rng() % std::min(E, 8));
    const int policy = (int)(rng() % 2), adopt = (rng() % 3 == 0) ? -1 : (int)(rng() % 1001);
    moe::SlotPlanner p(E, S, policy, adopt);
    if (rng() % 4 == 0) {
      std::vector<uint32_t> counts(E);
      for (auto &c : counts) c = (uint32_t)(rng() % 50);
      p.preload(counts.data());
    }
    moe::CallPlan plan;
    for (int call = 0; call < 40; ++call) {
      const int T = 1 + (int)(rng() % 6), mode = (int)(rng() % 2);
      const int max_fills = mode == 1 ? (int)(rng() % 4) - 1 : -1;
      std::vector<int32_t> idx((size_t)T * k);
      for (int t = 0; t < T; ++t) {
        std::set<int32_t> used;
        for (int j = 0; j < k; ++j) {
          int32_t e;
          do e = (int32_t)(rng() % E); while (used.count(e));
          used.insert(e);
          idx[(size_t)t * k + j] = e;
        }
      }
      p.plan(idx.data(), T * k, T, mode, max_fills, plan);
      // slot_of and expert_in are inverse maps
      for (int s = 0; s < S; ++s)
        if (p.expert_in()[s] >= 0) CHECK(p.slot_of()[p.expert_in()[s]] == s);
      for (int e = 0; e < E; ++e)
        if (p.slot_of()[e] >= 0) CHECK(p.expert_in()[p.slot_of()[e]] == e);
      // every selected expert is placed exactly once over the call's tables
      std::vector<int32_t> sv(E), hv(E);
      std::vector<int> placed(E, 0);
      for (size_t s = 0; s < plan.stages.size(); ++s) {
        p.stage_view(plan, (int32_t)s, sv.data(), hv.data());
        for (int e = 0; e < E; ++e) {
          CHECK(sv[e] >= -1 && sv[e] < S);
          placed[e] += sv[e] >= 0;
          if (s == 0) placed[e] += hv[e] >= 0;
        }
      }
      std::set<int32_t> sel(idx.begin(), idx.end());
      for (int32_t e : sel) CHECK(placed[e] == 1);
      CHECK(plan.hits + plan.misses == T * k);
      if (mode == 0) CHECK((int)plan.stages.size() >= 1);
      if (max_fills >= 0) CHECK(plan.fills <= max_fills);
    }
  }
}

static float half_to_float_ref(uint16_t h) {
  const int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
  float v = e == 0 ? std::ldexp((float)m, -24) : std::ldexp((float)(m | 1024), e - 25);
  return s ? -v : v;
}

static void host_expert_runs(std::mt19937_64 &rng) {
  moe::ThreadPool pool(3);
  for (int trial = 0; trial < 8; ++trial) {
    const int64_t d = 64 * (1 + (int64_t)(rng() % 4)), f = 32 * (1 + (int64_t)(rng() % 5));
    const int T = 1 + (int)(rng() % 4), k = 2, n_jobs = 1 + (int)(rng() % 3);
    const moe::RecordLayout L = moe::RecordLayout::make(d, f);
    std::vector<std::vector<uint8_t>> recs(n_jobs, std::vector<uint8_t>((size_t)L.bytes));
    for (auto &r : recs) {
      std::vector<uint8_t> inter((size_t)L.interchange_bytes);
      for (size_t i = 0; i < inter.size(); ++i) inter[i] = (uint8_t)rng();
      for (size_t b = 0; b + 18 <= inter.size(); b += 18) {  // small finite scales
        const uint16_t sc = (uint16_t)(0x1800 + rng() % 0x400);
        std::memcpy(&inter[b], &sc, 2);
      }
      moe::repack_expert(inter.data(), L, r.data());
    }
    std::vector<float> x((size_t)T * d), w((size_t)T * k), part((size_t)T * d), h;
    std::normal_distribution<float> nd(0.f, 1.f);
    for (auto &v : x) v = nd(rng);
    std::vector<moe::HostExpertJob> jobs(n_jobs);
    std::vector<int32_t> rank((size_t)T * k, -1);
    for (int j = 0; j < n_jobs; ++j) jobs[j].record = recs[j].data();
    for (int t = 0; t < T; ++t)
      for (int j = 0; j < k; ++j) {
        const int jb = (int)(rng() % (n_jobs + 1)) - 1;  // -1: the pair is not on the host
        rank[(size_t)t * k + j] = jb;
        w[(size_t)t * k + j] = 0.5f + 0.1f * j;
        if (jb >= 0 && (jobs[jb].tokens.empty() || jobs[jb].tokens.back() != t))
          jobs[jb].tokens.push_back(t);
      }
    moe::host_moe_partial(pool, L, jobs, rank.data(), w.data(), T, k, x.data(), part.data(), h);
    // scalar reference over the same slot-layout bytes
    for (int t = 0; t < T; ++t) {
      std::vector<double> ref((size_t)d, 0.0);
      for (int j = 0; j < k; ++j) {
        const int jb = rank[(size_t)t * k + j];
        if (jb < 0) continue;
        const uint8_t *r = recs[jb].data();
        auto wgt = [&](int64_t off_q, int64_t off_s, int64_t row, int64_t nb, int64_t i) {
          const uint8_t byte = r[off_q + (row * nb + i / 32) * 16 + (i % 32) % 16];
          const int q = (i % 32) < 16 ? (byte & 15) : (byte >> 4);
          uint16_t sc;
          std::memcpy(&sc, r + off_s + (row * nb + i / 32) * 2, 2);
          return (double)half_to_float_ref(sc) * (q - 8);
        };
        std::vector<double> hh((size_t)f);
        for (int64_t rr = 0; rr < f; ++rr) {
          double g = 0, u = 0;
          for (int64_t i = 0; i < d; ++i) {
            g += wgt(L.off_gq, L.off_gs, rr, L.nb_gu, i) * x[(size_t)t * d + i];
            u += wgt(L.off_uq, L.off_us, rr, L.nb_gu, i) * x[(size_t)t * d + i];
          }
          hh[(size_t)rr] = g / (1.0 + std::exp(-g)) * u;
        }
        for (int64_t i = 0; i < d; ++i) {
          double y = 0;
          for (int64_t rr = 0; rr < f; ++rr) y += wgt(L.off_dq, L.off_ds, i, L.nb_dn, rr) * hh[(size_t)rr];
          ref[(size_t)i] += w[(size_t)t * k + j] * y;
        }
      }
      double rms = 0, err = 0;
      for (int64_t i = 0; i < d; ++i) rms += ref[(size_t)i] * ref[(size_t)i];
      rms = std::sqrt(rms / d);
      for (int64_t i = 0; i < d; ++i) err = std::max(err, std::fabs(part[(size_t)t * d + i] - ref[(size_t)i]));
      CHECK(err <= 1e-4 * rms + 1e-12);
    }
  }
}

static void pool_runs(std::mt19937_64 &rng) {
  for (int n : {1, 2, 5}) {
    moe::ThreadPool pool(n);
    for (int run = 0; run < 240; ++run) {
      std::vector<int> ran((size_t)n, 0), mark((size_t)n, 0);
      std::atomic<int> after{0};
      moe::SpinBarrier bar(pool.size());
      const int tag = (int)(rng() % 1000) + 1;
      pool.run([&](int tid) {
        ran[(size_t)tid] += 1;
        mark[(size_t)tid] = tag;  // plain writes, ordered by the barrier
        bar.arrive_and_wait();
        for (int j = 0; j < n; ++j) CHECK(mark[(size_t)j] == tag);
        after.fetch_add(1);
      });
      CHECK(after.load() == n);
      for (int j = 0; j < n; ++j) CHECK(ran[(size_t)j] == 1);
      // now and then idle past the workers' spin, so that they sleep
      if (run % 40 == 39) std::this_thread::sleep_for(std::chrono::milliseconds(2));
    }
  }
}

// The caller's first task of host_moe_partial: runs once on the calling
// thread; its exception surfaces after the run, and the partial is complete.
static void caller_first_runs(std::mt19937_64 &rng) {
  moe::ThreadPool pool(4);
  const int64_t d = 128, f = 64;
  const int T = 2, k = 2;
  const moe::RecordLayout L = moe::RecordLayout::make(d, f);
  std::vector<uint8_t> inter((size_t)L.interchange_bytes), rec((size_t)L.bytes);
  for (size_t i = 0; i < inter.size(); ++i) inter[i] = (uint8_t)rng();
  for (size_t b = 0; b + 18 <= inter.size(); b += 18) {
    const uint16_t sc = (uint16_t)(0x1800 + rng() % 0x400);
    std::memcpy(&inter[b], &sc, 2);
  }
  moe::repack_expert(inter.data(), L, rec.data());
  std::vector<float> x((size_t)T * d), w((size_t)T * k, 0.5f), a((size_t)T * d), b((size_t)T * d), h;
  std::normal_distribution<float> nd(0.f, 1.f);
  for (auto &v : x) v = nd(rng);
  std::vector<moe::HostExpertJob> jobs(1);
  jobs[0].record = rec.data();
  jobs[0].tokens = {0, 1};
  std::vector<int32_t> rank = {0, -1, -1, 0};
  moe::host_moe_partial(pool, L, jobs, rank.data(), w.data(), T, k, x.data(), a.data(), h);
  int calls = 0;
  const std::thread::id me = std::this_thread::get_id();
  const std::function<void()> first = [&]() {
    CHECK(std::this_thread::get_id() == me);
    ++calls;
  };
  moe::host_moe_partial(pool, L, jobs, rank.data(), w.data(), T, k, x.data(), b.data(), h, &first);
  CHECK(calls == 1);
  CHECK(std::memcmp(a.data(), b.data(), a.size() * 4) == 0);
  std::fill(b.begin(), b.end(), 0.0f);
  const std::function<void()> throws = [&]() { throw std::runtime_error("first task failed"); };
  bool caught = false;
  try {
    moe::host_moe_partial(pool, L, jobs, rank.data(), w.data(), T, k, x.data(), b.data(), h,
                          &throws);
  } catch (const std::runtime_error &e) {
    caught = std::string(e.what()) == "first task failed";
  }
  CHECK(caught);
  CHECK(std::memcmp(a.data(), b.data(), a.size() * 4) == 0);
}

// Workspace layouts of every call shape the cache admits along the sweep:
// tokens 1..512, several top-k, expert counts, shared experts and model shapes;
// both miss modes share the layout (the page-locked buffers are separate).
// Every layout must pass ws_check; a layout with any region shrunk by 4 bytes
// must fail it; the decode decision must match the limits it is made of; and a
// mixed sequence of calls (small after large, decode after matrix-core) must
// always find its regions inside an arena that only grows.
static void workspace_runs(std::mt19937_64 &rng) {
  const int ks[] = {1, 2, 4, 8, 15, 16, 64};
  const int Es[] = {8, 64, 128, 256, 512};
  const int shapes[][2] = {{64, 32}, {256, 512}, {2816, 704}, {2048, 768}, {6144, 2048}};
  size_t arena = 0;
  int checked = 0;
  for (int T = 1; T <= 512; T += (T < 8 ? 1 : (T < 64 ? 7 : 61))) {
    for (int k : ks)
      for (int E : Es) {
        if (k > E) continue;
        for (int ns = 0; ns <= 1; ++ns)
          for (const auto &sh : shapes) {
            const moe::WsParams p{T, E, k, ns, sh[0], sh[1]};
            const moe::WsLayout L = moe::ws_layout(p);
            const char *bad = moe::ws_check(L, p);
            if (bad) std::fprintf(stderr, "T=%d k=%d E=%d ns=%d d=%d: %s\n", T, k, E, ns, sh[0], bad);
            CHECK(bad == nullptr);
            const bool small = T <= moe::kDecodeMaxTokens && T * (k + ns) <= moe::kDecodeMaxPairs;
            CHECK(L.decode == (small && moe::gemv_lds_bytes(true, sh[0] / 32, T) <= moe::kDecodeLdsBudget &&
                               moe::gemv_lds_bytes(false, sh[1] / 32, T) <= moe::kDecodeLdsBudget));
            CHECK(L.pairs == T * k + T * ns);
            // planted mistakes: every region, shrunk, must be caught
            moe::WsRegion moe::WsLayout::*regions[] = {
                &moe::WsLayout::z,  &moe::WsLayout::idx, &moe::WsLayout::w,
                &moe::WsLayout::h,  &moe::WsLayout::y,   &moe::WsLayout::xq,
                &moe::WsLayout::xs, &moe::WsLayout::buckets, &moe::WsLayout::pair_slot,
                &moe::WsLayout::meta, &moe::WsLayout::bucket_pair, &moe::WsLayout::items,
                &moe::WsLayout::xp, &moe::WsLayout::xscale, &moe::WsLayout::hp,
                &moe::WsLayout::hscale};
            for (auto r : regions) {
              if ((L.*r).bytes < 4) continue;
              moe::WsLayout M = L;
              (M.*r).bytes -= 4;
              CHECK(moe::ws_check(M, p) != nullptr);
            }
            // an overlap is caught too
            moe::WsLayout O = L;
            O.y.off = O.h.off;
            CHECK(moe::ws_check(O, p) != nullptr);
            ++checked;
          }
      }
  }
  CHECK(checked > 1000);
  // mixed call orders on one arena
  for (int call = 0; call < 4000; ++call) {
    const int E = Es[rng() % 5];
    int k = ks[rng() % 7];
    if (k > E) k = E;
    const int T = rng() % 3 ? 1 + (int)(rng() % 4) : 1 + (int)(rng() % 512);
    const auto &sh = shapes[rng() % 5];
    const moe::WsParams p{T, E, k, (int)(rng() % 2), sh[0], sh[1]};
    const moe::WsLayout L = moe::ws_layout(p);
    CHECK(moe::ws_check(L, p) == nullptr);
    arena = std::max(arena, L.total);  // the arena grows, never shrinks
    // every region of this call lies inside the arena as it stands
    for (const moe::WsRegion *r : {&L.z, &L.idx, &L.w, &L.h, &L.y, &L.xq, &L.xs, &L.buckets,
                                   &L.pair_slot, &L.meta, &L.bucket_pair, &L.items, &L.xp,
                                   &L.xscale, &L.hp, &L.hscale})
      CHECK(r->off + r->bytes <= L.total && L.total <= arena);
  }
}

// Exceptions inside the pool: a worker's (not only the caller's) reaches the
// caller of run() once every worker has finished, and the pool keeps working.
static void pool_exception_runs() {
  for (int n : {2, 5}) {
    moe::ThreadPool pool(n);
    for (int thrower = 0; thrower < n; ++thrower) {
      std::atomic<int> done{0};
      bool caught = false;
      try {
        pool.run([&](int tid) {
          done.fetch_add(1);
          if (tid == thrower) throw std::bad_alloc();
        });
      } catch (const std::bad_alloc &) {
        caught = true;
      }
      CHECK(caught);
      CHECK(done.load() == n);
      std::atomic<int> again{0};
      pool.run([&](int) { again.fetch_add(1); });
      CHECK(again.load() == n);
    }
  }
}

// The host's selection: any float32 logits, non-finite ones included, give k
// distinct ids in range and gating weights that are finite and sum to 1 when
// every logit is finite.
static void host_topk_runs(std::mt19937_64 &rng) {
  const float specials[] = {INFINITY, -INFINITY, NAN, -NAN, 0.0f, -0.0f, 1e38f, -1e-38f};
  for (int call = 0; call < 3000; ++call) {
    const int E = 1 + (int)(rng() % 512), k = 1 + (int)(rng() % E), T = 1 + (int)(rng() % 4);
    const bool finite = rng() % 2;
    std::vector<float> z((size_t)T * E);
    std::normal_distribution<float> nd(0.0f, 3.0f);
    for (float &v : z) v = (!finite && rng() % 8 == 0) ? specials[rng() % 8] : nd(rng);
    if (finite)
      for (float &v : z)
        if (rng() % 16 == 0) v = (rng() % 2) ? 0.0f : -0.0f;
    std::vector<int32_t> idx((size_t)T * k, -1);
    std::vector<float> w((size_t)T * k, -1.0f);
    moe::host_topk(z.data(), T, E, k, (int)(rng() % 2), idx.data(), w.data());
    for (int t = 0; t < T; ++t) {
      std::set<int32_t> seen;
      double sum = 0.0;
      for (int j = 0; j < k; ++j) {
        const int32_t e = idx[(size_t)t * k + j];
        CHECK(e >= 0 && e < E);
        seen.insert(e);
        sum += w[(size_t)t * k + j];
      }
      CHECK((int)seen.size() == k);
      if (finite) CHECK(std::isfinite(sum) && sum <= 1.0 + 1e-5);
    }
  }
}

int main(int argc, char **argv) {
  std::mt19937_64 rng(12345);
  const bool threads_only = argc > 1 && std::string(argv[1]) == "threads";
  if (!threads_only) planner_runs(rng);
  if (!threads_only) workspace_runs(rng);
  if (!threads_only) host_topk_runs(rng);
  pool_runs(rng);
  pool_exception_runs();
  caller_first_runs(rng);
  if (!threads_only) host_expert_runs(rng);
  std::printf("ok\n");
  return 0;
}
