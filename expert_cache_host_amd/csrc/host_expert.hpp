// Missed experts on host cores (host miss mode), reading the page-locked arena
// in the slot layout.  The CPU computes the experts the GPU cache does not hold,
// at the same time as the GPU computes the cached ones ("How it works" step 3
// and "Overlapping the GPU and the CPU", llama.cpp + MoE expert cache).
#pragma once
#include <atomic>
#include <condition_variable>
#include <cstdint>
#include <exception>
#include <functional>
#include <mutex>
#include <thread>
#include <vector>

#include "layout.hpp"

namespace moe {

class ThreadPool {
 public:
  explicit ThreadPool(int n);
  ~ThreadPool();
  int size() const { return n_; }
  // Runs f(tid) on every worker, the caller being tid 0; returns when all ended.
  // Every worker calls f exactly once per run, so f may hold a barrier over
  // size() threads.  An exception thrown by f on any thread is rethrown here
  // once every worker has finished (the first one, if several threw).
  void run(const std::function<void(int)> &f);

 private:
  void loop(int id);
  int n_;
  std::vector<std::thread> th_;
  std::mutex m_;
  std::condition_variable cv_;
  const std::function<void(int)> *job_ = nullptr;  // published by gen_
  std::atomic<uint64_t> gen_{0};
  std::atomic<int> pending_{0};
  std::atomic<bool> stop_{false};
  std::mutex err_m_;
  std::exception_ptr err_;  // first exception of the current run
};

// Spin barrier over a fixed number of threads, for one use.
class SpinBarrier {
 public:
  explicit SpinBarrier(int n) : n_(n) {}
  void arrive_and_wait();

 private:
  const int n_;
  std::atomic<int> arrived_{0};
};

// One host-side selection: token t picked expert `expert` with weight w at rank j.
struct HostPair {
  int32_t t, j;
  float w;
};

struct HostExpertJob {
  const uint8_t *record;           // slot-layout record of the expert (host)
  std::vector<int32_t> tokens;     // distinct tokens, ascending
};

// partial[t][i] = sum over host pairs of token t, in rank order j, of
// w * y_e(x_t)[i];  tokens without host pairs get 0.
//   jobs: one per host expert; rank_expert[t*k + j] = index into jobs or -1;
//   weights[t*k + j] the gating weights.
//   caller_first: when non-null, the calling thread runs it before it joins
//   the work (the other workers start at once).
//   An exception on any thread (caller_first's, or an allocation failure of a
//   worker) is rethrown once every worker has finished; every worker still
//   passes the barrier between the gate/up and the down rows.
void host_moe_partial(ThreadPool &pool, const RecordLayout &L, const std::vector<HostExpertJob> &jobs,
                      const int32_t *rank_job, const float *weights, int32_t T, int32_t k,
                      const float *x, float *partial, std::vector<float> &h_scratch,
                      const std::function<void()> *caller_first = nullptr);

// y [T][d] = expert(x) for one record (used by moe_host_expert_forward).
void host_expert_forward(ThreadPool &pool, const RecordLayout &L, const uint8_t *record,
                         const float *x, int32_t T, float *y);

}  // namespace moe
