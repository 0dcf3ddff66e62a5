// C ABI of libmoecache (declared in include/moe_cache.h).
//
// Per layer: a page-locked host arena holding every expert in the slot layout,
// a device arena of (slots + n_shared) records, an LRU planner and the record
// of its last call.  One side stream carries slot fills; the caller's stream
// carries the compute.  The copy protocol follows "Keeping the cache fresh"
// (llama.cpp + MoE expert cache): a slot leaves the table before its copy and
// is published after it, so no kernel ever reads a half-copied expert.  Here
// the publication points are fixed (stream mode: before the stage that needs
// the slot; host mode: the same layer's next call), which makes every table a
// deterministic function of the routing history.
#include <hip/hip_runtime_api.h>
#include <rocprofiler-sdk-roctx/roctx.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cstdio>
#include <cstring>
#include <memory>
#include <new>
#include <optional>
#include <stdexcept>
#include <string>
#include <thread>
#include <type_traits>
#include <vector>

#include "../../include/moe_cache.h"
#include "host_expert.hpp"
#include "host_routing.hpp"
#include "kernels.hpp"
#include "layout.hpp"
#include "planner.hpp"
#include "workspace.hpp"

// The header's stream type is HIP's own (no HIP header needed there).
static_assert(std::is_same<moe_stream_t, hipStream_t>::value, "moe_stream_t must be hipStream_t");

namespace {

thread_local std::string g_err;

moe_status fail(moe_status st, const std::string &msg) {
  g_err = msg;
  return st;
}

// A named range of host time for tracing tools (rocprofv3 --marker-trace):
// the call, the wait for the routing, the plan, the fill enqueue, the
// host-miss experts.  Costs a few nanoseconds when no tool is attached.
struct TraceRange {
  explicit TraceRange(const char *name) { roctxRangePushA(name); }
  ~TraceRange() { roctxRangePop(); }
  TraceRange(const TraceRange &) = delete;
  TraceRange &operator=(const TraceRange &) = delete;
};

struct HipError : std::runtime_error {
  using std::runtime_error::runtime_error;
};

// A device or page-locked allocation failed: MOE_ENOMEM, and the cache (if
// any) stays usable, since every allocation precedes the work that needs it.
struct AllocError : std::runtime_error {
  using std::runtime_error::runtime_error;
};

// Failure injection for tests (moe_debug_fail_alloc): the allocation this many
// allocations from now fails as if the device were out of memory (-1: none).
thread_local int64_t g_fail_alloc_in = -1;

bool injected_alloc_failure() {
  if (g_fail_alloc_in < 0) return false;
  if (g_fail_alloc_in-- > 0) return false;
  g_fail_alloc_in = -1;
  return true;
}

hipError_t dev_malloc(void **p, size_t n) {
  if (injected_alloc_failure()) return hipErrorOutOfMemory;
  return hipMalloc(p, n);
}

hipError_t host_malloc(void **p, size_t n, unsigned flags) {
  if (injected_alloc_failure()) return hipErrorOutOfMemory;
  return hipHostMalloc(p, n, flags);
}

#define ALLOCCHK(expr, what)                                                              \
  do {                                                                                    \
    hipError_t e_ = (expr);                                                               \
    if (e_ != hipSuccess) {                                                               \
      (void)hipGetLastError();                                                            \
      throw AllocError(std::string(what) + ": " + hipGetErrorString(e_));                 \
    }                                                                                     \
  } while (0)

#define HIPCHK(expr)                                                                      \
  do {                                                                                    \
    hipError_t e_ = (expr);                                                               \
    if (e_ != hipSuccess)                                                                 \
      throw HipError(std::string(#expr) + ": " + hipGetErrorString(e_));                  \
  } while (0)

double now_s() {
  return std::chrono::duration<double>(std::chrono::steady_clock::now().time_since_epoch())
      .count();
}

int default_threads() {
  unsigned n = std::thread::hardware_concurrency();
  return n > 1 ? (int)n - 1 : 1;
}

struct PinnedBuf {
  void *p = nullptr;
  size_t bytes = 0;
  void ensure(size_t n) {
    if (n <= bytes) return;
    if (p) (void)hipHostFree(p);
    p = nullptr;
    bytes = 0;
    ALLOCCHK(host_malloc(&p, n, hipHostMallocDefault), "page-locked buffer");
    bytes = n;
  }
  ~PinnedBuf() {
    if (p) (void)hipHostFree(p);
  }
};

struct DevBuf {
  void *p = nullptr;
  size_t bytes = 0;
  void ensure(size_t n) {
    if (n <= bytes) return;
    if (p) (void)hipFree(p);
    p = nullptr;
    bytes = 0;
    ALLOCCHK(dev_malloc(&p, n), "device buffer");
    bytes = n;
  }
  ~DevBuf() {
    if (p) (void)hipFree(p);
  }
};

// Pairs of timing events, summed on demand.
// One timed span: from `start` to `stop`, or, when `before` is set too, from
// the later of the two starts (see KTime).
struct TimedSpan {
  hipEvent_t start, stop, before;
};

struct TimingLog {
  std::vector<TimedSpan> pending;
  std::vector<hipEvent_t> free_list;
  double total = 0.0;
  hipEvent_t get() {
    if (!free_list.empty()) {
      hipEvent_t e = free_list.back();
      free_list.pop_back();
      return e;
    }
    // timing only: no system-scope fence (no cache writeback / invalidate
    // around the timed work); these events order nothing
    hipEvent_t e;
    HIPCHK(hipEventCreateWithFlags(&e, hipEventDisableSystemFence));
    return e;
  }
  void put_back(hipEvent_t e) {
    if (e) free_list.push_back(e);
  }
  void add(hipEvent_t start, hipEvent_t stop, hipEvent_t before = nullptr) {
    pending.push_back({start, stop, before});
  }
  void collect() {
    for (const TimedSpan &sp : pending) {
      HIPCHK(hipEventSynchronize(sp.stop));
      float ms = 0.f;
      HIPCHK(hipEventElapsedTime(&ms, sp.start, sp.stop));
      if (sp.before) {
        float mb = 0.f;
        HIPCHK(hipEventElapsedTime(&mb, sp.before, sp.stop));
        ms = std::min(ms, mb);
      }
      total += ms * 1e-3;
      put_back(sp.start);
      put_back(sp.stop);
      put_back(sp.before);
    }
    pending.clear();
  }
  ~TimingLog() {
    for (const TimedSpan &sp : pending)
      for (hipEvent_t e : {sp.start, sp.stop, sp.before})
        if (e) (void)hipEventDestroy(e);
    for (auto e : free_list) (void)hipEventDestroy(e);
  }
};

}  // namespace

// Copy streams the slot fills rotate over (each keeps a copy engine busy).
constexpr int kCopyStreams = 2;

struct LayerState {
  std::unique_ptr<moe::SlotPlanner> planner;
  uint8_t *d_slots = nullptr;     // (S + n_shared) records
  hipEvent_t fill_ev[kCopyStreams] = {};  // last fills of this layer (side streams)
  bool fill_used[kCopyStreams] = {};
  // host mode: recorded on the compute stream at the end of each call, after
  // its readers of the layer's slots
  hipEvent_t read_done = nullptr;
  bool read_done_set = false;
  bool fill_pending = false;
  moe::CallPlan plan;             // last call
  int32_t last_T = 0;
  std::vector<int32_t> last_idx;
  std::vector<float> last_w;
  std::vector<float> dbg_host;    // keep_debug: host partial
  DevBuf dbg_gpu;                 // keep_debug: GPU partial
  DevBuf dbg_z;                   // keep_debug: router logits
  moe_stats st{};
  TimingLog t_gpu, t_h2d;
};

struct KernelTiming {
  TimingLog log;
  int64_t launches = 0;
  double bytes = 0.0;
};

struct moe_cache {
  int32_t L = 0, E = 0, S = 0, d = 0, f = 0;
  KernelTiming kt[MOE_K_COUNT];
  moe_cache_opts o{};
  moe::RecordLayout lay;
  int device = 0;
  uint8_t *h_arena = nullptr;   // L * (E + n_shared) records, page-locked
  std::vector<LayerState> layers;
  hipStream_t side[kCopyStreams] = {};  // slot fills rotate over the copy streams
  int fill_rr = 0;                      // copy stream of the next fill
  hipEvent_t ev_idx = nullptr, ev_ready = nullptr;
  int32_t fill_delay_us = 0;  // moe_debug_fill_delay: host wait before each fill batch
  // decode calls: the router publishes every logit here as (seq << 32) | bits
  // (page-locked, coherent, [kDecodeMaxTokens][E]); the host selects from it
  uint64_t *h_z = nullptr;
  uint32_t z_seq = 0;
  bool poisoned = false;
  bool timing = false;   // per-layer compute and fill events
  uint32_t kmask = 0;    // kernels timed one launch at a time (bit MOE_K_*)
  // device workspace of moe_layer_forward (grown on demand) and the fixed
  // scratch array of moe_layer_forward_noalloc on this device
  DevBuf arena;
  void *scratch = nullptr;
  // stream of the last call: the workspace above is shared by every layer
  hipStream_t last_stream = nullptr;
  bool called = false;
  // pinned host staging
  PinnedBuf h_idx, h_w, h_x, partial[2];
  hipEvent_t partial_ev[2] = {nullptr, nullptr};
  bool partial_used[2] = {false, false};
  int partial_cur = 0;
  std::vector<float> h_scratch;
  std::vector<float> h_zf;  // the published logits as floats
  // host-mode bookkeeping, reused across calls
  std::vector<moe::HostExpertJob> jobs;
  std::vector<int32_t> job_of, rank_job;
  std::unique_ptr<moe::ThreadPool> pool;

  size_t rec() const { return (size_t)lay.bytes; }
  moe::WsParams ws_params(int32_t T) const { return {T, E, o.top_k, o.n_shared, d, f}; }
  int32_t n_total() const { return E + o.n_shared; }
  const uint8_t *host_record(int32_t l, int32_t e) const {
    return h_arena + ((size_t)l * n_total() + e) * rec();
  }
  uint8_t *dev_slot(int32_t l, int32_t s) const { return layers[l].d_slots + (size_t)s * rec(); }

  ~moe_cache() {
    (void)hipSetDevice(device);
    for (auto sd : side)
      if (sd) (void)hipStreamSynchronize(sd);
    (void)hipDeviceSynchronize();
    for (auto &ly : layers) {
      if (ly.d_slots) (void)hipFree(ly.d_slots);
      for (auto &e : ly.fill_ev)
        if (e) (void)hipEventDestroy(e);
      if (ly.read_done) (void)hipEventDestroy(ly.read_done);
    }
    layers.clear();
    if (h_arena) (void)hipHostFree(h_arena);
    if (h_z) (void)hipHostFree(h_z);
    if (ev_idx) (void)hipEventDestroy(ev_idx);
    if (ev_ready) (void)hipEventDestroy(ev_ready);
    for (auto &e : partial_ev)
      if (e) (void)hipEventDestroy(e);
    for (auto sd : side)
      if (sd) (void)hipStreamDestroy(sd);
  }

  // Page-locked buffers of a call of T tokens: the routing copy and, in host
  // mode, the x copy and the two alternating host partials.
  bool pinned_fits(int32_t T) const {
    const size_t nk = (size_t)T * o.top_k * 4, nx = (size_t)T * d * 4;
    if (h_idx.bytes < nk || h_w.bytes < nk) return false;
    if (o.miss_mode == MOE_MISS_HOST)
      return h_x.bytes >= nx && partial[0].bytes >= nx && partial[1].bytes >= nx;
    return true;
  }
  // Grows them (waiting for the device first: earlier calls may still use them).
  void ensure_pinned(int32_t T) {
    if (pinned_fits(T)) return;
    HIPCHK(hipDeviceSynchronize());
    const size_t nk = (size_t)T * o.top_k * 4, nx = (size_t)T * d * 4;
    h_idx.ensure(nk);
    h_w.ensure(nk);
    if (o.miss_mode == MOE_MISS_HOST) {
      h_x.ensure(nx);
      for (auto &pb : partial) pb.ensure(nx);
    }
  }
  void ensure_arena(size_t bytes) {
    if (bytes <= arena.bytes) return;
    HIPCHK(hipDeviceSynchronize());
    arena.ensure(bytes);
  }
};

namespace {

// Device pointers of one call's workspace, carved from `base` by its layout.
struct Ws {
  void *z, *idx, *w, *h, *y;
  void *xq, *xs, *buckets, *pair_slot;
  void *meta, *bucket_pair, *items, *xp, *xscale, *hp, *hscale;
};

Ws carve(void *base, const moe::WsLayout &L) {
  auto at = [&](const moe::WsRegion &r) -> void * {
    return r.bytes ? (void *)((uint8_t *)base + r.off) : nullptr;
  };
  return Ws{at(L.z),    at(L.idx),         at(L.w),     at(L.h),  at(L.y),
            at(L.xq),   at(L.xs),          at(L.buckets), at(L.pair_slot),
            at(L.meta), at(L.bucket_pair), at(L.items), at(L.xp), at(L.xscale),
            at(L.hp),   at(L.hscale)};
}

moe::SlotView make_view(const std::vector<int32_t> &table) {
  moe::SlotView v;
  for (int i = 0; i < moe::kMaxExperts; ++i) v.slot[i] = -1;
  for (size_t e = 0; e < table.size(); ++e) v.slot[e] = (int16_t)table[e];
  return v;
}

// Event pair around one kernel launch (timing on only).
// Times the one kernel launched between construction and end().  The launch
// records `a` at its dispatch start and `b` at its end (set_launch_events);
// the GPU stamps `a` when it takes up the launch, which is before the launch
// has waited for earlier work on the stream when there is any.  `w`, recorded
// on the stream just before the launch, completes when that earlier work
// does, but on an idle stream it is stamped before the host has finished
// submitting the launch.  Both are lower bounds of the kernel's start, each
// tight in the case where the other is not, so the span runs from the later
// of the two to `b`.
struct KTime {
  moe_cache *c;
  int kid;
  hipEvent_t w = nullptr, a = nullptr, b = nullptr;
  KTime(moe_cache *c_, int kid_, hipStream_t st) : c(c_), kid(kid_) {
    if (c->kmask & (1u << kid)) {
      TimingLog &lg = c->kt[kid].log;
      try {
        w = lg.get();
        a = lg.get();
        b = lg.get();
        HIPCHK(hipEventRecord(w, st));
      } catch (...) {  // the destructor does not run for a throwing constructor
        release();
        throw;
      }
      moe::set_launch_events(a, b);
    }
  }
  void release() {
    TimingLog &lg = c->kt[kid].log;
    for (hipEvent_t e : {w, a, b})
      if (e) lg.put_back(e);
    w = a = b = nullptr;
  }
  void end(double bytes) {
    if (!a) return;
    if (moe::launch_events_pending()) {  // nothing was launched: the events go back
      release();
      return;
    }
    c->kt[kid].log.add(a, b, w);
    c->kt[kid].launches++;
    c->kt[kid].bytes += bytes;
    w = a = b = nullptr;
  }
  ~KTime() {
    if (a) {  // left by an exception: no later launch may take the pair
      (void)moe::launch_events_pending();
      release();
    }
  }
};

// Waits until the router has published every logit of the call (each word of
// h_z carries z_seq), then selects the call's experts and gating weights on the
// host into h_idx / h_w.  A stream that went idle without them, or 30 s
// without them, is an error rather than a hang.
void wait_routing(moe_cache *c, hipStream_t st, int32_t T) {
  const uint32_t want = c->z_seq;
  const int64_t n = (int64_t)T * c->E;
  const double t0 = now_s();
  int64_t ready = 0;  // words 0..ready-1 seen with the call's number
  for (uint64_t i = 0;; ++i) {
    while (ready < n && (uint32_t)(__atomic_load_n(c->h_z + ready, __ATOMIC_ACQUIRE) >> 32) == want)
      ++ready;
    if (ready == n) break;
    if ((i & 4095) == 4095) {
      const hipError_t e = hipStreamQuery(st);
      if (e != hipSuccess && e != hipErrorNotReady) HIPCHK(e);
      if (e == hipSuccess) {
        while (ready < n &&
               (uint32_t)(__atomic_load_n(c->h_z + ready, __ATOMIC_ACQUIRE) >> 32) == want)
          ++ready;
        if (ready == n) break;
        throw HipError("router logits missing after the call's kernels completed");
      }
      if (now_s() - t0 > 30.0) throw HipError("router logits not published within 30 s");
    }
    __builtin_ia32_pause();
  }
  float *z = c->h_zf.data();
  for (int64_t i = 0; i < n; ++i) {
    const uint32_t b = (uint32_t)c->h_z[i];
    std::memcpy(&z[i], &b, 4);
  }
  moe::host_topk(z, T, c->E, c->o.top_k, c->o.norm_topk, (int32_t *)c->h_idx.p,
                 (float *)c->h_w.p);
}

// Copies the fills of one stage on the side streams after every earlier reader
// of the victim slots (all of them are on `st`: see the stream rule at the top
// of a call), and records the layer's fill events.  Staged calls wait for the
// work enqueued so far on `st` (a stage's victims may be the previous stage's
// slots).  Host-mode calls (after_prev_call) wait only for the layer's previous
// call and fills: no slot a call reads is its own victim, so the copies need
// not wait for the call's own kernels.
// Host function on a copy stream (moe_debug_fill_delay): holds the stream.
void hold_fills(void *us) {
  std::this_thread::sleep_for(std::chrono::microseconds(*static_cast<const int32_t *>(us)));
}

void enqueue_fills(moe_cache *c, int32_t layer, const std::vector<moe::Fill> &fills,
                   hipStream_t st, bool after_prev_call = false) {
  LayerState &ly = c->layers[layer];
  if (!after_prev_call) HIPCHK(hipEventRecord(c->ev_ready, st));
  // the calls' fills rotate over the copy streams (a call's first fill takes
  // the stream after the previous call's last one), so that every copy engine
  // stays loaded
  const int n_sd = (int)std::min<size_t>(fills.size(), kCopyStreams);
  const int r0 = c->fill_rr;
  c->fill_rr = (int)((c->fill_rr + fills.size()) % kCopyStreams);
  auto phys = [&](int i) { return (r0 + i) % kCopyStreams; };  // i-th stream of this call
  hipEvent_t t0 = nullptr, t1 = nullptr;
  for (int i = 0; i < n_sd; ++i) {
    hipStream_t sd = c->side[phys(i)];
    if (!after_prev_call) {
      HIPCHK(hipStreamWaitEvent(sd, c->ev_ready, 0));
      continue;
    }
    if (ly.read_done_set) HIPCHK(hipStreamWaitEvent(sd, ly.read_done, 0));
    for (int p = 0; p < kCopyStreams; ++p)
      if (ly.fill_used[p] && p != phys(i)) HIPCHK(hipStreamWaitEvent(sd, ly.fill_ev[p], 0));
  }
  if (c->fill_delay_us > 0) {
    // a slow link, forced from the host: each copy stream holds its copies
    // back this long; nothing that reads a slot may get ahead of its copy
    for (int i = 0; i < n_sd; ++i)
      HIPCHK(hipLaunchHostFunc(c->side[phys(i)], hold_fills, &c->fill_delay_us));
  }
  if (c->timing) {
    t0 = ly.t_h2d.get();
    t1 = ly.t_h2d.get();
    HIPCHK(hipEventRecord(t0, c->side[phys(0)]));
    for (int i = 1; i < n_sd; ++i) HIPCHK(hipStreamWaitEvent(c->side[phys(i)], t0, 0));
  }
  for (size_t i = 0; i < fills.size(); ++i) {
    const moe::Fill &fl = fills[i];
    HIPCHK(hipMemcpyAsync(c->dev_slot(layer, fl.slot), c->host_record(layer, fl.expert), c->rec(),
                          hipMemcpyHostToDevice, c->side[phys((int)(i % n_sd))]));
  }
  for (int p = 0; p < kCopyStreams; ++p) ly.fill_used[p] = false;
  for (int i = 0; i < n_sd; ++i) {
    ly.fill_used[phys(i)] = true;
    HIPCHK(hipEventRecord(ly.fill_ev[phys(i)], c->side[phys(i)]));
  }
  if (c->timing) {
    for (int i = 1; i < n_sd; ++i)
      HIPCHK(hipStreamWaitEvent(c->side[phys(0)], ly.fill_ev[phys(i)], 0));
    HIPCHK(hipEventRecord(t1, c->side[phys(0)]));
    ly.t_h2d.add(t0, t1);
  }
  ly.st.fills += fills.size();
  ly.st.fill_bytes += fills.size() * (uint64_t)c->rec();
}

void wait_fills(moe_cache *c, LayerState &ly, hipStream_t st) {
  for (int i = 0; i < kCopyStreams; ++i)
    if (ly.fill_used[i]) HIPCHK(hipStreamWaitEvent(st, ly.fill_ev[i], 0));
}

// Gate/up + SwiGLU and down for the pairs whose expert `view` maps to a slot
// (plus the shared expert's pairs when with_shared), into h and y.  The decode
// path (few tokens) lets each workgroup find its bucket; larger batches bucket
// once with the remap kernel.  work_experts: experts read (byte counters).
void run_experts(moe_cache *c, int32_t layer, int32_t T, const moe::SlotView &view,
                 bool with_shared, int n_buckets, double work_experts, const float *x,
                 hipStream_t st, const Ws &ws, const moe::WsLayout &WL,
                 const moe::BucketTable *tab = nullptr) {
  if (n_buckets <= 0) return;
  const int32_t k = c->o.top_k;
  const int shared_slot = with_shared ? c->S : -1;
  const int P = T * k + (with_shared ? T : 0);
  // the layout was checked against every launch of the call (ws_check)
  const bool decode = WL.decode;
  if (tab && !decode) throw HipError("host-built buckets need the decode path");
  const moe::RecordLayout &L = c->lay;
  moe::GemvArgs a{};
  if (!decode && !tab) {
    KTime kt(c, MOE_K_REMAP, st);
    HIPCHK(moe::launch_remap((const int32_t *)ws.idx, T, k, view, shared_slot,
                             c->S + c->o.n_shared, (int32_t *)ws.meta,
                             (int32_t *)ws.bucket_pair, (int32_t *)ws.items, st));
    kt.end((double)P * 8);
    a.meta = (const int32_t *)ws.meta;
    a.bucket_pair = (const int32_t *)ws.bucket_pair;
    a.items = (const int32_t *)ws.items;
  }
  a.slots = c->layers[layer].d_slots;
  a.bt = decode && !tab ? (const int32_t *)ws.buckets : nullptr;
  a.xq = (const uint4 *)ws.xq;
  a.xs = (const float *)ws.xs;
  a.xp = (const uint32_t *)ws.xp;
  a.xscale = (const float *)ws.xscale;
  a.rec_bytes = L.bytes;
  a.T = T;
  a.k = k;
  a.idx = (const int32_t *)ws.idx;
  a.shared_slot = shared_slot;
  // gate/up + SwiGLU: rows f, K = d, input = prepared x by token
  a.off_q0 = L.off_gq;
  a.off_s0 = L.off_gs;
  a.off_q1 = L.off_uq;
  a.off_s1 = L.off_us;
  a.rows = c->f;
  a.nb = (int)L.nb_gu;
  a.in = x;
  a.in_by_pair = 0;
  a.out = (float *)ws.h;
  if (!decode && !tab) {
    // matrix-core grouped GEMM: gate/up + SwiGLU, h -> binary16 pairs, down;
    // one grid column per work item (bucket, token pass), bounded from above
    const int n_items = moe::gemm_items_bound(std::min(n_buckets, c->S + c->o.n_shared), P);
    {
      KTime kt(c, MOE_K_GATEUP, st);
      HIPCHK(moe::launch_mfma(a, true, n_items, st));
      kt.end(work_experts * 2.0 * (double)c->f * (double)L.nb_gu * 18.0);
    }
    const int P_all = T * k + T * c->o.n_shared;
    {
      KTime kt(c, MOE_K_PREP, st);
      HIPCHK(moe::launch_prep_pairs((const float *)ws.h, P_all, c->f, (uint32_t *)ws.hp,
                                    (float *)ws.hscale, st));
      kt.end((double)P_all * c->f * 8.0);
    }
    moe::GemvArgs b = a;
    b.off_q0 = L.off_dq;
    b.off_s0 = L.off_ds;
    b.rows = c->d;
    b.nb = (int)L.nb_dn;
    b.xp = (const uint32_t *)ws.hp;
    b.xscale = (const float *)ws.hscale;
    b.in_by_pair = 1;
    b.out = (float *)ws.y;
    {
      KTime kt(c, MOE_K_DOWN, st);
      HIPCHK(moe::launch_mfma(b, false, n_items, st));
      kt.end(work_experts * (double)c->d * (double)L.nb_dn * 18.0);
    }
    return;
  }
  moe::GemvShape sh1 = moe::choose_gemv(true, a.nb, T);
  {
    KTime kt(c, MOE_K_GATEUP, st);
    HIPCHK(moe::launch_gemv(a, tab, sh1, true, n_buckets, st));
    kt.end(work_experts * 2.0 * (double)c->f * (double)L.nb_gu * 18.0);
  }
  // down: rows d, K = f, input = h by pair
  moe::GemvArgs b = a;
  b.off_q0 = L.off_dq;
  b.off_s0 = L.off_ds;
  b.rows = c->d;
  b.nb = (int)L.nb_dn;
  b.in = (const float *)ws.h;
  b.in_by_pair = 1;
  b.out = (float *)ws.y;
  moe::GemvShape sh2 = moe::choose_gemv(false, b.nb, T);
  {
    KTime kt(c, MOE_K_DOWN, st);
    HIPCHK(moe::launch_gemv(b, tab, sh2, false, n_buckets, st));
    kt.end(work_experts * (double)c->d * (double)L.nb_dn * 18.0);
  }
}

// One layer call.  noalloc: the workspace is the fixed scratch array and
// nothing is allocated (the caller checked that the call fits); else the
// cache's arena and page-locked buffers grow as needed.
moe_status forward_impl(moe_cache *c, int32_t layer, const float *x, int32_t T,
                        const float *router_w, const float *router_bias, float *out,
                        hipStream_t st, bool noalloc = false) {
  LayerState &ly = c->layers[layer];
  const int32_t k = c->o.top_k, E = c->E, d = c->d;
  const bool host_mode = c->o.miss_mode == MOE_MISS_HOST;
  const int ns = c->o.n_shared;
  const moe::WsParams wp = c->ws_params(T);
  const moe::WsLayout WL = moe::ws_layout(wp);
  if (const char *bad = moe::ws_check(WL, wp))
    throw HipError(std::string("workspace region ") + bad + " does not cover the call");
  void *base;
  if (noalloc) {
    if (WL.total > moe::kNoAllocScratchBytes || !c->pinned_fits(T) || !c->scratch)
      throw HipError("call does not fit the fixed scratch");
    base = c->scratch;
  } else {
    c->ensure_pinned(T);
    c->ensure_arena(WL.total);
    base = c->arena.p;
  }
  const Ws ws = carve(base, WL);
  // Stream rule: slot fills (the pull kernel on `st`, copies after an event on
  // `st`) rely on every earlier reader of the victims being before them on
  // `st`, and every layer's calls share the cache's workspace (logits, planes,
  // bucket list, partial results).  A call on another stream than the cache's
  // last call therefore waits for the device first (rare; keeps the usual
  // path free of markers).
  if (c->called && c->last_stream != st) HIPCHK(hipDeviceSynchronize());
  c->last_stream = st;
  c->called = true;
  std::optional<TraceRange> enqueue_range;
  enqueue_range.emplace("moe.enqueue");
  hipEvent_t g0 = nullptr, g1 = nullptr;
  if (c->timing) {
    g0 = ly.t_gpu.get();
    g1 = ly.t_gpu.get();
    HIPCHK(hipEventRecord(g0, st));
  }
  // publication of the previous call's fills (host mode)
  if (ly.fill_pending) {
    wait_fills(c, ly, st);
    ly.fill_pending = false;
  }
  // table published at call start: the hits run on it before the host plans
  const moe::SlotView pre = make_view(ly.planner->slot_of());
  const bool dec = WL.decode;
  // host mode: the host experts read x from page-locked memory; the decode
  // router writes that copy itself, else a copy on the stream does
  const bool router_x = host_mode && dec && moe::router_decode_fits(T, d, E);
  if (host_mode && !router_x)
    HIPCHK(hipMemcpyAsync(c->h_x.p, x, (size_t)T * d * 4, hipMemcpyDeviceToHost, st));
  if (dec) {
    // router with the digit planes of the decode GEMV, then the decode top-k
    KTime kt(c, MOE_K_ROUTER, st);
    moe::DecodeTopk a;
    a.k = k;
    a.norm_topk = c->o.norm_topk;
    a.idx = (int32_t *)ws.idx;
    a.w = (float *)ws.w;
    a.view = pre;
    a.shared_slot = ns > 0 ? c->S : -1;
    a.buckets = (int32_t *)ws.buckets;
    a.pair_slot = (int32_t *)ws.pair_slot;
    // a new number for every call: words left from earlier calls never match
    if (++c->z_seq == 0) ++c->z_seq;
    HIPCHK(moe::launch_router(x, T, d, router_w, router_bias, E, (float *)ws.z, nullptr,
                              nullptr, (uint4 *)ws.xq, (float *)ws.xs, st,
                              router_x ? (float *)c->h_x.p : nullptr,
                              (unsigned long long *)c->h_z, c->z_seq));
    kt.end(4.0 * ((double)E * d + (double)T * d * 2 + (double)T * E + (router_bias ? E : 0)));
    KTime kt2(c, MOE_K_TOPK, st);
    HIPCHK(moe::launch_topk_decode((const float *)ws.z, T, E, a, st));
    kt2.end(4.0 * ((double)T * E + 4.0 * T * k));
  } else {
    {
      KTime kt(c, MOE_K_ROUTER, st);
      // the matrix-core GEMM takes binary16 pairs
      HIPCHK(moe::launch_router(x, T, d, router_w, router_bias, E, (float *)ws.z,
                                (uint32_t *)ws.xp, (float *)ws.xscale, nullptr,
                                (float *)ws.xs, st));
      kt.end(4.0 * ((double)E * d + (double)T * d * 2 + (double)T * E + (router_bias ? E : 0)));
    }
    KTime kt(c, MOE_K_TOPK, st);
    HIPCHK(moe::launch_topk((const float *)ws.z, T, E, k, c->o.norm_topk, (int32_t *)ws.idx,
                            (float *)ws.w, (int32_t *)c->h_idx.p, (float *)c->h_w.p, st));
    kt.end(4.0 * ((double)T * E + 4.0 * T * k));
  }
  if (!dec) HIPCHK(hipEventRecord(c->ev_idx, st));
  if (c->o.keep_debug) {
    ly.dbg_z.ensure((size_t)T * E * 4);
    HIPCHK(hipMemcpyAsync(ly.dbg_z.p, ws.z, (size_t)T * E * 4, hipMemcpyDeviceToDevice, st));
  }

  // Cached experts (and the shared one) on the table published at call start,
  // enqueued before the host reads the routing.
  const int nb_hits = std::min(T * k, c->S) + (ns > 0 ? 1 : 0);
  run_experts(c, layer, T, pre, ns > 0, nb_hits, 0.0, x, st, ws, WL);
  enqueue_range.reset();

  float *dbg_gpu = nullptr;
  if (c->o.keep_debug) {
    ly.dbg_gpu.ensure((size_t)T * d * 4);
    dbg_gpu = (float *)ly.dbg_gpu.p;
  }
  {
    TraceRange tr("moe.wait_routing");
    if (dec)
      wait_routing(c, st, T);
    else
      HIPCHK(hipEventSynchronize(c->ev_idx));
  }
  const double tp = now_s();
  {
    TraceRange tr("moe.plan");
    ly.planner->plan((const int32_t *)c->h_idx.p, T * k, T, host_mode ? 1 : 0,
                     host_mode ? c->o.max_fills_per_call : -1, ly.plan);
  }
  ly.st.plan_s += now_s() - tp;
  if (c->kmask & ((1u << MOE_K_GATEUP) | (1u << MOE_K_DOWN))) {
    const double n_hit = (double)(ly.plan.stages[0].members.size() -
                                  (host_mode ? 0 : ly.plan.stages[0].fills.size())) + ns;
    if (c->kmask & (1u << MOE_K_GATEUP))
      c->kt[MOE_K_GATEUP].bytes += n_hit * 2.0 * (double)c->f * (double)c->lay.nb_gu * 18.0;
    if (c->kmask & (1u << MOE_K_DOWN))
      c->kt[MOE_K_DOWN].bytes += n_hit * (double)c->d * (double)c->lay.nb_dn * 18.0;
  }
  bool combined = false;
  if (!host_mode && WL.decode) {
    // every miss is pulled from the pinned arena into its slot by a copy kernel
    // on the compute stream (after every earlier reader of the victims), then
    // computed there from host-built buckets
    const int32_t *hidx = (const int32_t *)c->h_idx.p;
    for (size_t s = 0; s < ly.plan.stages.size(); ++s) {
      const moe::PlanStage &stg = ly.plan.stages[s];
      for (size_t f0 = 0; f0 < stg.fills.size(); f0 += moe::kTabMax) {
        moe::BucketTable tab;
        moe::PullList pl;
        tab.n = 0;
        for (size_t f = f0; f < stg.fills.size() && tab.n < moe::kTabMax; ++f) {
          const moe::Fill &fl = stg.fills[f];
          const int b = tab.n++;
          pl.src[b] = c->host_record(layer, fl.expert);
          pl.dst[b] = c->dev_slot(layer, fl.slot);
          tab.src[b] = c->dev_slot(layer, fl.slot);
          int cnt = 0;
          for (int32_t p = 0; p < T * k; ++p)
            if (hidx[p] == fl.expert) tab.pairs[b][cnt++] = (uint8_t)p;
          tab.cnt[b] = (uint8_t)cnt;
          for (int i = cnt; i < moe::kDecodeMaxTokens; ++i) tab.pairs[b][i] = tab.pairs[b][0];
        }
        pl.n = tab.n;
        pl.per_expert = 32;
        pl.bytes16 = (long long)c->rec() / 16;
        {
          TraceRange tr("moe.fill_pull");
          KTime kt(c, MOE_K_FILL, st);
          HIPCHK(moe::launch_pull(pl, st));
          kt.end((double)pl.n * (double)c->rec());
        }
        run_experts(c, layer, T, pre, false, tab.n, (double)tab.n, x, st, ws, WL, &tab);
      }
      ly.st.fills += stg.fills.size();
      ly.st.fill_bytes += stg.fills.size() * (uint64_t)c->rec();
    }
    if (c->o.keep_debug) ly.dbg_host.assign((size_t)T * d, 0.0f);
  } else if (!host_mode) {
    // every miss is streamed into a slot, stage by stage, then computed there
    std::vector<int32_t> table(E, -1);
    for (size_t s = 0; s < ly.plan.stages.size(); ++s) {
      const moe::PlanStage &stg = ly.plan.stages[s];
      if (stg.fills.empty()) continue;
      {
        TraceRange tr("moe.fill_copies");
        enqueue_fills(c, layer, stg.fills, st);
      }
      wait_fills(c, ly, st);
      std::fill(table.begin(), table.end(), -1);
      for (const moe::Fill &fl : stg.fills) table[fl.expert] = fl.slot;
      const int nb = (int)stg.fills.size();
      run_experts(c, layer, T, make_view(table), false, nb, (double)nb, x, st, ws, WL);
    }
    if (c->o.keep_debug) ly.dbg_host.assign((size_t)T * d, 0.0f);
  } else {
    // Fills land at the layer's next call, so the calling thread enqueues
    // them while the other workers start on the missed experts.
    const moe::PlanStage &stg = ly.plan.stages[0];
    const std::function<void()> fills = [&]() {
      if (stg.fills.empty()) return;
      TraceRange tr("moe.fill_copies");
      enqueue_fills(c, layer, stg.fills, st, true);
      ly.fill_pending = true;
    };
    if (ly.plan.host_experts.empty()) fills();
    if (!ly.plan.host_experts.empty()) {
      const double th = now_s();
      const int b = c->partial_cur;
      c->partial_cur ^= 1;
      if (c->partial_used[b]) HIPCHK(hipEventSynchronize(c->partial_ev[b]));
      // host jobs: one per missed expert, its tokens ascending (the cache's
      // vectors, reused from call to call)
      std::vector<moe::HostExpertJob> &jobs = c->jobs;
      std::vector<int32_t> &job_of = c->job_of, &rank_job = c->rank_job;
      jobs.resize(ly.plan.host_experts.size());
      job_of.assign(E, -1);
      for (size_t i = 0; i < jobs.size(); ++i) {
        const int32_t e = ly.plan.host_experts[i];
        job_of[e] = (int32_t)i;
        jobs[i].record = c->host_record(layer, e);
        jobs[i].tokens.clear();
      }
      const int32_t *hidx = (const int32_t *)c->h_idx.p;
      rank_job.assign((size_t)T * k, -1);
      for (int32_t t = 0; t < T; ++t)
        for (int32_t j = 0; j < k; ++j) {
          const int32_t jb = job_of[hidx[t * k + j]];
          rank_job[(size_t)t * k + j] = jb;
          if (jb >= 0) jobs[jb].tokens.push_back(t);
        }
      {
        TraceRange tr("moe.host_experts");
        moe::host_moe_partial(*c->pool, c->lay, jobs, rank_job.data(), (const float *)c->h_w.p, T,
                              k, (const float *)c->h_x.p, (float *)c->partial[b].p, c->h_scratch,
                              &fills);
      }
      const float *host_part = (const float *)c->partial[b].p;
      if (c->o.keep_debug) ly.dbg_host.assign(host_part, host_part + (size_t)T * d);
      ly.st.host_s += now_s() - th;
      ly.st.host_selections += ly.plan.misses;
      {
        TraceRange tr("moe.combine");
        KTime kt(c, MOE_K_COMBINE, st);
        HIPCHK(moe::launch_combine((const float *)ws.y, (const float *)ws.w,
                                   (const int32_t *)ws.idx, pre, 0,
                                   dec ? (const int32_t *)ws.pair_slot : nullptr, T, k, d, ns,
                                   host_part, out, dbg_gpu, st));
        kt.end(4.0 * (double)T * d * (k + ns + 2));
      }
      HIPCHK(hipEventRecord(c->partial_ev[b], st));
      c->partial_used[b] = true;
      combined = true;
    } else if (c->o.keep_debug) {
      ly.dbg_host.assign((size_t)T * d, 0.0f);
    }
  }
  if (!combined) {
    TraceRange tr("moe.combine");
    KTime kt(c, MOE_K_COMBINE, st);
    HIPCHK(moe::launch_combine((const float *)ws.y, (const float *)ws.w,
                               (const int32_t *)ws.idx, pre, host_mode ? 0 : 1,
                               dec ? (const int32_t *)ws.pair_slot : nullptr, T, k, d, ns,
                               nullptr, out, dbg_gpu, st));
    kt.end(4.0 * (double)T * d * (k + ns + 1));
  }
  if (host_mode) {
    // the layer's next fills start after this call's readers of its slots
    HIPCHK(hipEventRecord(ly.read_done, st));
    ly.read_done_set = true;
  }
  if (c->timing) {
    HIPCHK(hipEventRecord(g1, st));
    ly.t_gpu.add(g0, g1);
  }
  // record of the call
  ly.last_T = T;
  ly.last_idx.assign((const int32_t *)c->h_idx.p, (const int32_t *)c->h_idx.p + (size_t)T * k);
  ly.last_w.assign((const float *)c->h_w.p, (const float *)c->h_w.p + (size_t)T * k);
  moe_stats &s = ly.st;
  s.calls++;
  s.tokens += T;
  s.selections += (uint64_t)T * k;
  s.hits += ly.plan.hits;
  s.misses += ly.plan.misses;
  s.unique += ly.plan.unique;
  s.evictions += ly.plan.evictions;
  s.stages += ly.plan.stages.size();
  return MOE_OK;
}

template <class F>
moe_status guarded(moe_cache *c, F &&f) {
  if (c && c->poisoned) return fail(MOE_ESTATE, "cache poisoned by an earlier HIP failure");
  try {
    if (c) HIPCHK(hipSetDevice(c->device));
    return f();
  } catch (const HipError &e) {
    if (c) c->poisoned = true;
    return fail(MOE_EHIP, e.what());
  } catch (const AllocError &e) {
    return fail(MOE_ENOMEM, e.what());
  } catch (const std::bad_alloc &) {
    return fail(MOE_ENOMEM, "host allocation failed");
  } catch (const std::exception &e) {
    return fail(MOE_EINVAL, e.what());
  }
}

}  // namespace

extern "C" {

void moe_cache_default_opts(moe_cache_opts *o) {
  if (!o) return;
  std::memset(o, 0, sizeof(*o));
  o->top_k = 8;
  o->miss_mode = MOE_MISS_STREAM;
  o->n_shared = 0;
  o->norm_topk = 1;
  o->host_threads = 0;
  o->max_fills_per_call = -1;
  o->keep_debug = 0;
  o->preheat = 0;
  o->adopt = 1000;
}

const char *moe_last_error(void) { return g_err.c_str(); }

int64_t moe_slot_bytes(int32_t d_model, int32_t d_ff) {
  if (d_model <= 0 || d_ff <= 0 || d_model % 64 || d_ff % 32) return 0;
  return moe::RecordLayout::make(d_model, d_ff).bytes;
}

moe_status moe_cache_create(int32_t layers, int32_t n_experts, int32_t slots, int32_t d_model,
                            int32_t d_ff, const void *host_q4_weights, const moe_cache_opts *opts,
                            moe_cache **out) {
  g_err.clear();
  if (!out) return fail(MOE_EINVAL, "out is NULL");
  *out = nullptr;
  moe_cache_opts o;
  moe_cache_default_opts(&o);
  if (opts) o = *opts;
  if (layers < 1) return fail(MOE_EINVAL, "layers must be >= 1");
  if (n_experts < 1 || n_experts > MOE_MAX_EXPERTS)
    return fail(MOE_EINVAL, "n_experts must be in [1, 512]");
  if (slots < 1 || slots > n_experts) return fail(MOE_EINVAL, "slots must be in [1, n_experts]");
  if (d_model <= 0 || d_model % 64) return fail(MOE_EINVAL, "d_model must be a positive multiple of 64");
  if (d_ff <= 0 || d_ff % 32) return fail(MOE_EINVAL, "d_ff must be a positive multiple of 32");
  if (!host_q4_weights) return fail(MOE_EINVAL, "host_q4_weights is NULL");
  if (o.top_k < 1 || o.top_k > n_experts || o.top_k > MOE_MAX_TOPK)
    return fail(MOE_EINVAL, "top_k must be in [1, min(n_experts, 64)]");
  if (o.miss_mode != MOE_MISS_STREAM && o.miss_mode != MOE_MISS_HOST)
    return fail(MOE_EINVAL, "miss_mode must be MOE_MISS_STREAM or MOE_MISS_HOST");
  if (o.n_shared < 0 || o.n_shared > 1) return fail(MOE_EINVAL, "n_shared must be 0 or 1");
  if (o.norm_topk != 0 && o.norm_topk != 1) return fail(MOE_EINVAL, "norm_topk must be 0 or 1");
  if (o.max_fills_per_call < -1) return fail(MOE_EINVAL, "max_fills_per_call must be >= -1");
  if (o.keep_debug != 0 && o.keep_debug != 1) return fail(MOE_EINVAL, "keep_debug must be 0 or 1");
  if (o.timing != 0 && o.timing != 1) return fail(MOE_EINVAL, "timing must be 0 or 1");
  if (o.policy != MOE_POLICY_LRU && o.policy != MOE_POLICY_SCORE)
    return fail(MOE_EINVAL, "policy must be MOE_POLICY_LRU or MOE_POLICY_SCORE");
  if (o.preheat != 0 && o.preheat != 1) return fail(MOE_EINVAL, "preheat must be 0 or 1");
  if (o.adopt < 0 || o.adopt > 1000) return fail(MOE_EINVAL, "adopt must be in [0, 1000]");
  for (int i = 0; i < 5; ++i)
    if (o.reserved[i] != 0) return fail(MOE_EINVAL, "reserved fields must be 0");

  std::unique_ptr<moe_cache> c;
  try {
    c.reset(new moe_cache());
  } catch (const std::bad_alloc &) {
    return fail(MOE_ENOMEM, "host allocation failed");
  }
  c->L = layers;
  c->E = n_experts;
  c->S = slots;
  c->d = d_model;
  c->f = d_ff;
  c->o = o;
  c->timing = o.timing != 0;
  c->kmask = o.timing ? (1u << MOE_K_COUNT) - 1u : 0u;
  c->lay = moe::RecordLayout::make(d_model, d_ff);
  moe_status rc = guarded(nullptr, [&]() -> moe_status {
    HIPCHK(hipGetDevice(&c->device));
    const size_t ntot = (size_t)n_experts + o.n_shared;
    const size_t arena = (size_t)layers * ntot * c->rec();
    if (host_malloc((void **)&c->h_arena, arena, hipHostMallocDefault) != hipSuccess) {
      c->h_arena = nullptr;
      (void)hipGetLastError();
      return fail(MOE_ENOMEM, "page-locked host arena allocation failed");
    }
    const int nthr = o.host_threads > 0 ? o.host_threads : default_threads();
    c->pool.reset(new moe::ThreadPool(nthr));
    {
      const uint8_t *src = (const uint8_t *)host_q4_weights;
      const size_t total = (size_t)layers * ntot;
      const size_t ib = (size_t)c->lay.interchange_bytes;
      std::atomic<size_t> next{0};
      moe::RecordLayout lay = c->lay;
      uint8_t *dst = c->h_arena;
      const size_t rb = c->rec();
      c->pool->run([&](int) {
        for (;;) {
          const size_t i = next.fetch_add(1);
          if (i >= total) break;
          moe::repack_expert(src + i * ib, lay, dst + i * rb);
        }
      });
    }
    for (auto &sd : c->side) HIPCHK(hipStreamCreateWithFlags(&sd, hipStreamNonBlocking));
    HIPCHK(hipEventCreateWithFlags(&c->ev_idx, hipEventDisableTiming));
    HIPCHK(hipEventCreateWithFlags(&c->ev_ready, hipEventDisableTiming));
    // completion only (the host or the copy streams wait for readers to finish):
    // no system-scope fence
    for (auto &e : c->partial_ev)
      HIPCHK(hipEventCreateWithFlags(&e, hipEventDisableTiming | hipEventDisableSystemFence));
    {
      const size_t nz = (size_t)moe::kDecodeMaxTokens * n_experts;
      ALLOCCHK(host_malloc((void **)&c->h_z, nz * 8, hipHostMallocCoherent), "logit buffer");
      std::memset(c->h_z, 0, nz * 8);
      c->h_zf.resize(nz);
    }
    // the fixed scratch of moe_layer_forward_noalloc on this device, and the
    // page-locked buffers and host bookkeeping of its largest call
    HIPCHK(moe::noalloc_scratch(&c->scratch));
    c->ensure_pinned(moe::kNoAllocMaxTokens);
    c->jobs.resize((size_t)n_experts);
    for (auto &j : c->jobs) j.tokens.reserve(moe::kNoAllocMaxTokens);
    c->job_of.reserve((size_t)n_experts);
    c->rank_job.reserve((size_t)moe::kNoAllocMaxTokens * o.top_k);
    c->layers.resize(layers);
    for (int32_t l = 0; l < layers; ++l) {
      LayerState &ly = c->layers[l];
      ly.planner.reset(
          new moe::SlotPlanner(n_experts, slots, o.policy, o.preheat ? o.adopt : -1));
      const size_t nslots = (size_t)slots + o.n_shared;
      if (dev_malloc((void **)&ly.d_slots, nslots * c->rec()) != hipSuccess) {
        ly.d_slots = nullptr;
        (void)hipGetLastError();
        return fail(MOE_ENOMEM, "device slot arena allocation failed");
      }
      for (auto &e : ly.fill_ev) HIPCHK(hipEventCreateWithFlags(&e, hipEventDisableTiming));
      HIPCHK(hipEventCreateWithFlags(&ly.read_done,
                                     hipEventDisableTiming | hipEventDisableSystemFence));
      // preload: slot s <- expert s; shared slot S <- expert E
      for (int32_t s = 0; s < slots; ++s)
        HIPCHK(hipMemcpyAsync(c->dev_slot(l, s), c->host_record(l, s), c->rec(),
                              hipMemcpyHostToDevice, c->side[s & 1]));
      for (int32_t s = 0; s < o.n_shared; ++s)
        HIPCHK(hipMemcpyAsync(c->dev_slot(l, slots + s), c->host_record(l, n_experts + s), c->rec(),
                              hipMemcpyHostToDevice, c->side[0]));
    }
    for (auto sd : c->side) HIPCHK(hipStreamSynchronize(sd));
    return MOE_OK;
  });
  if (rc != MOE_OK) return rc;
  *out = c.release();
  return MOE_OK;
}

moe_status moe_layer_forward(moe_cache *c, int32_t layer, const float *x, int32_t n_tokens,
                             const float *router_w, const float *router_bias, float *out,
                             moe_stream_t stream) {
  g_err.clear();
  if (!c) return fail(MOE_EINVAL, "cache is NULL");
  if (layer < 0 || layer >= c->L) return fail(MOE_EINVAL, "layer out of range");
  if (n_tokens < 1) return fail(MOE_EINVAL, "n_tokens must be >= 1");
  if (n_tokens > (1 << 20)) return fail(MOE_EINVAL, "n_tokens too large");
  if (!x || !router_w || !out) return fail(MOE_EINVAL, "x, router_w and out must be non-NULL");
  return guarded(c, [&]() {
    TraceRange tr("moe.layer_forward");
    return forward_impl(c, layer, x, n_tokens, router_w, router_bias, out, stream);
  });
}

moe_status moe_layer_forward_noalloc(moe_cache *c, int32_t layer, const float *x,
                                     int32_t n_tokens, const float *router_w,
                                     const float *router_bias, float *out, moe_stream_t stream) {
  g_err.clear();
  if (!c) return fail(MOE_EINVAL, "cache is NULL");
  if (layer < 0 || layer >= c->L) return fail(MOE_EINVAL, "layer out of range");
  if (n_tokens < 1) return fail(MOE_EINVAL, "n_tokens must be >= 1");
  if (n_tokens > moe::kNoAllocMaxTokens)
    return fail(MOE_EINVAL, "n_tokens exceeds the allocation-free maximum (4)");
  if (!x || !router_w || !out) return fail(MOE_EINVAL, "x, router_w and out must be non-NULL");
  if (c->o.keep_debug)
    return fail(MOE_EINVAL, "keep_debug copies allocate: use moe_layer_forward");
  const moe::WsLayout WL = moe::ws_layout(c->ws_params(n_tokens));
  if (WL.total > moe::kNoAllocScratchBytes)
    return fail(MOE_EINVAL, "the call's workspace (" + std::to_string(WL.total) +
                                " bytes) exceeds the fixed scratch (" +
                                std::to_string(moe::kNoAllocScratchBytes) + " bytes)");
  if (!c->pinned_fits(n_tokens)) return fail(MOE_EINVAL, "page-locked buffers too small");
  return guarded(c, [&]() {
    TraceRange tr("moe.layer_forward_noalloc");
    // no timing events here: creating them would allocate
    const bool timing = c->timing;
    const uint32_t kmask = c->kmask;
    c->timing = false;
    c->kmask = 0;
    struct Restore {
      moe_cache *c;
      bool t;
      uint32_t m;
      ~Restore() {
        c->timing = t;
        c->kmask = m;
      }
    } restore{c, timing, kmask};
    return forward_impl(c, layer, x, n_tokens, router_w, router_bias, out, stream,
                        true);
  });
}

moe_status moe_cache_stats(moe_cache *c, int32_t layer, moe_stats *out) {
  g_err.clear();
  if (!c || !out) return fail(MOE_EINVAL, "NULL argument");
  if (layer < -1 || layer >= c->L) return fail(MOE_EINVAL, "layer out of range");
  return guarded(c, [&]() {
    std::memset(out, 0, sizeof(*out));
    for (int32_t l = 0; l < c->L; ++l) {
      if (layer >= 0 && l != layer) continue;
      LayerState &ly = c->layers[l];
      ly.t_gpu.collect();
      ly.t_h2d.collect();
      ly.st.gpu_s = ly.t_gpu.total;
      ly.st.h2d_s = ly.t_h2d.total;
      const moe_stats &s = ly.st;
      out->calls += s.calls;
      out->tokens += s.tokens;
      out->selections += s.selections;
      out->hits += s.hits;
      out->misses += s.misses;
      out->unique += s.unique;
      out->fills += s.fills;
      out->fill_bytes += s.fill_bytes;
      out->evictions += s.evictions;
      out->host_selections += s.host_selections;
      out->stages += s.stages;
      out->plan_s += s.plan_s;
      out->h2d_s += s.h2d_s;
      out->host_s += s.host_s;
      out->gpu_s += s.gpu_s;
    }
    return MOE_OK;
  });
}

moe_status moe_cache_set_timing(moe_cache *c, int32_t on) {
  g_err.clear();
  if (!c) return fail(MOE_EINVAL, "cache is NULL");
  if (on != 0 && on != 1) return fail(MOE_EINVAL, "on must be 0 or 1");
  c->timing = on != 0;
  c->kmask = on ? (1u << MOE_K_COUNT) - 1u : 0u;
  return MOE_OK;
}

moe_status moe_cache_set_kernel_timing(moe_cache *c, uint32_t kernel_mask) {
  g_err.clear();
  if (!c) return fail(MOE_EINVAL, "cache is NULL");
  if (kernel_mask >> MOE_K_COUNT) return fail(MOE_EINVAL, "kernel_mask has bits past MOE_K_COUNT");
  c->kmask = kernel_mask;
  return MOE_OK;
}

moe_status moe_cache_kernel_stats(moe_cache *c, int32_t kernel, int64_t *launches, double *seconds,
                                  double *bytes) {
  g_err.clear();
  if (!c) return fail(MOE_EINVAL, "cache is NULL");
  if (kernel < 0 || kernel >= MOE_K_COUNT) return fail(MOE_EINVAL, "kernel id out of range");
  return guarded(c, [&]() {
    KernelTiming &k = c->kt[kernel];
    k.log.collect();
    if (launches) *launches = k.launches;
    if (seconds) *seconds = k.log.total;
    if (bytes) *bytes = k.bytes;
    return MOE_OK;
  });
}

moe_status moe_cache_reset_stats(moe_cache *c) {
  g_err.clear();
  if (!c) return fail(MOE_EINVAL, "cache is NULL");
  return guarded(c, [&]() {
    for (auto &k : c->kt) {
      k.log.collect();
      k.log.total = 0.0;
      k.launches = 0;
      k.bytes = 0.0;
    }
    for (auto &ly : c->layers) {
      ly.t_gpu.collect();
      ly.t_h2d.collect();
      ly.t_gpu.total = 0;
      ly.t_h2d.total = 0;
      std::memset(&ly.st, 0, sizeof(ly.st));
    }
    return MOE_OK;
  });
}

moe_status moe_cache_sync(moe_cache *c) {
  g_err.clear();
  if (!c) return fail(MOE_EINVAL, "cache is NULL");
  return guarded(c, [&]() {
    for (auto sd : c->side) HIPCHK(hipStreamSynchronize(sd));
    return MOE_OK;
  });
}

moe_status moe_cache_usage(moe_cache *c, uint32_t *counts) {
  g_err.clear();
  if (!c || !counts) return fail(MOE_EINVAL, "NULL argument");
  for (int32_t l = 0; l < c->L; ++l) {
    const auto &u = c->layers[l].planner->usage();
    std::copy(u.begin(), u.end(), counts + (size_t)l * c->E);
  }
  return MOE_OK;
}

moe_status moe_cache_preload(moe_cache *c, const uint32_t *counts) {
  g_err.clear();
  if (!c || !counts) return fail(MOE_EINVAL, "NULL argument");
  return guarded(c, [&]() {
    // nothing may read or fill a slot while it is replaced
    HIPCHK(hipDeviceSynchronize());
    for (int32_t l = 0; l < c->L; ++l) {
      LayerState &ly = c->layers[l];
      ly.planner->preload(counts + (size_t)l * c->E);
      const auto &ein = ly.planner->expert_in();
      for (int32_t s = 0; s < c->S; ++s)
        HIPCHK(hipMemcpy(c->dev_slot(l, s), c->host_record(l, ein[s]), c->rec(),
                         hipMemcpyHostToDevice));
      ly.fill_pending = false;
      for (bool &u : ly.fill_used) u = false;
    }
    return MOE_OK;
  });
}

void moe_cache_destroy(moe_cache *c) { delete c; }

moe_status moe_debug_fill_delay(moe_cache *c, int32_t usec) {
  g_err.clear();
  if (!c) return fail(MOE_EINVAL, "cache is NULL");
  if (usec < 0 || usec > 1000000) return fail(MOE_EINVAL, "usec must be in [0, 1000000]");
  c->fill_delay_us = usec;
  return MOE_OK;
}

moe_status moe_debug_fail_alloc(int32_t nth) {
  g_err.clear();
  if (nth < -1) return fail(MOE_EINVAL, "nth must be >= -1");
  g_fail_alloc_in = nth;
  return MOE_OK;
}

moe_status moe_debug_last_call(moe_cache *c, int32_t layer, int32_t *n_stages, int32_t *n_tokens) {
  g_err.clear();
  if (!c) return fail(MOE_EINVAL, "cache is NULL");
  if (layer < 0 || layer >= c->L) return fail(MOE_EINVAL, "layer out of range");
  const LayerState &ly = c->layers[layer];
  if (n_stages) *n_stages = ly.last_T ? (int32_t)ly.plan.stages.size() : 0;
  if (n_tokens) *n_tokens = ly.last_T;
  return MOE_OK;
}

moe_status moe_debug_routing(moe_cache *c, int32_t layer, int32_t *idx, float *w) {
  g_err.clear();
  if (!c) return fail(MOE_EINVAL, "cache is NULL");
  if (layer < 0 || layer >= c->L) return fail(MOE_EINVAL, "layer out of range");
  const LayerState &ly = c->layers[layer];
  if (idx) std::copy(ly.last_idx.begin(), ly.last_idx.end(), idx);
  if (w) std::copy(ly.last_w.begin(), ly.last_w.end(), w);
  return MOE_OK;
}

moe_status moe_debug_views(moe_cache *c, int32_t layer, int32_t stage, int32_t *slot_view,
                           int32_t *host_view) {
  g_err.clear();
  if (!c) return fail(MOE_EINVAL, "cache is NULL");
  if (layer < 0 || layer >= c->L) return fail(MOE_EINVAL, "layer out of range");
  const LayerState &ly = c->layers[layer];
  if (!ly.last_T) return fail(MOE_EINVAL, "layer has no call yet");
  if (stage < 0 || stage >= (int32_t)ly.plan.stages.size()) return fail(MOE_EINVAL, "stage out of range");
  ly.planner->stage_view(ly.plan, stage, slot_view, host_view);
  return MOE_OK;
}

moe_status moe_debug_slots(moe_cache *c, int32_t layer, int32_t *expert_in, uint64_t *last_use) {
  g_err.clear();
  if (!c) return fail(MOE_EINVAL, "cache is NULL");
  if (layer < 0 || layer >= c->L) return fail(MOE_EINVAL, "layer out of range");
  const auto &p = *c->layers[layer].planner;
  if (expert_in) std::copy(p.expert_in().begin(), p.expert_in().end(), expert_in);
  if (last_use) std::copy(p.last_use().begin(), p.last_use().end(), last_use);
  return MOE_OK;
}

moe_status moe_debug_scores(moe_cache *c, int32_t layer, double *scores) {
  g_err.clear();
  if (!c || !scores) return fail(MOE_EINVAL, "NULL argument");
  if (layer < 0 || layer >= c->L) return fail(MOE_EINVAL, "layer out of range");
  const auto &p = *c->layers[layer].planner;
  std::copy(p.scores().begin(), p.scores().end(), scores);
  return MOE_OK;
}

static void copy_log(const std::vector<moe::EvictRecord> &log, moe_evict_rec *buf, size_t cap,
                     size_t *n) {
  const size_t m = std::min(cap, log.size());
  for (size_t i = 0; i < m; ++i) {
    buf[i].call = log[i].call;
    buf[i].stage = log[i].stage;
    buf[i].slot = log[i].slot;
    buf[i].evicted_expert = log[i].evicted;
    buf[i].inserted_expert = log[i].inserted;
  }
  if (n) *n = log.size();
}

moe_status moe_debug_evictions(moe_cache *c, int32_t layer, moe_evict_rec *buf, size_t cap,
                               size_t *n) {
  g_err.clear();
  if (!c) return fail(MOE_EINVAL, "cache is NULL");
  if (layer < 0 || layer >= c->L) return fail(MOE_EINVAL, "layer out of range");
  if (cap && !buf) return fail(MOE_EINVAL, "buf is NULL");
  copy_log(c->layers[layer].planner->log(), buf, cap, n);
  return MOE_OK;
}

moe_status moe_debug_partials(moe_cache *c, int32_t layer, float *gpu_part, float *host_part) {
  g_err.clear();
  if (!c) return fail(MOE_EINVAL, "cache is NULL");
  if (layer < 0 || layer >= c->L) return fail(MOE_EINVAL, "layer out of range");
  if (!c->o.keep_debug) return fail(MOE_EINVAL, "create the cache with keep_debug = 1");
  LayerState &ly = c->layers[layer];
  if (!ly.last_T) return fail(MOE_EINVAL, "layer has no call yet");
  return guarded(c, [&]() {
    const size_t n = (size_t)ly.last_T * c->d;
    if (gpu_part) {
      HIPCHK(hipDeviceSynchronize());
      HIPCHK(hipMemcpy(gpu_part, ly.dbg_gpu.p, n * 4, hipMemcpyDeviceToHost));
    }
    if (host_part) std::copy(ly.dbg_host.begin(), ly.dbg_host.begin() + n, host_part);
    return MOE_OK;
  });
}

moe_status moe_debug_logits(moe_cache *c, int32_t layer, float *z) {
  g_err.clear();
  if (!c || !z) return fail(MOE_EINVAL, "cache and z must be non-NULL");
  if (layer < 0 || layer >= c->L) return fail(MOE_EINVAL, "layer out of range");
  if (!c->o.keep_debug) return fail(MOE_EINVAL, "create the cache with keep_debug = 1");
  LayerState &ly = c->layers[layer];
  if (!ly.last_T) return fail(MOE_EINVAL, "layer has no call yet");
  return guarded(c, [&]() {
    HIPCHK(hipDeviceSynchronize());
    HIPCHK(hipMemcpy(z, ly.dbg_z.p, (size_t)ly.last_T * c->E * 4, hipMemcpyDeviceToHost));
    return MOE_OK;
  });
}

// ---------------------------------------------------------------- planner only

struct moe_planner {
  std::unique_ptr<moe::SlotPlanner> p;
  int32_t mode = 0, max_fills = -1;
  moe::CallPlan last;
  bool has_call = false;
};

moe_status moe_planner_create(int32_t n_experts, int32_t slots, int32_t miss_mode,
                              int32_t max_fills_per_call, int32_t policy, moe_planner **out) {
  g_err.clear();
  if (!out) return fail(MOE_EINVAL, "out is NULL");
  *out = nullptr;
  if (n_experts < 1 || n_experts > MOE_MAX_EXPERTS) return fail(MOE_EINVAL, "n_experts out of range");
  if (slots < 1 || slots > n_experts) return fail(MOE_EINVAL, "slots must be in [1, n_experts]");
  if (miss_mode != MOE_MISS_STREAM && miss_mode != MOE_MISS_HOST)
    return fail(MOE_EINVAL, "bad miss_mode");
  if (max_fills_per_call < -1) return fail(MOE_EINVAL, "max_fills_per_call must be >= -1");
  if (policy != MOE_POLICY_LRU && policy != MOE_POLICY_SCORE) return fail(MOE_EINVAL, "bad policy");
  try {
    auto *p = new moe_planner();
    p->p.reset(new moe::SlotPlanner(n_experts, slots, policy));
    p->mode = miss_mode;
    p->max_fills = max_fills_per_call;
    *out = p;
  } catch (const std::bad_alloc &) {
    return fail(MOE_ENOMEM, "host allocation failed");
  }
  return MOE_OK;
}

moe_status moe_planner_plan(moe_planner *p, const int32_t *idx, int32_t n_sel, int32_t n_tokens,
                            int32_t *n_stages, int32_t *hits, int32_t *misses) {
  g_err.clear();
  if (!p || (!idx && n_sel > 0)) return fail(MOE_EINVAL, "NULL argument");
  if (n_sel < 1) return fail(MOE_EINVAL, "n_sel must be >= 1");
  if (n_tokens < 1 || n_sel % n_tokens) return fail(MOE_EINVAL, "n_sel must be a multiple of n_tokens");
  for (int32_t i = 0; i < n_sel; ++i)
    if (idx[i] < 0 || idx[i] >= p->p->n_experts()) return fail(MOE_EINVAL, "expert id out of range");
  try {
    p->p->plan(idx, n_sel, n_tokens, p->mode, p->max_fills, p->last);
  } catch (const std::bad_alloc &) {
    return fail(MOE_ENOMEM, "host allocation failed");
  }
  p->has_call = true;
  if (n_stages) *n_stages = (int32_t)p->last.stages.size();
  if (hits) *hits = p->last.hits;
  if (misses) *misses = p->last.misses;
  return MOE_OK;
}

moe_status moe_planner_views(moe_planner *p, int32_t stage, int32_t *slot_view, int32_t *host_view) {
  g_err.clear();
  if (!p) return fail(MOE_EINVAL, "planner is NULL");
  if (!p->has_call) return fail(MOE_EINVAL, "no call planned yet");
  if (stage < 0 || stage >= (int32_t)p->last.stages.size()) return fail(MOE_EINVAL, "stage out of range");
  p->p->stage_view(p->last, stage, slot_view, host_view);
  return MOE_OK;
}

moe_status moe_planner_slots(moe_planner *p, int32_t *expert_in, uint64_t *last_use) {
  g_err.clear();
  if (!p) return fail(MOE_EINVAL, "planner is NULL");
  if (expert_in) std::copy(p->p->expert_in().begin(), p->p->expert_in().end(), expert_in);
  if (last_use) std::copy(p->p->last_use().begin(), p->p->last_use().end(), last_use);
  return MOE_OK;
}

moe_status moe_planner_evictions(moe_planner *p, moe_evict_rec *buf, size_t cap, size_t *n) {
  g_err.clear();
  if (!p) return fail(MOE_EINVAL, "planner is NULL");
  if (cap && !buf) return fail(MOE_EINVAL, "buf is NULL");
  copy_log(p->p->log(), buf, cap, n);
  return MOE_OK;
}

moe_status moe_planner_usage(moe_planner *p, uint32_t *counts) {
  g_err.clear();
  if (!p || !counts) return fail(MOE_EINVAL, "NULL argument");
  std::copy(p->p->usage().begin(), p->p->usage().end(), counts);
  return MOE_OK;
}

moe_status moe_planner_preload(moe_planner *p, const uint32_t *counts) {
  g_err.clear();
  if (!p || !counts) return fail(MOE_EINVAL, "NULL argument");
  p->p->preload(counts);
  return MOE_OK;
}

moe_status moe_planner_set_adopt(moe_planner *p, int32_t adopt) {
  g_err.clear();
  if (!p) return fail(MOE_EINVAL, "planner is NULL");
  if (adopt < -1 || adopt > 1000) return fail(MOE_EINVAL, "adopt must be -1 or in [0, 1000]");
  p->p->set_adopt(adopt);
  return MOE_OK;
}

moe_status moe_planner_scores(moe_planner *p, double *scores) {
  g_err.clear();
  if (!p || !scores) return fail(MOE_EINVAL, "NULL argument");
  std::copy(p->p->scores().begin(), p->p->scores().end(), scores);
  return MOE_OK;
}

void moe_planner_destroy(moe_planner *p) { delete p; }

moe_status moe_host_topk(const float *z, int32_t n_tokens, int32_t n_experts, int32_t top_k,
                         int32_t norm_topk, int32_t *idx, float *w) {
  g_err.clear();
  if (!z || !idx || !w) return fail(MOE_EINVAL, "NULL argument");
  if (n_tokens < 1) return fail(MOE_EINVAL, "n_tokens must be >= 1");
  if (n_experts < 1 || n_experts > MOE_MAX_EXPERTS) return fail(MOE_EINVAL, "n_experts out of range");
  if (top_k < 1 || top_k > n_experts) return fail(MOE_EINVAL, "top_k must be in [1, n_experts]");
  if (norm_topk != 0 && norm_topk != 1) return fail(MOE_EINVAL, "norm_topk must be 0 or 1");
  moe::host_topk(z, n_tokens, n_experts, top_k, norm_topk, idx, w);
  return MOE_OK;
}

moe_status moe_host_expert_forward(const void *expert_q4, int32_t d_model, int32_t d_ff,
                                   const float *x, int32_t n_tokens, float *y, int32_t threads) {
  g_err.clear();
  if (!expert_q4 || !x || !y) return fail(MOE_EINVAL, "NULL argument");
  if (d_model <= 0 || d_model % 64 || d_ff <= 0 || d_ff % 32) return fail(MOE_EINVAL, "bad shape");
  if (n_tokens < 1) return fail(MOE_EINVAL, "n_tokens must be >= 1");
  try {
    const moe::RecordLayout L = moe::RecordLayout::make(d_model, d_ff);
    std::vector<uint8_t> rec((size_t)L.bytes);
    moe::repack_expert((const uint8_t *)expert_q4, L, rec.data());
    moe::ThreadPool pool(threads > 0 ? threads : default_threads());
    moe::host_expert_forward(pool, L, rec.data(), x, n_tokens, y);
  } catch (const std::bad_alloc &) {
    return fail(MOE_ENOMEM, "host allocation failed");
  } catch (const std::exception &e) {
    return fail(MOE_EINVAL, e.what());
  }
  return MOE_OK;
}

}  // extern "C"
