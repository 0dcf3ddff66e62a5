/*
 * moe_cache.h -- C ABI of libmoecache: a routed Mixture-of-Experts FFN layer
 * served from a per-layer GPU cache of hot experts, for one AMD Instinct MI355X
 * (gfx950).
 *
 * The method (pages: "llama.cpp + MoE expert cache", section "How it works";
 * "longhaul.md", section "Longhaul MoE loading"):
 *   - every expert of every layer stays in host RAM in 4-bit blocks (32 weights
 *     plus a binary16 scale in 18 bytes);
 *   - each layer owns a fixed number of GPU slots holding copies of experts,
 *     replaced least-recently-used, independently per layer; the experts the
 *     current batch already needs are protected from eviction and duplicate ids
 *     load once;
 *   - routing gives two tables, expert -> GPU slot (-1 when not cached) and
 *     expert -> host id (-1 when cached); cached experts are computed on the GPU,
 *     misses either on host cores in parallel (MOE_MISS_HOST) or streamed into
 *     slots first (MOE_MISS_STREAM); every selected expert is computed exactly
 *     once and the partial results are summed;
 *   - when a step selects more experts than there are slots, the routed work
 *     runs in stages whose partial results are summed.
 *
 * Conventions for every call below:
 *   - A function returns MOE_OK (0) or a negative moe_status.  On failure
 *     moe_last_error() returns a message (thread-local, valid until the next
 *     call on the same thread).  No C++ exception crosses this interface.
 *   - MOE_EINVAL: an argument is invalid; nothing was changed.
 *   - MOE_ENOMEM: an allocation failed; nothing leaks.
 *   - MOE_EHIP: a HIP runtime call failed; the cache is poisoned and every later
 *     call on it returns MOE_ESTATE (destroy still works).
 *   - "device pointer" means memory the current HIP device can read/write
 *     (hipMalloc, or a torch CUDA tensor's data_ptr()); "host pointer" means
 *     ordinary process memory.
 *   - One cache is driven by one host thread at a time; calls are not
 *     re-entrant.  Calls for different layers may interleave in any order.
 */
#ifndef MOE_CACHE_H
#define MOE_CACHE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The caller's HIP stream.  hip/hip_runtime.h declares hipStream_t as a pointer
 * to struct ihipStream_t; this is the same type, declared here so that the
 * header needs no HIP header.  NULL is the default stream. */
struct ihipStream_t;
typedef struct ihipStream_t *moe_stream_t;

typedef int32_t moe_status;
#define MOE_OK 0
#define MOE_EINVAL (-1)
#define MOE_ENOMEM (-2)
#define MOE_EHIP (-3)
#define MOE_ESTATE (-4)

/* Miss handling ("How it works" step 3 computes misses on the CPU; longhaul.md
 * populates missing slots and continues with cache-local ids). */
#define MOE_MISS_STREAM 0
#define MOE_MISS_HOST 1

/* Slot policy.  MOE_POLICY_LRU: least-recently-used replacement per layer, the
 * batch's experts protected ("Longhaul MoE loading", introduction and "Current
 * scope").  MOE_POLICY_SCORE: a decayed usage score per expert, x0.9 per token
 * and +1 per selection; a missed expert is admitted only when it scores
 * strictly more than the weakest unprotected slot, within max_fills_per_call
 * copies per call ("Keeping the cache fresh", llama.cpp + MoE expert cache).
 * In stream mode every miss is still filled and the weakest slot is the victim. */
#define MOE_POLICY_LRU 0
#define MOE_POLICY_SCORE 1

/* Prefill preheat (opts.preheat = 1; "Prefill preheat", llama.cpp fork with
 * multi GPU acceleration: the cache keeps a prompt batch's most-used experts in
 * place of cached experts the batch used less, and an adopt share bounds how
 * many of a layer's slots one batch may replace).  It applies to stream-mode
 * calls whose misses outnumber the slots holding none of their hits, which run
 * in stages through the slots.  Experts rank by (-count in the call, id); the
 * slots holding none of the call's S top-ranked experts, weakest first (lowest
 * -ranked expert first), give a pool of min(their number, adopt * S / 1000)
 * slots (at least one: staging needs a slot); only pool slots take fills, the
 * lowest-ranked misses first, so the pool ends holding the call's best-ranked
 * misses and the other slots keep their experts.  With adopt = 1000 the layer
 * ends holding exactly the call's S top-ranked experts.  Other calls, and host
 * mode, follow the policy's plain rule. */

/* Limits of the library. */
#define MOE_MAX_EXPERTS 512 /* routed experts per layer */
#define MOE_MAX_TOPK 64

typedef struct moe_cache moe_cache; /* opaque, owned by the library */

typedef struct moe_cache_opts {
  int32_t top_k;              /* k experts per token, 1..min(n_experts, 64)     default 8 */
  int32_t miss_mode;          /* MOE_MISS_STREAM or MOE_MISS_HOST               default STREAM */
  int32_t n_shared;           /* 0 or 1 always-resident shared experts/layer    default 0 */
  int32_t norm_topk;          /* 1: renormalise the k softmax weights           default 1 */
  int32_t host_threads;       /* host-miss workers, 0 = cores - 1               default 0 */
  int32_t max_fills_per_call; /* host mode: fills per call, -1 = every miss     default -1 */
  int32_t keep_debug;         /* 1: keep per-layer GPU/host partials            default 0 */
  int32_t timing;             /* 1: time fills and compute with HIP events       default 0 */
  int32_t policy;             /* MOE_POLICY_LRU or MOE_POLICY_SCORE             default LRU */
  int32_t preheat;            /* 1: prefill preheat for staged stream calls      default 0 */
  int32_t adopt;              /* preheat share of the slots, per mille 0..1000   default 1000 */
  int32_t reserved[5];        /* must be 0 */
} moe_cache_opts;

/* Counters since create or the last moe_cache_reset_stats.  A "selection" is one
 * (token, rank) pick of the router; hits and misses count selections, which is
 * how the hit rates of "llama.cpp + MoE expert cache" (The idea: cache the hot
 * experts on the GPU) are counted. */
typedef struct moe_stats {
  uint64_t calls;           /* moe_layer_forward calls */
  uint64_t tokens;          /* tokens over all calls */
  uint64_t selections;      /* tokens * top_k */
  uint64_t hits;            /* selections whose expert was cached at call start */
  uint64_t misses;          /* selections - hits */
  uint64_t unique;          /* distinct experts per call, summed */
  uint64_t fills;           /* experts copied host -> slot */
  uint64_t fill_bytes;      /* bytes of those copies */
  uint64_t evictions;       /* fills that replaced a cached expert */
  uint64_t host_selections; /* selections computed on host cores (host mode) */
  uint64_t stages;          /* stages over all calls (1 per call unless staged) */
  double plan_s;            /* host time in the slot planner */
  double h2d_s;             /* device time of slot fills (opts.timing only) */
  double host_s;            /* host time computing missed experts */
  double gpu_s;             /* device time of the call's GPU work (opts.timing only) */
} moe_stats;

/* One slot replacement: in call `call` (per layer, from 0), stage `stage`, slot
 * `slot` changed from `evicted_expert` (-1 = was empty) to `inserted_expert`. */
typedef struct moe_evict_rec {
  int64_t call;
  int32_t stage;
  int32_t slot;
  int32_t evicted_expert;
  int32_t inserted_expert;
} moe_evict_rec;

/* Fills *o with the defaults listed in moe_cache_opts. */
void moe_cache_default_opts(moe_cache_opts *o);

/*
 * moe_cache_create -- build a cache for `layers` MoE layers.
 *
 * host_q4_weights (host pointer, read during this call only): every expert of
 * every layer in the interchange layout -- for layer l, for expert e in
 * [0, n_experts + n_shared): gate rows [d_ff][d_model], up rows [d_ff][d_model],
 * down rows [d_model][d_ff]; each row quantised along its reduction dimension
 * in 18-byte blocks (bytes 0-1: binary16 scale d, little-endian; byte 2+j:
 * element j in the low nibble, element j+16 in the high nibble; w = d*(q-8)),
 * blocks in K order, no padding.  The 18/32 bytes per weight are the Q4_0 size
 * of "Multi-GPU LLM Calculator" (Memory placement).  Shared experts follow the
 * routed ones of their layer.
 *
 * The library copies the weights into its own page-locked host arena (repacked
 * per expert so that one slot fill is one contiguous copy), allocates
 * (slots + n_shared) device slots per layer, uploads the shared experts, and
 * preloads slot s with expert s (s < slots) so that slots == n_experts gives
 * hits from the first call.  Uses the current HIP device.
 *
 * Requirements: layers >= 1; 1 <= n_experts <= MOE_MAX_EXPERTS;
 * 1 <= slots <= n_experts; d_model % 64 == 0; d_ff % 32 == 0; opts may be NULL.
 * On success *out receives the cache.
 */
moe_status moe_cache_create(int32_t layers, int32_t n_experts, int32_t slots, int32_t d_model,
                            int32_t d_ff, const void *host_q4_weights, const moe_cache_opts *opts,
                            moe_cache **out);

/*
 * moe_layer_forward -- out = the MoE layer `layer` applied to x.
 *
 *   x           device pointer, float32 [n_tokens][d_model], row-major
 *   router_w    device pointer, float32 [n_experts][d_model], row-major
 *   router_bias device pointer, float32 [n_experts], or NULL (no bias)
 *   out         device pointer, float32 [n_tokens][d_model]; overwritten
 *   stream      the caller's hipStream_t (NULL = the default stream)
 *
 * Router logits z = x . router_w^T + bias are formed in float32 in one fixed
 * order (64 lane partials over i = l, l+64, ..., product and sum rounded
 * separately, then a halving tree, then the bias); the k largest are selected,
 * ties to the lower expert id, ordered by decreasing z; gating weights are the
 * softmax over all n_experts logits, renormalised over the k when norm_topk.
 * Each selected expert computes y = D (silu(G x) * (U x)); shared experts add
 * with weight 1; out[t] = sum_j w[t,j] y_{idx[t,j]} + shared.
 *
 * MOE_MISS_STREAM: the call waits for the routing (the top-k kernel writes
 * the ids to page-locked memory and raises a flag), plans, copies missed
 * experts into slots (decode-sized calls: a copy kernel on `stream`; larger
 * calls: the copy engines on side streams) and computes every selected expert
 * on the GPU, in stages when more experts are selected than slots exist.
 * MOE_MISS_HOST: GPU work on cached experts is enqueued
 * before the routing reaches the host; host threads then compute the misses,
 * the misses' slot fills are queued on the side stream and become visible at
 * the same layer's next call, and the GPU adds the host partial; the call
 * returns when the host partial has been handed to `stream`.
 *
 * x, router_w, router_bias and out must stay valid until `stream` has passed
 * this call's work.  Calls are ordered on their stream; a call on another
 * stream than the cache's previous call (of any layer) first waits for the
 * whole device (hipDeviceSynchronize), since every layer shares the cache's
 * workspace and no earlier reader of a slot may race with its refill.
 * Requirements: 0 <= layer < layers; 1 <= n_tokens; the
 * pointers non-NULL except router_bias and stream.
 */
moe_status moe_layer_forward(moe_cache *c, int32_t layer, const float *x, int32_t n_tokens,
                             const float *router_w, const float *router_bias, float *out,
                             moe_stream_t stream);

/*
 * moe_layer_forward_noalloc -- moe_layer_forward for callers that cannot
 * allocate: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.  Same arguments, same kernels and the same results as
 * moe_layer_forward (outputs, routing, slot tables, eviction log and stats).
 *
 * It calls no hipMalloc, hipFree, hipHostMalloc or other allocating routine:
 * the call's device workspace is a fixed array of 16 MiB per device inside the
 * library (looked up once per device at moe_cache_create and held until the
 * process ends), and its page-locked routing and host-partial buffers were
 * sized at create for its largest call.  It records no timing events.  Host
 * bookkeeping (planner, host-miss jobs) reuses the cache's vectors, whose
 * capacity create reserves.
 *
 * Limits (MOE_EINVAL, nothing changed): 1 <= n_tokens <= 4; the call's
 * workspace (router logits, routing, prepared activations, the pairs' hidden
 * rows and outputs, bucket lists) must fit the 16 MiB; the cache must not have
 * keep_debug set.
 *
 * The array is shared by every call on the device and keeps the last call's
 * contents (every region is written before it is read).  Calls that overlap on
 * one device -- two caches, or streams that are not ordered -- race on it; a
 * cache orders its own calls (a call on another stream than its last one waits
 * for the device first).  It may be mixed with moe_layer_forward on the same
 * cache.
 */
moe_status moe_layer_forward_noalloc(moe_cache *c, int32_t layer, const float *x,
                                     int32_t n_tokens, const float *router_w,
                                     const float *router_bias, float *out, moe_stream_t stream);

/* Counters of one layer (layer >= 0) or summed over layers (layer == -1).
 * Synchronises the library's own streams to read device timings. */
moe_status moe_cache_stats(moe_cache *c, int32_t layer, moe_stats *out);

/* Turns the event timing of opts.timing on (1) or off (0) from now on. */
/* Usage profile ("Persistent hot experts", llama.cpp fork with multi GPU
 * acceleration: the cache saves how often each expert was used and the next
 * start preloads each layer's most-used experts).
 *
 * moe_cache_usage writes counts[layers * n_experts] (layer-major, uint32): the
 * selections of each expert since create, plus any counts preloaded.
 *
 * moe_cache_preload reads counts[layers * n_experts] from the caller (host
 * memory, read during the call only).  It waits for the device, then per layer
 * puts the S most-used experts by (-count, id) in the slots (the least used of
 * them in slot 0, the most used in slot S-1, so the least used is evicted
 * first), copies their records in, makes every slot unprotected from the next
 * call on, resets the usage scores and adds the counts to the lifetime counts.
 * Meant at start-up, before the first moe_layer_forward; any time is allowed. */
moe_status moe_cache_usage(moe_cache *c, uint32_t *counts);
moe_status moe_cache_preload(moe_cache *c, const uint32_t *counts);

moe_status moe_cache_set_timing(moe_cache *c, int32_t on);

/* Kernels timed one launch at a time when timing is on. */
#define MOE_K_ROUTER 0  /* router logits */
#define MOE_K_TOPK 1    /* top-k + softmax gating weights */
#define MOE_K_REMAP 2   /* expert -> slot remap and bucketing */
#define MOE_K_GATEUP 3  /* Q4 gate/up projections + SwiGLU */
#define MOE_K_DOWN 4    /* Q4 down projection */
#define MOE_K_COMBINE 5 /* weighted combine */
#define MOE_K_FILL 6    /* slot fills pulled from the page-locked arena by a kernel */
#define MOE_K_PREP 7    /* binary16 hi/lo preparation of h for the prefill down GEMM */
#define MOE_K_COUNT 8

/* Times only the kernels whose bit (1 << MOE_K_*) is set in kernel_mask, one
 * launch at a time, from now on; the per-layer compute and fill timings of
 * moe_cache_set_timing stay as they are.  moe_cache_set_timing(c, 1) sets every
 * bit, (c, 0) clears them.  A timed launch carries a start and a stop event
 * that the GPU records at that kernel's own dispatch (hipExtLaunchKernel),
 * and a third event is recorded on the stream just before it; the time runs
 * from the later of the two starts to the stop, which leaves out both the
 * host's launch latency (idle stream) and the wait for earlier work on the
 * stream (busy stream).  MOE_EINVAL for bits at or past MOE_K_COUNT. */
moe_status moe_cache_set_kernel_timing(moe_cache *c, uint32_t kernel_mask);

/* Launches, summed device seconds (the launches' own events on the launching
 * stream, as set out for moe_cache_set_kernel_timing, read when this is called) and summed algorithmic bytes of kernel `kernel` since the
 * last reset.  Algorithmic bytes: router = W_r + x + logits; Q4 kernels = the
 * 18/32-byte-per-weight bytes of every expert matrix the launch reads; fill =
 * the slot records copied host -> device; prep = h read + pairs written;
 * combine = expert outputs read + layer output written.  On batches beyond the
 * decode path (more than 4 tokens) MOE_K_GATEUP / MOE_K_DOWN time the matrix-core
 * grouped GEMM. */
moe_status moe_cache_kernel_stats(moe_cache *c, int32_t kernel, int64_t *launches, double *seconds,
                                  double *bytes);

/* Zeroes every counter and timing (slot contents and eviction logs stay). */
moe_status moe_cache_reset_stats(moe_cache *c);

/* Waits for the library's side-stream work (slot fills) to finish. */
moe_status moe_cache_sync(moe_cache *c);

/* Frees everything the cache owns; waits for its streams first.  NULL is a no-op. */
void moe_cache_destroy(moe_cache *c);

/* Message of the last failure on this thread ("" if none). */
const char *moe_last_error(void);

/* Bytes of one expert in the library's slot layout (>= 3*d*f*18/32, rounded up
 * to 4096); 0 for invalid shapes. */
int64_t moe_slot_bytes(int32_t d_model, int32_t d_ff);

/* ---- inspection of the LAST call of a layer (host pointers, caller-owned) ---- */

/* Number of stages and tokens of the last call of `layer` (0 before any call). */
moe_status moe_debug_last_call(moe_cache *c, int32_t layer, int32_t *n_stages,
                               int32_t *n_tokens);

/* idx [n_tokens*top_k] int32 and w [n_tokens*top_k] float32 of the last call
 * (either may be NULL).  Synchronises the compute work of that call. */
moe_status moe_debug_routing(moe_cache *c, int32_t layer, int32_t *idx, float *w);

/* The two lookup tables of stage `stage` of the last call, [n_experts] each:
 * slot_view[e] = slot computing e in that stage or -1; host_view[e] = e when
 * e is computed on host cores, else -1 (all -1 in stream mode). */
moe_status moe_debug_views(moe_cache *c, int32_t layer, int32_t stage, int32_t *slot_view,
                           int32_t *host_view);

/* Current slot state: expert_in[slots] (-1 = empty) and last_use[slots]. */
moe_status moe_debug_slots(moe_cache *c, int32_t layer, int32_t *expert_in, uint64_t *last_use);

/* Usage scores of `layer`'s experts, scores[n_experts] (binary64; all 0 under
 * MOE_POLICY_LRU). */
moe_status moe_debug_scores(moe_cache *c, int32_t layer, double *scores);

/* The layer's whole replacement log since create; copies min(cap, total)
 * records into buf (may be NULL when cap == 0) and stores the total in *n. */
moe_status moe_debug_evictions(moe_cache *c, int32_t layer, moe_evict_rec *buf, size_t cap,
                               size_t *n);

/* Requires opts.keep_debug.  gpu_part [n_tokens*d_model]: the GPU's sum (routed
 * experts on slots + shared); host_part: the host cores' weighted sum (zeros in
 * stream mode).  out == gpu_part + host_part element by element. */
moe_status moe_debug_partials(moe_cache *c, int32_t layer, float *gpu_part, float *host_part);

/* Requires opts.keep_debug.  z [n_tokens*n_experts] float32: the router logits
 * of the last call of `layer` (bias included), in the fixed summation order of
 * the router (routing: "llama.cpp + MoE expert cache", *How it works*), for
 * bit-for-bit comparison.  Synchronises the device. */
moe_status moe_debug_logits(moe_cache *c, int32_t layer, float *z);

/* ---- failure forcing for tests (host-driven; every kernel still runs normally) ---- */

/* Holds every batch of copy-engine slot fills of this cache (host mode, staged
 * calls) for usec microseconds before it starts (a host function on the copy
 * stream), as a slow link would.  Results, tables and logs must not change:
 * no kernel reads a slot before its copy has landed ("Keeping the cache
 * fresh", llama.cpp + MoE expert cache: a slot leaves the table before its copy
 * and is published after it).  0 turns it off; usec in [0, 1e6]. */
moe_status moe_debug_fill_delay(moe_cache *c, int32_t usec);

/* Makes the nth device or page-locked allocation from now on, on this thread,
 * fail as if memory were exhausted (0 = the next one; -1 = none).  The call
 * that needed it returns MOE_ENOMEM: moe_cache_create frees everything it had
 * allocated, moe_layer_forward leaves the cache usable (its allocations precede
 * its work).  Fires once. */
moe_status moe_debug_fail_alloc(int32_t nth);

/* ---- host-only pieces, callable without a GPU ---- */

typedef struct moe_planner moe_planner; /* the per-layer LRU slot planner alone */

/* A planner with the same rules and initial state as one layer of a cache
 * (slot s holds expert s, every score 0).  miss_mode, max_fills_per_call and
 * policy as in moe_cache_opts. */
moe_status moe_planner_create(int32_t n_experts, int32_t slots, int32_t miss_mode,
                              int32_t max_fills_per_call, int32_t policy, moe_planner **out);

/* Prefill preheat of the planner, as opts.preheat / opts.adopt: adopt = -1 turns
 * it off (the state after create), 0..1000 turns it on with that share. */
moe_status moe_planner_set_adopt(moe_planner *p, int32_t adopt);

/* Plans one call on the router ids idx[n_sel], token-major, n_sel = n_tokens *
 * top_k (n_sel a multiple of n_tokens >= 1).  After it, *n_stages, *hits and
 * *misses describe the call. */
moe_status moe_planner_plan(moe_planner *p, const int32_t *idx, int32_t n_sel, int32_t n_tokens,
                            int32_t *n_stages, int32_t *hits, int32_t *misses);

/* The usage scores after the last call, scores[n_experts] (all 0 under LRU). */
moe_status moe_planner_scores(moe_planner *p, double *scores);

/* Lifetime counts and profile preload of one layer, as moe_cache_usage and
 * moe_cache_preload (counts[n_experts]). */
moe_status moe_planner_usage(moe_planner *p, uint32_t *counts);
moe_status moe_planner_preload(moe_planner *p, const uint32_t *counts);

/* Tables of one stage of the last planned call, as moe_debug_views. */
moe_status moe_planner_views(moe_planner *p, int32_t stage, int32_t *slot_view,
                             int32_t *host_view);

/* Slot state and full replacement log, as moe_debug_slots / moe_debug_evictions. */
moe_status moe_planner_slots(moe_planner *p, int32_t *expert_in, uint64_t *last_use);
moe_status moe_planner_evictions(moe_planner *p, moe_evict_rec *buf, size_t cap, size_t *n);

void moe_planner_destroy(moe_planner *p);

/* The host's expert selection on decode calls: per token, the k largest of the
 * E logits z[t][*], ordered by decreasing value, equal values (-0 == +0) to the
 * lower expert id, and the gating weights (softmax over all E logits in
 * binary64, renormalised over the k when norm_topk, rounded to float32).  The
 * GPU's top-k kernel selects the same ids from the same float32 logits: both
 * order by the float's bits mapped to an order-preserving key, so even
 * non-finite logits (outside the method) get one order, a NaN with the sign
 * bit clear above +inf and one with it set below -inf.
 * z: host float32 [n_tokens][n_experts]; idx, w: host [n_tokens][top_k].
 * Requirements: n_tokens >= 1; 1 <= top_k <= n_experts <= MOE_MAX_EXPERTS;
 * norm_topk 0 or 1. */
moe_status moe_host_topk(const float *z, int32_t n_tokens, int32_t n_experts, int32_t top_k,
                         int32_t norm_topk, int32_t *idx, float *w);

/* One expert on host cores, as host mode computes a miss: y[t] = D (silu(G x_t)
 * * (U x_t)) for t < n_tokens.  expert_q4: host pointer to ONE expert in the
 * interchange layout; x, y: host float32 [n_tokens][d_model]; threads <= 0
 * means cores - 1. */
moe_status moe_host_expert_forward(const void *expert_q4, int32_t d_model, int32_t d_ff,
                                   const float *x, int32_t n_tokens, float *y, int32_t threads);

#ifdef __cplusplus
}
#endif
#endif /* MOE_CACHE_H */
