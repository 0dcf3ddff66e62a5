// Launchers of the gfx950 kernels (host-callable; no device code here).
#pragma once
#include <hip/hip_runtime_api.h>

#include <cstdint>

#include "shapes.hpp"

namespace moe {

// The next kernel launch of the calling host thread records `start` at its
// dispatch start and `stop` at its end (both may be null: no timing).
void set_launch_events(hipEvent_t start, hipEvent_t stop);
// True when events set by set_launch_events were not taken by a launch (the
// launch function returned without launching); clears them either way.
bool launch_events_pending();


// Expert -> slot table of one stage, passed by value as a kernel argument so
// that each launch carries its own table (no copy, no reuse hazard).
struct SlotView {
  int16_t slot[kMaxExperts];
};

// z[t][e] = x[t] . W[e] (+ b[e]) in the fixed fp32 order.  The waves also
// prepare each token's x for the expert kernels, in one of two forms:
// - xq != nullptr (decode GEMV): digit planes of X = rint(x / s) with one scale
//   per 32-element block b, s = max|x over the block| / 30000 (xs[t][b], row
//   stride 4 * xs_units(d/32)); per block b and word j,
//   xq[(t*d/32 + b)*4 + j] holds planes 0..3 as x, y, z, w (the layout is
//   described with the decode GEMV);
// - xp != nullptr (matrix-core GEMM): a power-of-two scale 2^-e that brings
//   max|x| into [2^13, 2^14) (xscale[t] = 2^e, e in [-126, 127]); the scaled x
//   as binary16 hi and lo pairs in the order the nibble decoder yields weights
//   (for 32-bit word j of block b = j/4 and g = 4*(j%4): (x[g],x[g+2]),
//   (x[g+16],x[g+18]), (x[g+1],x[g+3]), (x[g+17],x[g+19]) of the block, hi then
//   lo).
// h_z (page-locked, coherent; when given): logit t*E + e also goes to
// h_z[t*E + e] as (seq << 32) | bits in one 8-byte store, the host's copy of the
// routing input.
// h_x (decode planes only, when router_decode_fits): page-locked host copy of
// x [T][d]; a workgroup's part of it reaches host memory before its logits.
hipError_t launch_router(const float *x, int T, int d, const float *W, const float *bias, int E,
                         float *z, uint32_t *xp, float *xscale, uint4 *xq, float *xs,
                         hipStream_t s, float *h_x = nullptr, unsigned long long *h_z = nullptr,
                         uint32_t seq = 0);
// The one-workgroup-per-expert decode router handles this call.
bool router_decode_fits(int T, int d, int E);

// Per token: k largest logits (ties to the lower id), softmax gating weights,
// written to device memory (idx, w) and to page-locked host memory (h_idx, h_w).
hipError_t launch_topk(const float *z, int T, int E, int k, int norm_topk, int32_t *idx,
                       float *w, int32_t *h_idx, float *h_w, hipStream_t s);

// Decode top-k (T <= kDecodeMaxTokens, T*k + shared pairs <= kDecodeMaxPairs;
// else hipErrorInvalidValue): as launch_topk on the device (idx, w), and also
// maps each routed pair to its slot through `view` (pair_slot[T*k], -1 when not
// cached) and writes the bucket list of the cached experts plus, when
// shared_slot >= 0, one bucket of the shared expert's T pairs (pair T*k + t) at
// slot shared_slot.  Writes nothing to host memory.
struct DecodeTopk {
  int k, norm_topk;
  int32_t *idx;
  float *w;
  SlotView view;
  int shared_slot;
  int32_t *buckets, *pair_slot;
};
hipError_t launch_topk_decode(const float *z, int T, int E, const DecodeTopk &a, hipStream_t s);

// Expert -> slot remap of the routed pairs (plus one shared pair per token when
// shared_slot >= 0) and stable bucketing per slot, for batches beyond the
// decode path.  meta: [0] = buckets, [1] = pairs, [2 + b] = slot,
// [2 + kMetaB + b] = first pair position, [2 + 2 kMetaB + b] = pair count;
// bucket_pair holds pair ids grouped by bucket, ascending within a bucket;
// items[0] = work items, items[1 + i] = bucket | (pass << 16), buckets in order
// and passes ascending (room for gemm_items_bound(n_slot_ids, pairs) + 1).
// n_slot_ids must lie in [1, kMetaB] (else hipErrorInvalidValue).
hipError_t launch_remap(const int32_t *idx, int T, int k, const SlotView &view, int shared_slot,
                        int n_slot_ids, int32_t *meta, int32_t *bucket_pair, int32_t *items,
                        hipStream_t s);

struct GemvArgs {
  const uint8_t *slots;  // slot arena of the layer
  const uint4 *xq;       // decode gate/up: digit planes of x [T][d/32][4]
  const float *xs;       // decode gate/up: block scales [T][4 * xs_units(d/32)]
  const uint32_t *xp;    // matrix-core gate/up: activation pairs [T][d/8][8]
  const float *xscale;   // matrix-core gate/up: 2^e per token
  long long rec_bytes;   // slot stride
  long long off_q0, off_s0;  // nibbles / scales of the first matrix in a record
  long long off_q1, off_s1;  // second matrix (up projection) for the fused GLU
  int rows;              // output rows per expert
  int nb;                // blocks per row
  const float *in;       // decode down: input rows (h by pair) of nb*32 floats
  int in_by_pair;        // 0: input row = token of the pair, 1: input row = pair
  int T, k;              // tokens and top-k (pair -> token)
  const int32_t *meta;         // matrix-core path: buckets from launch_remap
  const int32_t *bucket_pair;
  const int32_t *items;        // matrix-core path: work items from launch_remap
  const int32_t *idx;          // router ids [T*k]
  int shared_slot;             // slot of the shared expert or -1
  const int32_t *bt;           // decode path: bucket list (launch_topk_decode)
  float *out;                  // [pairs][rows]
};

// Buckets built on the host (stream mode, decode path, after the slot fills):
// bucket b reads the expert record at src[b] (a device slot).
struct BucketTable {
  const uint8_t *src[kTabMax];
  int n;                                  // buckets, or -1 for "no table"
  uint8_t cnt[kTabMax];                   // pairs per bucket (<= kDecodeMaxTokens)
  uint8_t pairs[kTabMax][kDecodeMaxTokens];  // pair ids (< kDecodeMaxPairs)
};

// Decode GEMV over Q4 slot records with 4-bit integer dot products.  glu = 1:
// out[pair][r] = silu(G x) * (U x) from the router's digit planes and block
// scales (xq, xs);
// glu = 0: out[pair][r] = (D h)[r] with h = in[pair] (fp32), turned into digit
// planes with one scale per 32-element block inside each workgroup.  Buckets
// come from *tab when tab != nullptr, else from the list at a.bt; a grid of
// n_buckets columns covers at most that many buckets.
hipError_t launch_gemv(const GemvArgs &a, const BucketTable *tab, const GemvShape &sh, bool glu,
                       int n_buckets, hipStream_t s);

// Prefill grouped GEMM on the matrix cores (batches beyond the decode path).
// Work items from launch_remap; per workgroup of 8 waves one pass of up to
// kGemmTokens of a bucket's tokens and 128 weight rows of both GLU matrices
// (256 rows of the down matrix).  Each wave streams 32 rows' nibbles through
// registers (two K chunks in flight) and decodes them to exact binary16 (q - 8)
// operands; activations come as binary16 hi/lo pairs in the same K order (xp /
// xscale as prepared for the gate/up GEMM, indexed by token for gate/up and by
// pair for down), staged per chunk in LDS.  Each 32-weight block is one pair of
// v_mfma_f32_16x16x32_f16 (hi, lo) per 16-token tile and 16 rows, and its scale
// is applied per block in fp32.  glu: out[p][r] = silu(g) * u; else out = M in.
// A grid of n_items columns covers at most that many work items (more than
// 65535: hipErrorInvalidValue).
hipError_t launch_mfma(const GemvArgs &a, bool glu, int n_items, hipStream_t s);

// Binary16 hi/lo pairs and power-of-two scale of `rows` float rows of length K
// (the preparation the router does for x), for the down GEMM's input h.
hipError_t launch_prep_pairs(const float *in, int rows, int K, uint32_t *xp, float *xscale,
                             hipStream_t s);

// Copies n expert records (bytes16 x 16 bytes each) from the page-locked host
// arena into device slots; `per_expert` workgroups each read one contiguous
// chunk, two 16-byte loads in flight per lane (more requests in flight read
// page-locked memory more slowly).
struct PullList {
  const uint8_t *src[kTabMax];
  uint8_t *dst[kTabMax];
  int n;
  int per_expert;
  long long bytes16;
};
hipError_t launch_pull(const PullList &l, hipStream_t s);

// out[t] = sum_j [pair on GPU] w * y[t*k+j] (j ascending) + shared + host part,
// where a pair is on the GPU when all_gpu, else when pair_slot[p] >= 0 (if
// pair_slot != nullptr), else when view.slot[idx[p]] >= 0.
hipError_t launch_combine(const float *y, const float *w, const int32_t *idx,
                          const SlotView &view, int all_gpu, const int32_t *pair_slot, int T,
                          int k, int d, int n_shared, const float *host_part, float *out,
                          float *dbg_gpu, hipStream_t s);

// Device address of the fixed scratch array (kNoAllocScratchBytes, one per
// device, held until the process ends) on the current device.  The first call
// on a device looks the address up with that device current and keeps it; the
// array's host-side name is not a device address and is never used on the host.
hipError_t noalloc_scratch(void **ptr);

}  // namespace moe
