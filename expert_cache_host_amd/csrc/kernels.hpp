// Launchers of the gfx950 kernels (host-callable; no device code here).
#pragma once
#include <hip/hip_runtime_api.h>

#include <cstdint>

namespace moe {

constexpr int kMaxExperts = 512;
constexpr int kMetaB = 520;  // bucket capacity of the meta block (>= kMaxExperts + 1)
constexpr int kMetaInts = 2 + 3 * kMetaB;

// Expert -> slot table of one stage, passed by value as a kernel argument so
// that each launch carries its own table (no copy, no reuse hazard).
struct SlotView {
  int16_t slot[kMaxExperts];
};

// z[t][e] = x[t] . W[e] (+ b[e]) in the fixed fp32 order.
hipError_t launch_router(const float *x, int T, int d, const float *W, const float *bias, int E,
                         float *z, hipStream_t s);

// Per token: k largest logits (ties to the lower id), softmax gating weights;
// clears pair_gpu[t*k + j].
hipError_t launch_topk(const float *z, int T, int E, int k, int norm_topk, int32_t *idx,
                       float *w, int32_t *pair_gpu, hipStream_t s);

// Expert -> slot remap of the routed pairs (plus one shared pair per token when
// shared_slot >= 0) and stable bucketing per slot.  meta: [0] = buckets,
// [1] = pairs, [2 + b] = slot, [2 + kMetaB + b] = first pair position,
// [2 + 2 kMetaB + b] = pair count; bucket_pair holds pair ids grouped by bucket,
// ascending within a bucket.  Sets pair_gpu[p] = 1 for bucketed routed pairs.
hipError_t launch_remap(const int32_t *idx, int T, int k, const SlotView &view, int shared_slot,
                        int n_slot_ids, int32_t *meta, int32_t *bucket_pair, int32_t *pair_gpu,
                        hipStream_t s);

struct GemvArgs {
  const uint8_t *slots;  // slot arena of the layer
  long long rec_bytes;   // slot stride
  long long off_q0, off_s0;  // nibbles / scales of the first matrix in a record
  long long off_q1, off_s1;  // second matrix (up projection) for the fused GLU
  int rows;              // output rows per expert
  int nb;                // blocks per row
  const float *in;       // input rows of nb*32 floats
  int in_by_pair;        // 0: input row = token of the pair, 1: input row = pair
  int T, k;              // tokens and top-k (pair -> token)
  const int32_t *meta;
  const int32_t *bucket_pair;
  float *out;            // [pairs][rows]
};

struct GemvShape {
  int G, V, TT, R;
};

// Chooses lanes per row G, words per unit V, token tile TT and rows per lane R.
GemvShape choose_gemv(int rows, int nb, int n_buckets, int max_tokens);

// glu = 1: out = silu(G x) * (U x) ; glu = 0: out = M x.
hipError_t launch_gemv(const GemvArgs &a, const GemvShape &sh, bool glu, int n_buckets,
                       hipStream_t s);

// out[t] = sum_j pair_gpu ? w * y[t*k+j] : 0 (j ascending) + shared + host part.
hipError_t launch_combine(const float *y, const float *w, const int32_t *pair_gpu, int T, int k,
                          int d, int n_shared, const float *host_part, float *out,
                          float *dbg_gpu, hipStream_t s);

}  // namespace moe
