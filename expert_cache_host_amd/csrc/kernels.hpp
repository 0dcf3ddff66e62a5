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

// z[t][e] = x[t] . W[e] (+ b[e]) in the fixed fp32 order.  When xp != nullptr
// every wave also derives its tokens' activation scale and the waves together
// prepare the activations for the gate/up kernel: a power-of-two scale 2^-e
// that keeps |x| below 2^14 (xscale[t] = 2^e); the scaled x as binary16 hi and
// lo pairs in the order the nibble decoder yields weights (for 32-bit word j of
// block b = j/4 and g = 4*(j%4): (x[g],x[g+2]), (x[g+16],x[g+18]),
// (x[g+1],x[g+3]), (x[g+17],x[g+19]) of the block, hi then lo); and the sum of
// each word's 8 scaled values (xsw).
hipError_t launch_router(const float *x, int T, int d, const float *W, const float *bias, int E,
                         float *z, uint32_t *xp, float *xsw, float *xscale, hipStream_t s);

// Per token: k largest logits (ties to the lower id), softmax gating weights,
// written to device memory (idx, w) and to page-locked host memory (h_idx, h_w).
hipError_t launch_topk(const float *z, int T, int E, int k, int norm_topk, int32_t *idx,
                       float *w, int32_t *h_idx, float *h_w, hipStream_t s);

// Expert -> slot remap of the routed pairs (plus one shared pair per token when
// shared_slot >= 0) and stable bucketing per slot, for batches beyond the
// decode path.  meta: [0] = buckets, [1] = pairs, [2 + b] = slot,
// [2 + kMetaB + b] = first pair position, [2 + 2 kMetaB + b] = pair count;
// bucket_pair holds pair ids grouped by bucket, ascending within a bucket.
hipError_t launch_remap(const int32_t *idx, int T, int k, const SlotView &view, int shared_slot,
                        int n_slot_ids, int32_t *meta, int32_t *bucket_pair, hipStream_t s);

struct GemvArgs {
  const uint8_t *slots;  // slot arena of the layer
  const uint32_t *xp;    // gate/up: activation pairs [T][d/8][8]
  const float *xsw;      // gate/up: per-word sums [T][d/8]
  const float *xscale;   // gate/up: 2^e per token
  long long rec_bytes;   // slot stride
  long long off_q0, off_s0;  // nibbles / scales of the first matrix in a record
  long long off_q1, off_s1;  // second matrix (up projection) for the fused GLU
  int rows;              // output rows per expert
  int nb;                // blocks per row
  const float *in;       // input rows of nb*32 floats
  int in_by_pair;        // 0: input row = token of the pair, 1: input row = pair
  int T, k;              // tokens and top-k (pair -> token)
  const int32_t *meta;         // buckets from launch_remap, or nullptr: decode path
  const int32_t *bucket_pair;
  const int32_t *idx;          // decode path: router ids [T*k]
  int shared_slot;             // decode path: slot of the shared expert or -1
  float *out;                  // [pairs][rows]
};

// Decode path: at most this many (token, rank) pairs per call, tokens <= 4.
constexpr int kDecodeMaxPairs = 64;
constexpr int kDecodeMaxTokens = 4;

// Buckets built on the host (stream mode, decode path, after the slot fills):
// bucket b reads the expert record at src[b] (a device slot).
constexpr int kTabMax = 32;
struct BucketTable {
  const uint8_t *src[kTabMax];
  int n;                                  // buckets, or -1 for "no table"
  uint8_t cnt[kTabMax];                   // pairs per bucket (<= kDecodeMaxTokens)
  uint8_t pairs[kTabMax][kDecodeMaxTokens];  // pair ids (< kDecodeMaxPairs)
};

struct GemvShape {
  int G, V, TT, R;
  int KS;  // waves of a workgroup that split one row group's K (down: 1 or 4; gate/up: 4)
};

// Chooses lanes per row G, words per unit V, token tile TT and rows per lane R
// for the gate/up kernel (glu, K split over the 4 waves of a workgroup) or the
// down kernel (whole K per wave).
GemvShape choose_gemv(bool glu, int rows, int nb, int n_buckets, int max_tokens);

// glu = 1: out = silu(G x) * (U x) from the prepared activation pairs;
// glu = 0: out = M in, in float32.  On the decode path (a.meta == nullptr) each
// workgroup finds its bucket itself from a.idx and `view`: bucket b is the b-th
// pair (in pair order) whose slot has not appeared before.
// With tab != nullptr the buckets come from *tab instead.

hipError_t launch_gemv(const GemvArgs &a, const SlotView &view, const BucketTable *tab,
                       const GemvShape &sh, bool glu, int n_buckets, hipStream_t s);

// Prefill grouped GEMM on the matrix cores (batches beyond the decode path).
// Buckets from launch_remap; per workgroup 64 weight rows of one bucket's expert
// and up to 64 of its tokens at a time.  Weights are decoded chunk by chunk into
// LDS as binary16 (1024 + q), activations come as binary16 hi/lo pairs in the
// same K order (xp / xsw / xscale as prepared for the gate/up GEMV, indexed by
// token for gate/up and by pair for down), each 32-weight block is one pair of
// v_mfma_f32_16x16x32_f16 (hi, lo) and its scale and the 1032 * sum(x) offset are
// applied per block in fp32.  glu: out[p][r] = silu(g) * u; else out = M in.
hipError_t launch_mfma(const GemvArgs &a, bool glu, int n_buckets, hipStream_t s);

// Binary16 hi/lo pairs, word sums and power-of-two scale of `rows` float rows of
// length K (the preparation the router does for x), for the down GEMM's input h.
hipError_t launch_prep_pairs(const float *in, int rows, int K, uint32_t *xp, float *xsw,
                             float *xscale, hipStream_t s);

// Copies n expert records (bytes16 x 16 bytes each) from the page-locked host
// arena into device slots; `per_expert` workgroups each read one contiguous
// chunk with wide loads (PCIe reads stay long and in flight).
struct PullList {
  const uint8_t *src[kTabMax];
  uint8_t *dst[kTabMax];
  int n;
  int per_expert;
  long long bytes16;
};
hipError_t launch_pull(const PullList &l, hipStream_t s);

// out[t] = sum_j [pair on GPU] w * y[t*k+j] (j ascending) + shared + host part,
// where a pair is on the GPU when all_gpu or view.slot[idx] >= 0.
hipError_t launch_combine(const float *y, const float *w, const int32_t *idx,
                          const SlotView &view, int all_gpu, int T, int k, int d, int n_shared,
                          const float *host_part, float *out, float *dbg_gpu, hipStream_t s);

}  // namespace moe
