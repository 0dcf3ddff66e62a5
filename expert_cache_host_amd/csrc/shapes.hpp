// Limits and launch shapes shared by the kernels and the host runtime (plain
// C++, no HIP types: the host-only builds include it too).
#pragma once
#include <cstddef>
#include <cstdint>

namespace moe {

constexpr int kMaxExperts = 512;
// Decode path: at most this many (token, rank) pairs per call, tokens <= 4.
constexpr int kDecodeMaxPairs = 64;
constexpr int kDecodeMaxTokens = 4;
constexpr int kMetaB = 520;  // bucket capacity of the meta block (>= kMaxExperts + 1)
constexpr int kMetaInts = 2 + 3 * kMetaB;

// Decode bucket list: buckets[0] = count; bucket b at buckets + 1 + b*kBucketInts
// holds {slot, pair count, pairs[kDecodeMaxTokens]} (pairs ascending, the last
// one repeated past the count).
constexpr int kBucketInts = 6;  // 2 + kDecodeMaxTokens
static_assert(kBucketInts == 2 + kDecodeMaxTokens, "bucket list entry size");

// Buckets of one host-built table (stream mode, decode path, after the slot
// fills) and slot records of one pull launch.
constexpr int kTabMax = 32;

// Tokens of one bucket that one matrix-core workgroup takes per pass.
constexpr int kGemmTokens = 32;

// 16-byte units of one token's decode block scales: nb floats padded to a
// multiple of 4 (the row stride of the block scales is 4 * xs_units(nb) floats).
inline constexpr int xs_units(int nb) { return (nb + 3) / 4; }

// Work items of the matrix-core GEMM for `pairs` pairs in at most `buckets`
// buckets: one per started pass of kGemmTokens tokens of a bucket.
inline int gemm_items_bound(int buckets, int pairs) {
  return buckets + (pairs + kGemmTokens - 1) / kGemmTokens;
}

struct GemvShape {
  int G;        // lanes per row
  int KS;       // waves of a workgroup that split a row's K blocks
  int R;        // rows per lane
  int TT;       // tokens per bucket pass (1, 2 or 4)
  int NW;       // waves per workgroup
  int rows_wg;  // rows per workgroup
};

// Decode GEMV shape for rows of nb blocks and buckets of up to `tokens` pairs:
// glu = gate/up (+ SwiGLU), else down.
GemvShape choose_gemv(bool glu, int nb, int tokens);

// Dynamic LDS of one decode GEMV workgroup: the bucket's activation planes and
// block scales and the workgroup's row scales.
size_t gemv_lds_bytes(bool glu, int nb, int tokens);

}  // namespace moe
