// Device workspace of one layer call (plain C++, no HIP calls).
//
// A call's kernels index a handful of device buffers: the router logits, the
// routing, the prepared activations, the expert hidden rows h and outputs y,
// and either the decode GEMV's bucket list or the matrix-core GEMM's bucket
// metadata.  ws_layout() decides which path a call takes and carves every
// region it needs from one base address at 256-byte boundaries; ws_check()
// restates, launch by launch, what each kernel indexes and verifies that the
// layout covers it.  moe_layer_forward carves a device arena grown on demand;
// moe_layer_forward_noalloc carves the library's fixed scratch array and
// rejects calls whose layout does not fit it.
#pragma once
#include <cstddef>
#include <cstdint>

#include "shapes.hpp"

namespace moe {

// Bytes of the fixed per-device scratch array of moe_layer_forward_noalloc.
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
// Tokens per call that moe_layer_forward_noalloc accepts (its page-locked
// routing and host-partial buffers are sized for this at create).
constexpr int kNoAllocMaxTokens = kDecodeMaxTokens;
// Dynamic LDS a decode GEMV workgroup may use.
constexpr size_t kDecodeLdsBudget = 60 * 1024;
constexpr size_t kWsAlign = 256;

struct WsParams {
  int T;         // tokens of the call
  int E;         // routed experts
  int k;         // top-k
  int n_shared;  // resident shared experts (0 or 1)
  int d, f;      // d_model, d_ff
};

struct WsRegion {
  size_t off = 0, bytes = 0;
};

struct WsLayout {
  bool decode = false;  // decode GEMV path, else the matrix-core GEMM
  int pairs = 0;        // T*k routed pairs + T*n_shared shared pairs
  // every call
  WsRegion z, idx, w, h, y;
  // decode path
  WsRegion xq, xs, buckets, pair_slot;
  // matrix-core path
  WsRegion meta, bucket_pair, items, xp, xscale, hp, hscale;
  size_t total = 0;  // bytes from the base address
};

// True when the call takes the decode GEMV: at most kDecodeMaxTokens tokens,
// at most kDecodeMaxPairs pairs, and both GEMV workgroups' LDS within budget.
bool decode_path(const WsParams &p);

// Regions of the call's path (the other path's regions stay empty).
WsLayout ws_layout(const WsParams &p);

// nullptr when every region a launch of this call indexes lies inside the
// layout, is at least as large as that launch reads or writes, starts on a
// kWsAlign boundary and overlaps no other region; else the name of the first
// region that fails.
const char *ws_check(const WsLayout &L, const WsParams &p);

}  // namespace moe
