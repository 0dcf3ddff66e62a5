// Top-k selection and gating weights on the host, from the router logits the
// GPU publishes (plain C++, no HIP).
//
// The selection is the one the GPU's top-k kernel makes ("How it works",
// llama.cpp + MoE expert cache, steps 1-2: the router's top-k experts decide
// where each token goes): per token, the k largest logits ordered by
// decreasing value, equal values to the lower expert id (-0 equals +0).  On the
// same float32 logits both sides pick the same ids in the same order, so the
// host plans exactly the experts the GPU's buckets hold.  The gating weights
// are the softmax over all E logits, renormalised over the k when norm_topk;
// computed here in binary64 and rounded to float32 (they weight the host's own
// partial sum; the GPU's float32 weights weight its part).
#pragma once
#include <cstdint>

namespace moe {

// z [T][E] float32, idx / w [T][k]; 1 <= k <= E <= kMaxExperts.
void host_topk(const float *z, int32_t T, int32_t E, int32_t k, int32_t norm_topk, int32_t *idx,
               float *w);

}  // namespace moe
