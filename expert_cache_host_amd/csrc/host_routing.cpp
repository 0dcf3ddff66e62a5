#include "host_routing.hpp"

#include <algorithm>
#include <cmath>
#include <cstring>

#include "shapes.hpp"

namespace moe {

namespace {

// The GPU top-k's order: the bits of v + 0 (so -0 and +0 are one value) mapped
// to an unsigned key that orders as the floats do, NaNs included (a NaN with
// the sign bit clear ranks above +inf, one with it set below -inf).  Integer
// keys make the comparison a strict weak ordering for every input.
inline uint32_t order_key(float v) {
  const float u = v + 0.0f;
  uint32_t b;
  std::memcpy(&b, &u, 4);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

}  // namespace

void host_topk(const float *z, int32_t T, int32_t E, int32_t k, int32_t norm_topk, int32_t *idx,
               float *w) {
  int32_t order[kMaxExperts];
  uint32_t key[kMaxExperts];
  for (int32_t t = 0; t < T; ++t) {
    const float *zt = z + (int64_t)t * E;
    for (int32_t e = 0; e < E; ++e) {
      order[e] = e;
      key[e] = order_key(zt[e]);
    }
    // larger key first, equal keys (-0 == +0) to the lower id
    std::partial_sort(order, order + k, order + E, [&key](int32_t a, int32_t b) {
      return key[a] > key[b] || (key[a] == key[b] && a < b);
    });
    const double zmax = zt[order[0]];
    double den = 0.0;
    if (norm_topk) {
      for (int32_t j = 0; j < k; ++j) den += std::exp((double)zt[order[j]] - zmax);
    } else {
      for (int32_t e = 0; e < E; ++e) den += std::exp((double)zt[e] - zmax);
    }
    for (int32_t j = 0; j < k; ++j) {
      idx[(int64_t)t * k + j] = order[j];
      w[(int64_t)t * k + j] = (float)(std::exp((double)zt[order[j]] - zmax) / den);
    }
  }
}

}  // namespace moe
