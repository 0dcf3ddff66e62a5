#include "host_routing.hpp"

#include <algorithm>
#include <cmath>

#include "shapes.hpp"

namespace moe {

void host_topk(const float *z, int32_t T, int32_t E, int32_t k, int32_t norm_topk, int32_t *idx,
               float *w) {
  int32_t order[kMaxExperts];
  for (int32_t t = 0; t < T; ++t) {
    const float *zt = z + (int64_t)t * E;
    for (int32_t e = 0; e < E; ++e) order[e] = e;
    // larger value first, equal values (-0 == +0) to the lower id
    std::partial_sort(order, order + k, order + E, [zt](int32_t a, int32_t b) {
      return zt[a] > zt[b] || (zt[a] == zt[b] && a < b);
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
