// Streaming-read ceiling of the GPU at the expert GEMV's sizes: each
// workgroup reads a contiguous run of a buffer with 16-byte loads (plain or
// nontemporal) and folds it into one word, timed between two HIP events per
// launch as the library times its kernels.  Prints one JSON line per (size,
// load kind, workgroup count): the mean and best of 40 launches.  Runs of up to
// 256 MiB take four windows a quarter of the 1 GiB buffer apart in turn; at 64
// MiB and below the four windows fit the 256 MB last-level cache together, so
// those figures may include cache hits and overstate the HBM rate.
//
//   hipcc --offload-arch=gfx950 -O3 -Xclang -target-feature -Xclang -packed-fp32-ops \
//       expert_cache_host_amd/probes/readbw.hip -o readbw && ./readbw
#include <hip/hip_runtime.h>
#include <cstdio>
#include <cstdlib>
#include <vector>
#define CK(x) do { hipError_t e_ = (x); if (e_) { printf("err %s line %d\n", hipGetErrorString(e_), __LINE__); exit(1); } } while (0)
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
template <int NT, int U>
__global__ __launch_bounds__(256) void rd(const uint4 *p, size_t n16, size_t per_wg, unsigned *out) {
  const size_t b0 = (size_t)blockIdx.x * per_wg, b1 = b0 + per_wg < n16 ? b0 + per_wg : n16;
  unsigned acc = 0;
  for (size_t i = b0 + threadIdx.x; i < b1; i += 256 * U) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t j = i + 256 * u;
      if (j < b1) {
        if (NT) { u32x4_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p + j)); v[u] = make_uint4(t.x, t.y, t.z, t.w); }
        else v[u] = p[j];
      } else v[u] = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x12345678u) out[blockIdx.x] = acc;
}
int main() {
  const size_t maxb = (size_t)1 << 30;
  uint4 *p; unsigned *o;
  CK(hipMalloc(&p, maxb + (1 << 20)));
  CK(hipMalloc(&o, 1 << 22));
  CK(hipMemset(p, 1, maxb));
  hipEvent_t e0, e1; CK(hipEventCreate(&e0)); CK(hipEventCreate(&e1));
  const size_t sizes[] = {16u << 20, 32u << 20, 64u << 20, 128u << 20, 192u << 20, 256u << 20, 1024u << 20};
  const int wgs[] = {512, 1024, 2048, 4096, 8192};
  for (size_t sz : sizes) {
    for (int nt = 0; nt < 2; ++nt) for (int g : wgs) {
      const size_t n16 = sz / 16, per = (n16 + g - 1) / g;
      // four windows a quarter of the buffer apart, in turn
      const int reps = 40;
      float best = 1e9, tot = 0;
      for (int r = 0; r < reps + 5; ++r) {
        const size_t off = ((size_t)(r % 4) * (maxb / 4)) / 16;
        const size_t nn = sz <= maxb / 4 ? n16 : n16;
        const uint4 *q = sz <= maxb / 4 ? p + off : p;
        CK(hipEventRecord(e0));
        if (nt) hipLaunchKernelGGL((rd<1, 4>), dim3(g), dim3(256), 0, 0, q, nn, per, o);
        else hipLaunchKernelGGL((rd<0, 4>), dim3(g), dim3(256), 0, 0, q, nn, per, o);
        CK(hipEventRecord(e1));
        CK(hipEventSynchronize(e1));
        float ms; CK(hipEventElapsedTime(&ms, e0, e1));
        if (r >= 5) { tot += ms; if (ms < best) best = ms; }
      }
      const float avg = tot / reps;
      printf("{\"MB\": %.0f, \"nt\": %d, \"wgs\": %d, \"avg_us\": %.2f, \"best_us\": %.2f, \"avg_TBs\": %.3f, \"best_TBs\": %.3f}\n",
             sz / 1048576.0, nt, g, avg * 1e3, best * 1e3, sz / (avg * 1e-3) / 1e12, sz / (best * 1e-3) / 1e12);
      fflush(stdout);
    }
  }
  return 0;
}
