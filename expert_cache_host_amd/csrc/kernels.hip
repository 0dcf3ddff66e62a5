// gfx950 kernels of the routed-MoE layer served from per-layer expert slots.
//
// Wave64 throughout.  Q4 weights are read from the slot layout (layout.hpp):
// per matrix, row-major 16-byte nibble blocks and a separate binary16 scale
// array.  Element j of a block is the low nibble of byte j, element j+16 the
// high nibble; w = d * (q - 8).
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <algorithm>

#include "kernels.hpp"

namespace moe {

// ============================================================== router logits
// One wave per (expert, tile of TT tokens).  Lane l accumulates i = l, l+64, ...
// with the product and the sum rounded separately (no contraction), then a
// halving tree off = 32..1, then the bias: the fixed order that makes every
// top-k decision reproducible bit for bit on the host.
template <int TT>
__global__ __launch_bounds__(256) void router_kernel(const float *__restrict__ x, int T, int d,
                                                     const float *__restrict__ W,
                                                     const float *__restrict__ bias, int E,
                                                     float *__restrict__ z) {
#pragma clang fp contract(off)
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int t0 = blockIdx.y * TT;
  if (e >= E) return;
  const float *w = W + (long long)e * d;
  float p[TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) p[tt] = 0.0f;
  const int nt = min(TT, T - t0);
  for (int i = lane; i < d; i += 64) {
    const float wv = w[i];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      if (tt < nt) {
        const float prod = x[(long long)(t0 + tt) * d + i] * wv;
        p[tt] = p[tt] + prod;
      }
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      const float o = __shfl_down(p[tt], off, 64);
      if (lane < off) p[tt] = p[tt] + o;
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      if (tt < nt) z[(long long)(t0 + tt) * E + e] = bias ? p[tt] + bias[e] : p[tt];
    }
  }
}

hipError_t launch_router(const float *x, int T, int d, const float *W, const float *bias, int E,
                         float *z, hipStream_t s) {
  const int gx = (E + 3) / 4;
  if (T <= 1) {
    hipLaunchKernelGGL(router_kernel<1>, dim3(gx, T), dim3(256), 0, s, x, T, d, W, bias, E, z);
  } else if (T <= 4) {
    hipLaunchKernelGGL(router_kernel<4>, dim3(gx, 1), dim3(256), 0, s, x, T, d, W, bias, E, z);
  } else {
    hipLaunchKernelGGL(router_kernel<8>, dim3(gx, (T + 7) / 8), dim3(256), 0, s, x, T, d, W, bias,
                       E, z);
  }
  return hipGetLastError();
}

// ============================================================== top-k + softmax
// One wave per token; E <= 512, so each lane owns up to 8 logits.
__global__ __launch_bounds__(64) void topk_kernel(const float *__restrict__ z, int T, int E, int k,
                                                  int norm_topk, int32_t *__restrict__ idx,
                                                  float *__restrict__ w,
                                                  int32_t *__restrict__ pair_gpu) {
  const int t = blockIdx.x;
  const int lane = threadIdx.x;
  __shared__ int sel_e[64];
  __shared__ float sel_v[64];
  float v[8];
  bool ok[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int e = lane + 64 * c;
    ok[c] = e < E;
    v[c] = ok[c] ? z[(long long)t * E + e] : 0.0f;
  }
  for (int j = 0; j < k; ++j) {
    float bv = 0.0f;
    int be = E;  // sentinel: nothing yet
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      if (ok[c] && (be == E || v[c] > bv)) {
        bv = v[c];
        be = lane + 64 * c;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off, 64);
      const int oe = __shfl_xor(be, off, 64);
      if (oe != E && (be == E || ov > bv || (ov == bv && oe < be))) {
        bv = ov;
        be = oe;
      }
    }
#pragma unroll
    for (int c = 0; c < 8; ++c)
      if (lane + 64 * c == be) ok[c] = false;
    if (lane == 0) {
      sel_e[j] = be;
      sel_v[j] = bv;
    }
  }
  __syncthreads();
  const float zmax = sel_v[0];
  float ex = 0.0f;
  if (lane < k) ex = expf(sel_v[lane] - zmax);
  float denom;
  if (norm_topk) {
    denom = ex;
  } else {
    denom = 0.0f;
#pragma unroll
    for (int c = 0; c < 8; ++c)
      if (lane + 64 * c < E) denom += expf(v[c] - zmax);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) denom += __shfl_xor(denom, off, 64);
  if (lane < k) {
    idx[(long long)t * k + lane] = sel_e[lane];
    w[(long long)t * k + lane] = ex / denom;
    pair_gpu[(long long)t * k + lane] = 0;
  }
}

hipError_t launch_topk(const float *z, int T, int E, int k, int norm_topk, int32_t *idx, float *w,
                       int32_t *pair_gpu, hipStream_t s) {
  hipLaunchKernelGGL(topk_kernel, dim3(T), dim3(64), 0, s, z, T, E, k, norm_topk, idx, w,
                     pair_gpu);
  return hipGetLastError();
}

// ============================================================== remap + bucket
// One workgroup.  Counts pairs per slot, lays buckets out in slot order, then
// places pairs stably (ascending pair id inside a bucket), 256 pairs at a time.
__global__ __launch_bounds__(256) void remap_kernel(const int32_t *__restrict__ idx, int T, int k,
                                                    SlotView view, int shared_slot, int n_ids,
                                                    int32_t *__restrict__ meta,
                                                    int32_t *__restrict__ bucket_pair,
                                                    int32_t *__restrict__ pair_gpu) {
  __shared__ int cnt[kMetaB];
  __shared__ int base[kMetaB];
  __shared__ int run[kMetaB];
  __shared__ int sl[256];
  const int tid = threadIdx.x;
  const int P_routed = T * k;
  const int P = P_routed + (shared_slot >= 0 ? T : 0);
  for (int s = tid; s < n_ids; s += 256) {
    cnt[s] = 0;
    run[s] = 0;
  }
  __syncthreads();
  auto slot_of = [&](int p) -> int {
    return p < P_routed ? (int)view.slot[idx[p]] : shared_slot;
  };
  for (int p = tid; p < P; p += 256) {
    const int s = slot_of(p);
    if (s >= 0) atomicAdd(&cnt[s], 1);
  }
  __syncthreads();
  if (tid < 64) {
    const int lane = tid;
    const int chunk = (n_ids + 63) / 64;
    const int s0 = min(n_ids, lane * chunk), s1 = min(n_ids, s0 + chunk);
    int na = 0, np = 0;
    for (int s = s0; s < s1; ++s)
      if (cnt[s] > 0) {
        na++;
        np += cnt[s];
      }
    int ia = na, ip = np;  // inclusive scans
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int oa = __shfl_up(ia, off, 64), op = __shfl_up(ip, off, 64);
      if (lane >= off) {
        ia += oa;
        ip += op;
      }
    }
    int a = ia - na, q = ip - np;
    for (int s = s0; s < s1; ++s) {
      if (cnt[s] > 0) {
        meta[2 + a] = s;
        meta[2 + kMetaB + a] = q;
        meta[2 + 2 * kMetaB + a] = cnt[s];
        base[s] = q;
        q += cnt[s];
        a++;
      }
    }
    if (lane == 63) {
      meta[0] = ia;
      meta[1] = ip;
    }
  }
  __syncthreads();
  for (int c = 0; c < P; c += 256) {
    const int p = c + tid;
    const int s = p < P ? slot_of(p) : -1;
    sl[tid] = s;
    __syncthreads();
    if (s >= 0) {
      int rank = 0;
      for (int i = 0; i < tid; ++i) rank += (sl[i] == s) ? 1 : 0;
      bucket_pair[base[s] + run[s] + rank] = p;
      if (p < P_routed) pair_gpu[p] = 1;
    }
    __syncthreads();
    if (s >= 0) atomicAdd(&run[s], 1);
    __syncthreads();
  }
}

hipError_t launch_remap(const int32_t *idx, int T, int k, const SlotView &view, int shared_slot,
                        int n_slot_ids, int32_t *meta, int32_t *bucket_pair, int32_t *pair_gpu,
                        hipStream_t s) {
  hipLaunchKernelGGL(remap_kernel, dim3(1), dim3(256), 0, s, idx, T, k, view, shared_slot,
                     n_slot_ids, meta, bucket_pair, pair_gpu);
  return hipGetLastError();
}

// ============================================================== Q4 grouped GEMV
// Workgroup = 4 waves, one slot bucket (blockIdx.y) and a tile of rows
// (blockIdx.x).  In a wave, G lanes share a row and RG = 64/G rows run side by
// side; each lane walks the row's units u = lane%G, +G, ... where a unit is V
// consecutive 32-bit nibble words (V = 4: a whole block, V = 2: half a block);
// R rows per lane reuse the unit's activations from registers.  The -8 offset
// is folded in as d * (sum q x - 8 sum x).  Partial sums meet across the G
// lanes with xor shuffles.
__device__ __forceinline__ float word_dot(uint32_t q, const float4 &xl, const float4 &xh) {
  const uint32_t lo = q & 0x0F0F0F0Fu;
  const uint32_t hi = (q >> 4) & 0x0F0F0F0Fu;
  float acc = (float)(lo & 0xFFu) * xl.x;
  acc += (float)((lo >> 8) & 0xFFu) * xl.y;
  acc += (float)((lo >> 16) & 0xFFu) * xl.z;
  acc += (float)(lo >> 24) * xl.w;
  acc += (float)(hi & 0xFFu) * xh.x;
  acc += (float)((hi >> 8) & 0xFFu) * xh.y;
  acc += (float)((hi >> 16) & 0xFFu) * xh.z;
  acc += (float)(hi >> 24) * xh.w;
  return acc;
}

template <int V>
__device__ __forceinline__ void load_words(const uint32_t *p, uint32_t (&q)[V]) {
  if constexpr (V == 4) {
    const uint4 v = *reinterpret_cast<const uint4 *>(p);
    q[0] = v.x;
    q[1] = v.y;
    q[2] = v.z;
    q[3] = v.w;
  } else {
    const uint2 v = *reinterpret_cast<const uint2 *>(p);
    q[0] = v.x;
    q[1] = v.y;
  }
}

__device__ __forceinline__ float silu_f(float v) { return v / (1.0f + expf(-v)); }

template <int G, int V, int TT, int R, bool GLU>
__global__ __launch_bounds__(256) void q4_gemv_kernel(GemvArgs a) {
  constexpr int RG = 64 / G;
  constexpr int ROWS_WAVE = R * RG;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int bucket = blockIdx.y;
  if (bucket >= a.meta[0]) return;
  const int slot = a.meta[2 + bucket];
  const int off = a.meta[2 + kMetaB + bucket];
  const int cnt = a.meta[2 + 2 * kMetaB + bucket];
  const uint8_t *rec = a.slots + (long long)slot * a.rec_bytes;
  const int grp = lane / G, gl = lane % G;
  const int row0 = (blockIdx.x * 4 + wave) * ROWS_WAVE + grp;
  const int row_words = a.nb * 4;
  const int units = row_words / V;
  const int K = a.nb * 32;
  const uint32_t *q0b = reinterpret_cast<const uint32_t *>(rec + a.off_q0);
  const __half *s0b = reinterpret_cast<const __half *>(rec + a.off_s0);
  const uint32_t *q1b = reinterpret_cast<const uint32_t *>(rec + a.off_q1);
  const __half *s1b = reinterpret_cast<const __half *>(rec + a.off_s1);

  for (int tg = 0; tg < cnt; tg += TT) {
    const int nt = min(TT, cnt - tg);
    const float *xin[TT];
    int prs[TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      const int p = a.bucket_pair[off + tg + min(tt, nt - 1)];
      prs[tt] = p;
      const int r = a.in_by_pair ? p : (p < a.T * a.k ? p / a.k : p - a.T * a.k);
      xin[tt] = a.in + (long long)r * K;
    }
    float acc0[R][TT], acc1[R][TT];
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        acc0[i][tt] = 0.0f;
        acc1[i][tt] = 0.0f;
      }
    for (int u = gl; u < units; u += G) {
      const int w0 = u * V;
      const int blk = w0 >> 2;
      float4 xl[TT][V], xh[TT][V];
      float xs[TT];
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        xs[tt] = 0.0f;
#pragma unroll
        for (int v = 0; v < V; ++v) {
          const int wb = (w0 + v) & 3;
          const float *xp = xin[tt] + blk * 32 + 4 * wb;
          xl[tt][v] = *reinterpret_cast<const float4 *>(xp);
          xh[tt][v] = *reinterpret_cast<const float4 *>(xp + 16);
          xs[tt] += (xl[tt][v].x + xl[tt][v].y) + (xl[tt][v].z + xl[tt][v].w) +
                    (xh[tt][v].x + xh[tt][v].y) + (xh[tt][v].z + xh[tt][v].w);
        }
      }
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const int r = row0 + i * RG;
        if (r < a.rows) {
          uint32_t q0[V];
          load_words<V>(q0b + (long long)r * row_words + w0, q0);
          const float sc0 = __half2float(s0b[(long long)r * a.nb + blk]);
          uint32_t q1[V];
          float sc1 = 0.0f;
          if constexpr (GLU) {
            load_words<V>(q1b + (long long)r * row_words + w0, q1);
            sc1 = __half2float(s1b[(long long)r * a.nb + blk]);
          }
#pragma unroll
          for (int tt = 0; tt < TT; ++tt) {
            float d0 = 0.0f;
#pragma unroll
            for (int v = 0; v < V; ++v) d0 += word_dot(q0[v], xl[tt][v], xh[tt][v]);
            acc0[i][tt] += sc0 * (d0 - 8.0f * xs[tt]);
            if constexpr (GLU) {
              float d1 = 0.0f;
#pragma unroll
              for (int v = 0; v < V; ++v) d1 += word_dot(q1[v], xl[tt][v], xh[tt][v]);
              acc1[i][tt] += sc1 * (d1 - 8.0f * xs[tt]);
            }
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
#pragma unroll
        for (int o = G / 2; o >= 1; o >>= 1) {
          acc0[i][tt] += __shfl_xor(acc0[i][tt], o, 64);
          if constexpr (GLU) acc1[i][tt] += __shfl_xor(acc1[i][tt], o, 64);
        }
      }
    if (gl == 0) {
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const int r = row0 + i * RG;
        if (r < a.rows) {
#pragma unroll
          for (int tt = 0; tt < TT; ++tt) {
            if (tt < nt) {
              const float val = GLU ? silu_f(acc0[i][tt]) * acc1[i][tt] : acc0[i][tt];
              a.out[(long long)prs[tt] * a.rows + r] = val;
            }
          }
        }
      }
    }
  }
}

GemvShape choose_gemv(int rows, int nb, int n_buckets, int max_tokens) {
  GemvShape best{64, 4, 1, 1};
  double best_eff = -1.0;
  const int gs[3] = {64, 32, 16};
  const int vs[2] = {4, 2};
  for (int vi = 0; vi < 2; ++vi)
    for (int gi = 0; gi < 3; ++gi) {
      const int V = vs[vi], G = gs[gi];
      const int units = nb * 4 / V;
      const int ni = (units + G - 1) / G;
      const double eff = (double)units / (double)(G * ni) + 1e-3 * V + 1e-5 * G;
      if (eff > best_eff) {
        best_eff = eff;
        best.G = G;
        best.V = V;
      }
    }
  best.TT = max_tokens <= 1 ? 1 : (max_tokens <= 2 ? 2 : 4);
  const int RG = 64 / best.G;
  best.R = 1;
  const int rs[2] = {4, 2};
  for (int ri = 0; ri < 2; ++ri) {
    const int R = rs[ri];
    const long long waves = (long long)n_buckets * ((rows + R * RG - 1) / (R * RG));
    if (waves >= 4096) {
      best.R = R;
      break;
    }
  }
  return best;
}

template <int G, int V, int TT, int R, bool GLU>
static hipError_t launch_one(const GemvArgs &a, int n_buckets, hipStream_t s) {
  constexpr int rows_blk = 4 * R * (64 / G);
  const dim3 grid((a.rows + rows_blk - 1) / rows_blk, n_buckets);
  hipLaunchKernelGGL((q4_gemv_kernel<G, V, TT, R, GLU>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int G, int V, int TT, bool GLU>
static hipError_t launch_r(const GemvArgs &a, int R, int nbk, hipStream_t s) {
  switch (R) {
    case 4: return launch_one<G, V, TT, 4, GLU>(a, nbk, s);
    case 2: return launch_one<G, V, TT, 2, GLU>(a, nbk, s);
    default: return launch_one<G, V, TT, 1, GLU>(a, nbk, s);
  }
}

template <int G, int V, bool GLU>
static hipError_t launch_t(const GemvArgs &a, const GemvShape &sh, int nbk, hipStream_t s) {
  switch (sh.TT) {
    case 1: return launch_r<G, V, 1, GLU>(a, sh.R, nbk, s);
    case 2: return launch_r<G, V, 2, GLU>(a, sh.R, nbk, s);
    default: return launch_r<G, V, 4, GLU>(a, sh.R, nbk, s);
  }
}

template <int G, bool GLU>
static hipError_t launch_v(const GemvArgs &a, const GemvShape &sh, int nbk, hipStream_t s) {
  return sh.V == 4 ? launch_t<G, 4, GLU>(a, sh, nbk, s) : launch_t<G, 2, GLU>(a, sh, nbk, s);
}

template <bool GLU>
static hipError_t launch_g(const GemvArgs &a, const GemvShape &sh, int nbk, hipStream_t s) {
  switch (sh.G) {
    case 64: return launch_v<64, GLU>(a, sh, nbk, s);
    case 32: return launch_v<32, GLU>(a, sh, nbk, s);
    default: return launch_v<16, GLU>(a, sh, nbk, s);
  }
}

hipError_t launch_gemv(const GemvArgs &a, const GemvShape &sh, bool glu, int n_buckets,
                       hipStream_t s) {
  if (n_buckets <= 0) return hipSuccess;
  return glu ? launch_g<true>(a, sh, n_buckets, s) : launch_g<false>(a, sh, n_buckets, s);
}

// ============================================================== combine
__global__ __launch_bounds__(256) void combine_kernel(const float *__restrict__ y,
                                                      const float *__restrict__ w,
                                                      const int32_t *__restrict__ pair_gpu, int T,
                                                      int k, int d, int n_shared,
                                                      const float *__restrict__ host_part,
                                                      float *__restrict__ out,
                                                      float *__restrict__ dbg_gpu) {
  const int t = blockIdx.y;
  const int i = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= d) return;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < k; ++j) {
    const long long p = (long long)t * k + j;
    if (pair_gpu[p]) {
      const float wv = w[p];
      const float4 yv = *reinterpret_cast<const float4 *>(y + p * d + i);
      acc.x += wv * yv.x;
      acc.y += wv * yv.y;
      acc.z += wv * yv.z;
      acc.w += wv * yv.w;
    }
  }
  if (n_shared) {
    const float4 yv = *reinterpret_cast<const float4 *>(y + ((long long)T * k + t) * d + i);
    acc.x += yv.x;
    acc.y += yv.y;
    acc.z += yv.z;
    acc.w += yv.w;
  }
  if (dbg_gpu) *reinterpret_cast<float4 *>(dbg_gpu + (long long)t * d + i) = acc;
  if (host_part) {
    const float4 hv = *reinterpret_cast<const float4 *>(host_part + (long long)t * d + i);
    acc.x += hv.x;
    acc.y += hv.y;
    acc.z += hv.z;
    acc.w += hv.w;
  }
  *reinterpret_cast<float4 *>(out + (long long)t * d + i) = acc;
}

hipError_t launch_combine(const float *y, const float *w, const int32_t *pair_gpu, int T, int k,
                          int d, int n_shared, const float *host_part, float *out,
                          float *dbg_gpu, hipStream_t s) {
  const dim3 grid((d / 4 + 255) / 256, T);
  hipLaunchKernelGGL(combine_kernel, grid, dim3(256), 0, s, y, w, pair_gpu, T, k, d, n_shared,
                     host_part, out, dbg_gpu);
  return hipGetLastError();
}

}  // namespace moe
