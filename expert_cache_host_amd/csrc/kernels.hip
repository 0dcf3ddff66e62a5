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

// ============================================================== small helpers

__device__ __forceinline__ uint32_t pack_h2(float a, float b) {
  const _Float16 ha = (_Float16)a, hb = (_Float16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, ha) |
         ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
}

template <int CTRL>
__device__ __forceinline__ int mov_dpp(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, true);
}

// (value, id) order for top-k: larger value first, then lower id; id == sent
// marks "no candidate".
__device__ __forceinline__ void take_better(float &bv, int &be, float ov, int oe, int sent) {
  if (oe != sent && (be == sent || ov > bv || (ov == bv && oe < be))) {
    bv = ov;
    be = oe;
  }
}

template <int CTRL>
__device__ __forceinline__ void argmax_step(float &bv, int &be, int sent) {
  const float ov = __builtin_bit_cast(float, mov_dpp<CTRL>(__builtin_bit_cast(int, bv)));
  const int oe = mov_dpp<CTRL>(be);
  take_better(bv, be, ov, oe, sent);
}

// Best (value, id) over the wave, uniform in every lane: DPP within rows of 16
// lanes (xor 1, xor 2, half-row mirror, row mirror), then the four row results.
__device__ __forceinline__ void wave_argmax(float &bv, int &be, int sent) {
  argmax_step<0xB1>(bv, be, sent);   // quad_perm [1,0,3,2]
  argmax_step<0x4E>(bv, be, sent);   // quad_perm [2,3,0,1]
  argmax_step<0x141>(bv, be, sent);  // row_half_mirror
  argmax_step<0x140>(bv, be, sent);  // row_mirror
  float rv = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, bv), 0));
  int re = __builtin_amdgcn_readlane(be, 0);
#pragma unroll
  for (int r = 1; r < 4; ++r) {
    const float ov =
        __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, bv), 16 * r));
    const int oe = __builtin_amdgcn_readlane(be, 16 * r);
    take_better(rv, re, ov, oe, sent);
  }
  bv = rv;
  be = re;
}

// ============================================================== router logits
// One wave per (expert, tile of TT tokens).  Lane l accumulates i = l, l+64, ...
// with the product and the sum rounded separately (no contraction), then a
// halving tree off = 32..1, then the bias: the fixed order that makes every
// top-k decision reproducible bit for bit on the host.  Loads are issued CH at
// a time ahead of the ordered adds.  The waves also prepare the activations of
// the gate/up kernel (see kernels.hpp).
template <int TT, int CH>
__global__ __launch_bounds__(256) void router_kernel(const float *__restrict__ x, int T, int d,
                                                     const float *__restrict__ W,
                                                     const float *__restrict__ bias, int E,
                                                     float *__restrict__ z,
                                                     uint32_t *__restrict__ xp,
                                                     float *__restrict__ xsw,
                                                     float *__restrict__ xscale) {
#pragma clang fp contract(off)
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int t0 = blockIdx.y * TT;
  if (e >= E) return;
  const float *w = W + (long long)e * d + lane;
  const int nt = min(TT, T - t0);
  const float *xr[TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) xr[tt] = x + (long long)(t0 + min(tt, nt - 1)) * d + lane;
  float p[TT], mx[TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) {
    p[tt] = 0.0f;
    mx[tt] = 0.0f;
  }
  const int M = d / 64;
  for (int m0 = 0; m0 < M; m0 += CH) {
    float wv[CH], xv[TT][CH];
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int m = min(m0 + j, M - 1);
      wv[j] = w[64 * m];
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) xv[tt][j] = xr[tt][64 * m];
    }
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      if (m0 + j < M) {
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
          const float prod = xv[tt][j] * wv[j];
          p[tt] = p[tt] + prod;
          mx[tt] = fmaxf(mx[tt], fabsf(xv[tt][j]));
        }
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
  if (xp == nullptr) return;
  const int words = d / 8;
  const int gid = e * 64 + lane, stride = E * 64;
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) {
    if (tt >= nt) break;
    float m = mx[tt];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    int ex2 = 0;
    if (m > 0.0f && m <= 3.0e38f) {
      int fe;
      (void)frexpf(m, &fe);  // m = f * 2^fe, f in [0.5, 1)
      ex2 = max(0, fe - 14);
    }
    const float sc = ldexpf(1.0f, -ex2);
    const int t = t0 + tt;
    if (gid == 0) xscale[t] = ldexpf(1.0f, ex2);
    const float *xt = x + (long long)t * d;
    for (int j = gid; j < words; j += stride) {
      const int b = j >> 2, wq = j & 3;
      const float4 a = *reinterpret_cast<const float4 *>(xt + b * 32 + 4 * wq);
      const float4 c = *reinterpret_cast<const float4 *>(xt + b * 32 + 16 + 4 * wq);
      const float e0 = a.x * sc, e1 = a.y * sc, e2 = a.z * sc, e3 = a.w * sc;
      const float f0 = c.x * sc, f1 = c.y * sc, f2 = c.z * sc, f3 = c.w * sc;
      const float he0 = (float)(_Float16)e0, he1 = (float)(_Float16)e1;
      const float he2 = (float)(_Float16)e2, he3 = (float)(_Float16)e3;
      const float hf0 = (float)(_Float16)f0, hf1 = (float)(_Float16)f1;
      const float hf2 = (float)(_Float16)f2, hf3 = (float)(_Float16)f3;
      uint4 hi, lo;
      hi.x = pack_h2(he0, he2);
      hi.y = pack_h2(hf0, hf2);
      hi.z = pack_h2(he1, he3);
      hi.w = pack_h2(hf1, hf3);
      lo.x = pack_h2(e0 - he0, e2 - he2);
      lo.y = pack_h2(f0 - hf0, f2 - hf2);
      lo.z = pack_h2(e1 - he1, e3 - he3);
      lo.w = pack_h2(f1 - hf1, f3 - hf3);
      uint4 *dst = reinterpret_cast<uint4 *>(xp + ((long long)t * words + j) * 8);
      dst[0] = hi;
      dst[1] = lo;
      xsw[(long long)t * words + j] = ((e0 + e1) + (e2 + e3)) + ((f0 + f1) + (f2 + f3));
    }
  }
}

hipError_t launch_router(const float *x, int T, int d, const float *W, const float *bias, int E,
                         float *z, uint32_t *xp, float *xsw, float *xscale, hipStream_t s) {
  const int gx = (E + 3) / 4;
  if (T <= 1) {
    hipLaunchKernelGGL((router_kernel<1, 32>), dim3(gx, T), dim3(256), 0, s, x, T, d, W, bias, E,
                       z, xp, xsw, xscale);
  } else if (T <= 4) {
    hipLaunchKernelGGL((router_kernel<4, 16>), dim3(gx, 1), dim3(256), 0, s, x, T, d, W, bias, E,
                       z, xp, xsw, xscale);
  } else {
    hipLaunchKernelGGL((router_kernel<8, 8>), dim3(gx, (T + 7) / 8), dim3(256), 0, s, x, T, d, W,
                       bias, E, z, xp, xsw, xscale);
  }
  return hipGetLastError();
}

// ============================================================== top-k + softmax
// One wave per token; E <= 512, so each lane owns up to 8 logits.
__global__ __launch_bounds__(64) void topk_kernel(const float *__restrict__ z, int T, int E, int k,
                                                  int norm_topk, int32_t *__restrict__ idx,
                                                  float *__restrict__ w, int32_t *h_idx,
                                                  float *h_w) {
  const int t = blockIdx.x;
  const int lane = threadIdx.x;
  float v[8];
  bool ok[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int e = lane + 64 * c;
    ok[c] = e < E;
    v[c] = ok[c] ? z[(long long)t * E + e] : 0.0f;
  }
  int my_e = 0;
  float my_v = 0.0f;
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
    wave_argmax(bv, be, E);
#pragma unroll
    for (int c = 0; c < 8; ++c)
      if (lane + 64 * c == be) ok[c] = false;
    if (lane == j) {
      my_e = be;
      my_v = bv;
    }
  }
  const float zmax =
      __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_v), 0));
  float ex = 0.0f;
  if (lane < k) ex = expf(my_v - zmax);
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
    const long long o = (long long)t * k + lane;
    const float wv = ex / denom;
    idx[o] = my_e;
    w[o] = wv;
    h_idx[o] = my_e;
    h_w[o] = wv;
  }
}

hipError_t launch_topk(const float *z, int T, int E, int k, int norm_topk, int32_t *idx, float *w,
                       int32_t *h_idx, float *h_w, hipStream_t s) {
  hipLaunchKernelGGL(topk_kernel, dim3(T), dim3(64), 0, s, z, T, E, k, norm_topk, idx, w, h_idx,
                     h_w);
  return hipGetLastError();
}

// ============================================================== remap + bucket
// One workgroup.  Counts pairs per slot, lays buckets out in slot order, then
// places pairs stably (ascending pair id inside a bucket), 256 pairs at a time.
__global__ __launch_bounds__(256) void remap_kernel(const int32_t *__restrict__ idx, int T, int k,
                                                    SlotView view, int shared_slot, int n_ids,
                                                    int32_t *__restrict__ meta,
                                                    int32_t *__restrict__ bucket_pair) {
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
    }
    __syncthreads();
    if (s >= 0) atomicAdd(&run[s], 1);
    __syncthreads();
  }
}

hipError_t launch_remap(const int32_t *idx, int T, int k, const SlotView &view, int shared_slot,
                        int n_slot_ids, int32_t *meta, int32_t *bucket_pair, hipStream_t s) {
  hipLaunchKernelGGL(remap_kernel, dim3(1), dim3(256), 0, s, idx, T, k, view, shared_slot,
                     n_slot_ids, meta, bucket_pair);
  return hipGetLastError();
}

// ============================================================== bucket lookup
// The (slot, pairs) of bucket b.  With remap metadata it is a table read; on the
// decode path each wave derives it from the router ids: lane p takes pair p's
// slot, a pair opens a bucket when no lower pair has its slot, bucket b is the
// b-th opener, and its pairs are the lanes with the same slot, ascending.
template <int TT>
struct Bucket {
  int slot, off, cnt;
  int pairs[TT];  // decode path: the bucket's pairs (cnt <= TT)
  const uint8_t *src;
};

// Modes of a launch: buckets from remap metadata, derived on the device
// (decode), or given by the host in a BucketTable.
enum { BK_META = 0, BK_DEVICE = 1, BK_TABLE = 2 };

template <int TT, int MODE>
__device__ __forceinline__ bool find_bucket(const GemvArgs &a, const SlotView &view,
                                            const BucketTable &tab, int b, int *sl,
                                            Bucket<TT> &bk) {
  if constexpr (MODE == BK_TABLE) {
    if (b >= tab.n) return false;
    bk.src = tab.src[b];
    bk.cnt = tab.cnt[b];
    bk.off = 0;
    bk.slot = 0;
#pragma unroll
    for (int i = 0; i < TT; ++i) bk.pairs[i] = tab.pairs[b][i < kDecodeMaxTokens ? i : 0];
    return true;
  }
  if constexpr (MODE == BK_META) {
    if (b >= a.meta[0]) return false;
    bk.slot = a.meta[2 + b];
    bk.off = a.meta[2 + kMetaB + b];
    bk.cnt = a.meta[2 + 2 * kMetaB + b];
    bk.src = a.slots + (long long)bk.slot * a.rec_bytes;
    return true;
  }
  const int lane = threadIdx.x & 63;
  const int Pr = a.T * a.k;
  const int P = Pr + (a.shared_slot >= 0 ? a.T : 0);
  int s = -1;
  if (lane < P) s = lane < Pr ? (int)view.slot[a.idx[lane]] : a.shared_slot;
  sl[lane] = s;
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_s_waitcnt(0);
  bool first = s >= 0;
  for (int q = 0; q < lane; ++q)
    if (sl[q] == s) first = false;
  uint64_t openers = __ballot(first);
  if (__popcll(openers) <= b) return false;
  for (int i = 0; i < b; ++i) openers &= openers - 1;
  const int L = __ffsll((unsigned long long)openers) - 1;
  bk.slot = __builtin_amdgcn_readlane(s, L);
  bk.src = a.slots + (long long)bk.slot * a.rec_bytes;
  uint64_t same = __ballot(s == bk.slot);
  bk.cnt = __popcll(same);
  bk.off = 0;
  int last = 0;
#pragma unroll
  for (int i = 0; i < TT; ++i) {
    if (same) {
      last = __ffsll((unsigned long long)same) - 1;
      same &= same - 1;
    }
    bk.pairs[i] = last;
  }
  return true;
}

template <int TT, int MODE>
__device__ __forceinline__ int bucket_pair_at(const GemvArgs &a, const Bucket<TT> &bk, int i) {
  if constexpr (MODE == BK_META) return a.bucket_pair[bk.off + i];
  return bk.pairs[i < TT ? i : TT - 1];
}



// ============================================================== Q4 grouped GEMV
// Workgroup = 4 waves, one slot bucket (blockIdx.y) and a tile of rows
// (blockIdx.x).  In a wave, G lanes share a row and RG = 64/G rows run side by
// side; a lane walks its row's units (V consecutive 32-bit nibble words: V = 4 a
// whole block, V = 2 half a block) and R rows per lane reuse the unit's
// activations from registers.  The -8 offset of the weights is folded in per
// unit; partial sums meet across the G lanes with xor shuffles.
//
// gate/up (GLU): the K dimension is split over the 4 waves of the workgroup,
// whose partials meet in LDS in a fixed order.  A nibble word q holds the
// elements (0,2),(16,18),(1,3),(17,19) of its 4-element group as the low/high
// nibbles of bytes (0,2) and (1,3); OR-ing each nibble pair into 0x6400 gives two
// binary16 values 1024 + q, so one v_dot2 against the prepared hi and lo
// activation pairs accumulates (1024 + q) x in fp32, and 1032 * sum(x) per unit
// brings it back to (q - 8) x.
//
// down: whole K per wave; nibbles become floats with v_cvt_f32_ubyte0..3.

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ half2_t as_h2(uint32_t v) { return __builtin_bit_cast(half2_t, v); }

__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t o) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(m), "v"(o));
  return r;
}

// sum over one word of (1024 + q) * x, x given as hi and lo binary16 pairs
__device__ __forceinline__ float word_dot_h(uint32_t q, const uint4 &xh, const uint4 &xl,
                                            float acc) {
  const uint32_t m = 0x000F000Fu, mag = 0x64006400u;
  const uint32_t a = and_or(q, m, mag);
  const uint32_t b = and_or(q >> 4, m, mag);
  const uint32_t c = and_or(q >> 8, m, mag);
  const uint32_t d = and_or(q >> 12, m, mag);
  acc = __builtin_amdgcn_fdot2(as_h2(a), as_h2(xh.x), acc, false);
  acc = __builtin_amdgcn_fdot2(as_h2(b), as_h2(xh.y), acc, false);
  acc = __builtin_amdgcn_fdot2(as_h2(c), as_h2(xh.z), acc, false);
  acc = __builtin_amdgcn_fdot2(as_h2(d), as_h2(xh.w), acc, false);
  acc = __builtin_amdgcn_fdot2(as_h2(a), as_h2(xl.x), acc, false);
  acc = __builtin_amdgcn_fdot2(as_h2(b), as_h2(xl.y), acc, false);
  acc = __builtin_amdgcn_fdot2(as_h2(c), as_h2(xl.z), acc, false);
  acc = __builtin_amdgcn_fdot2(as_h2(d), as_h2(xl.w), acc, false);
  return acc;
}

// sum over one word of q * x in fp32 (x: elements 0..3 and 16..19 of the group)
__device__ __forceinline__ float word_dot_f(uint32_t q, const float4 &xl, const float4 &xh,
                                            float acc) {
  uint32_t lo = q & 0x0F0F0F0Fu;
  uint32_t hi = (q >> 4) & 0x0F0F0F0Fu;
  // hide the known-zero high nibbles so each byte converts with one v_cvt_f32_ubyteN
  asm volatile("" : "+v"(lo), "+v"(hi));
  acc += (float)(lo & 0xFFu) * xl.x;
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

__device__ __forceinline__ int pair_row(const GemvArgs &a, int p) {
  return p < a.T * a.k ? p / a.k : p - a.T * a.k;
}

template <int G, int V, int TT, int R, int MODE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4, 8)))
void q4_gateup_kernel(GemvArgs a, SlotView view, BucketTable tab) {
  constexpr int RG = 64 / G;
  constexpr int KS = 4;
  __shared__ float red[KS][R * RG][TT][2];
  __shared__ int sl[4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  Bucket<TT> bk;
  if (!find_bucket<TT, MODE>(a, view, tab, blockIdx.y, sl[wave], bk)) return;
  const uint8_t *rec = bk.src;
  const int grp = lane / G, gl = lane % G;
  const int row0 = blockIdx.x * (R * RG) + grp;
  const int row_words = a.nb * 4;
  const int units = row_words / V;
  const int words_x = a.nb * 4;  // words per activation row
  // rows past the end read the last row and are never written
  const uint32_t *qg[R];
  const uint32_t *qu[R];
  const __half *sg[R];
  const __half *su[R];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const long long r = min(row0 + i * RG, a.rows - 1);
    qg[i] = reinterpret_cast<const uint32_t *>(rec + a.off_q0) + r * row_words;
    qu[i] = reinterpret_cast<const uint32_t *>(rec + a.off_q1) + r * row_words;
    sg[i] = reinterpret_cast<const __half *>(rec + a.off_s0) + r * a.nb;
    su[i] = reinterpret_cast<const __half *>(rec + a.off_s1) + r * a.nb;
  }

  for (int tg = 0; tg < bk.cnt; tg += TT) {
    const int nt = min(TT, bk.cnt - tg);
    int prs[TT], tok[TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      prs[tt] = bucket_pair_at<TT, MODE>(a, bk, tg + min(tt, nt - 1));
      tok[tt] = pair_row(a, prs[tt]);
    }
    float ag[R][TT], au[R][TT];
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        ag[i][tt] = 0.0f;
        au[i][tt] = 0.0f;
      }
    for (int u = gl + G * wave; u < units; u += G * KS) {
      const int w0 = u * V;
      const int blk = w0 >> 2;
      uint4 xh[TT][V], xl[TT][V];
      float xs[TT];
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        const uint4 *xq =
            reinterpret_cast<const uint4 *>(a.xp + ((long long)tok[tt] * words_x + w0) * 8);
        const float *xw = a.xsw + (long long)tok[tt] * words_x + w0;
        xs[tt] = 0.0f;
#pragma unroll
        for (int v = 0; v < V; ++v) {
          xh[tt][v] = xq[2 * v];
          xl[tt][v] = xq[2 * v + 1];
          xs[tt] += xw[v];
        }
      }
      uint32_t q0[R][V], q1[R][V];
      float s0[R], s1[R];
#pragma unroll
      for (int i = 0; i < R; ++i) {
        load_words<V>(qg[i] + w0, q0[i]);
        load_words<V>(qu[i] + w0, q1[i]);
        s0[i] = __half2float(sg[i][blk]);
        s1[i] = __half2float(su[i][blk]);
      }
#pragma unroll
      for (int i = 0; i < R; ++i) {
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
          float d0 = -1032.0f * xs[tt], d1 = -1032.0f * xs[tt];
#pragma unroll
          for (int v = 0; v < V; ++v) {
            d0 = word_dot_h(q0[i][v], xh[tt][v], xl[tt][v], d0);
            d1 = word_dot_h(q1[i][v], xh[tt][v], xl[tt][v], d1);
          }
          ag[i][tt] += s0[i] * d0;
          au[i][tt] += s1[i] * d1;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
#pragma unroll
        for (int o = G / 2; o >= 1; o >>= 1) {
          ag[i][tt] += __shfl_xor(ag[i][tt], o, 64);
          au[i][tt] += __shfl_xor(au[i][tt], o, 64);
        }
      }
    if (gl == 0) {
#pragma unroll
      for (int i = 0; i < R; ++i)
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
          red[wave][i * RG + grp][tt][0] = ag[i][tt];
          red[wave][i * RG + grp][tt][1] = au[i][tt];
        }
    }
    __syncthreads();
    for (int o = threadIdx.x; o < R * RG * TT; o += 256) {
      const int rr = o / TT, tt = o % TT;
      const int r = blockIdx.x * (R * RG) + rr;
      if (r < a.rows && tt < nt) {
        const float sc = a.xscale[tok[tt]];
        const float g = (((red[0][rr][tt][0] + red[1][rr][tt][0]) + red[2][rr][tt][0]) +
                         red[3][rr][tt][0]) * sc;
        const float uu = (((red[0][rr][tt][1] + red[1][rr][tt][1]) + red[2][rr][tt][1]) +
                          red[3][rr][tt][1]) * sc;
        a.out[(long long)prs[tt] * a.rows + r] = silu_f(g) * uu;
      }
    }
    __syncthreads();
  }
}

template <int G, int V, int TT, int R, int MODE, int KS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4, 8)))
void q4_down_kernel(GemvArgs a, SlotView view, BucketTable tab) {
  constexpr int RG = 64 / G;
  constexpr int ROWS_WAVE = R * RG;
  constexpr int NRG = 4 / KS;  // row groups per workgroup; KS waves share a row group's K
  __shared__ int sl[4][64];
  __shared__ float red[KS > 1 ? 4 : 1][ROWS_WAVE][TT];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int kslice = wave % KS, rgrp = wave / KS;
  Bucket<TT> bk;
  if (!find_bucket<TT, MODE>(a, view, tab, blockIdx.y, sl[wave], bk)) return;
  const uint8_t *rec = bk.src;
  const int grp = lane / G, gl = lane % G;
  const int row0 = (blockIdx.x * NRG + rgrp) * ROWS_WAVE + grp;
  const int row_words = a.nb * 4;
  const int units = row_words / V;
  const int K = a.nb * 32;
  const uint32_t *qr[R];
  const __half *sr[R];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const long long r = min(row0 + i * RG, a.rows - 1);
    qr[i] = reinterpret_cast<const uint32_t *>(rec + a.off_q0) + r * row_words;
    sr[i] = reinterpret_cast<const __half *>(rec + a.off_s0) + r * a.nb;
  }

  for (int tg = 0; tg < bk.cnt; tg += TT) {
    const int nt = min(TT, bk.cnt - tg);
    const float *xin[TT];
    int prs[TT];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      const int p = bucket_pair_at<TT, MODE>(a, bk, tg + min(tt, nt - 1));
      prs[tt] = p;
      xin[tt] = a.in + (long long)(a.in_by_pair ? p : pair_row(a, p)) * K;
    }
    float acc[R][TT];
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) acc[i][tt] = 0.0f;
    for (int u = gl + G * kslice; u < units; u += G * KS) {
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
          const float *xq = xin[tt] + blk * 32 + 4 * wb;
          xl[tt][v] = *reinterpret_cast<const float4 *>(xq);
          xh[tt][v] = *reinterpret_cast<const float4 *>(xq + 16);
          xs[tt] += ((xl[tt][v].x + xl[tt][v].y) + (xl[tt][v].z + xl[tt][v].w)) +
                    ((xh[tt][v].x + xh[tt][v].y) + (xh[tt][v].z + xh[tt][v].w));
        }
      }
      uint32_t q0[R][V];
      float sc0[R];
#pragma unroll
      for (int i = 0; i < R; ++i) {
        load_words<V>(qr[i] + w0, q0[i]);
        sc0[i] = __half2float(sr[i][blk]);
      }
#pragma unroll
      for (int i = 0; i < R; ++i) {
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
          float d0 = -8.0f * xs[tt];
#pragma unroll
          for (int v = 0; v < V; ++v) d0 = word_dot_f(q0[i][v], xl[tt][v], xh[tt][v], d0);
          acc[i][tt] += sc0[i] * d0;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
#pragma unroll
        for (int o = G / 2; o >= 1; o >>= 1) acc[i][tt] += __shfl_xor(acc[i][tt], o, 64);
      }
    if constexpr (KS == 1) {
      if (gl == 0) {
#pragma unroll
        for (int i = 0; i < R; ++i) {
          const int r = row0 + i * RG;
          if (r < a.rows) {
#pragma unroll
            for (int tt = 0; tt < TT; ++tt)
              if (tt < nt) a.out[(long long)prs[tt] * a.rows + r] = acc[i][tt];
          }
        }
      }
    } else {
      // the KS waves of a row group meet in LDS, summed in wave order
      if (gl == 0) {
#pragma unroll
        for (int i = 0; i < R; ++i)
#pragma unroll
          for (int tt = 0; tt < TT; ++tt) red[wave][i * RG + grp][tt] = acc[i][tt];
      }
      __syncthreads();
      for (int o = threadIdx.x; o < NRG * ROWS_WAVE * TT; o += 256) {
        const int g = o / (ROWS_WAVE * TT), rr = (o / TT) % ROWS_WAVE, tt = o % TT;
        const int r = (blockIdx.x * NRG + g) * ROWS_WAVE + rr;
        if (r < a.rows && tt < nt) {
          float v = 0.0f;
#pragma unroll
          for (int q = 0; q < KS; ++q) v += red[g * KS + q][rr][tt];
          a.out[(long long)prs[tt] * a.rows + r] = v;
        }
      }
      __syncthreads();
    }
  }
}

// Shapes measured on MI355X (cold Infinity Cache) over the decode shapes
// d x f = 6144 x 2048, 2816 x 704, 2048 x 768 with 8 experts: half-block units
// (V = 2) always beat whole blocks; gate/up runs best with 32 lanes per row and
// 4 rows per lane; down with 16 lanes per row and 4 rows per lane, its K split
// over the workgroup's waves only when the grid is small.  Fewer rows per lane
// when the grid would otherwise leave the chip idle.
GemvShape choose_gemv(bool glu, int rows, int nb, int n_buckets, int max_tokens) {
  GemvShape sh{16, 2, 1, 1, 1};
  const int units = nb * 2;  // half-block units per row
  if (glu) {
    sh.KS = 4;
    sh.G = units >= 128 ? 32 : 16;
  } else {
    sh.KS = (long long)rows * n_buckets <= 16384 ? 4 : 1;
    sh.G = 16;
  }
  sh.TT = max_tokens <= 1 ? 1 : (max_tokens <= 2 ? 2 : 4);
  const int RG = 64 / sh.G;
  const int rows_wg_per_r = (4 / sh.KS) * RG;
  sh.R = 1;
  const int rs[2] = {4, 2};
  for (int ri = 0; ri < 2; ++ri) {
    const int R = rs[ri];
    const long long waves =
        4LL * n_buckets * ((rows + R * rows_wg_per_r - 1) / (R * rows_wg_per_r));
    if (waves >= 512) {
      sh.R = R;
      break;
    }
  }
  return sh;
}

struct LaunchCtx {
  const GemvArgs *a;
  const SlotView *view;
  const BucketTable *tab;
  bool glu;
  int nbk;
  hipStream_t s;
  int ks;
};

template <int G, int V, int TT, int R, int MODE>
static hipError_t launch_one(const LaunchCtx &c) {
  constexpr int RG = 64 / G;
  const GemvArgs &a = *c.a;
  if (c.glu) {
    const dim3 grid((a.rows + R * RG - 1) / (R * RG), c.nbk);
    hipLaunchKernelGGL((q4_gateup_kernel<G, V, TT, R, MODE>), grid, dim3(256), 0, c.s, a, *c.view,
                       *c.tab);
  } else if (c.ks == 4) {
    constexpr int rows_blk = R * RG;
    const dim3 grid((a.rows + rows_blk - 1) / rows_blk, c.nbk);
    hipLaunchKernelGGL((q4_down_kernel<G, V, TT, R, MODE, 4>), grid, dim3(256), 0, c.s, a,
                       *c.view, *c.tab);
  } else {
    constexpr int rows_blk = 4 * R * RG;
    const dim3 grid((a.rows + rows_blk - 1) / rows_blk, c.nbk);
    hipLaunchKernelGGL((q4_down_kernel<G, V, TT, R, MODE, 1>), grid, dim3(256), 0, c.s, a,
                       *c.view, *c.tab);
  }
  return hipGetLastError();
}

template <int G, int V, int TT, int R>
static hipError_t launch_m(const LaunchCtx &c) {
  if (c.tab->n >= 0) return launch_one<G, V, TT, R, BK_TABLE>(c);
  if (c.a->meta != nullptr) return launch_one<G, V, TT, R, BK_META>(c);
  return launch_one<G, V, TT, R, BK_DEVICE>(c);
}

template <int G, int V, int TT>
static hipError_t launch_r(const LaunchCtx &c, int R) {
  switch (R) {
    case 4: return launch_m<G, V, TT, 4>(c);
    case 2: return launch_m<G, V, TT, 2>(c);
    default: return launch_m<G, V, TT, 1>(c);
  }
}

template <int G, int V>
static hipError_t launch_t(const LaunchCtx &c, const GemvShape &sh) {
  switch (sh.TT) {
    case 1: return launch_r<G, V, 1>(c, sh.R);
    case 2: return launch_r<G, V, 2>(c, sh.R);
    default: return launch_r<G, V, 4>(c, sh.R);
  }
}

template <int G>
static hipError_t launch_v(const LaunchCtx &c, const GemvShape &sh) {
  return sh.V == 4 ? launch_t<G, 4>(c, sh) : launch_t<G, 2>(c, sh);
}

hipError_t launch_gemv(const GemvArgs &a, const SlotView &view, const BucketTable *tab,
                       const GemvShape &sh, bool glu, int n_buckets, hipStream_t s) {
  if (n_buckets <= 0) return hipSuccess;
  BucketTable none;
  none.n = -1;
  const LaunchCtx c{&a, &view, tab ? tab : &none, glu, n_buckets, s, sh.KS};
  switch (sh.G) {
    case 64: return launch_v<64>(c, sh);
    case 32: return launch_v<32>(c, sh);
    default: return launch_v<16>(c, sh);
  }
}

// ============================================================== prefill MFMA GEMM
// Per workgroup: 4 waves x 2 row blocks of 16 = 128 weight rows of one bucket's
// expert, and its tokens in passes of up to NT x 16.  The K dimension runs in
// chunks of KC blocks through two LDS buffers: while the waves multiply chunk c,
// the chunk c+1 loads (raw nibble words, block scales, the tokens' hi/lo
// activation pairs and block sums) are in flight and land in the other buffer.
// A lane turns its nibble word into binary16 (1024 + q) as it builds the MFMA A
// operand; each 32-weight block is one pair of v_mfma_f32_16x16x32_f16 (x hi,
// x lo), and d * (C - 1032 * sum x) is folded into the accumulators in fp32.
// Operand lanes: A lane l = row l%16 and the 8 K values of word l/16 of the
// block (elements g, g+2, g+16, g+18, g+1, g+3, g+17, g+19 with g = 4*(l/16));
// B lane l = token l%16 and the same 8 K values; C lane l = rows 4*(l/16)+i,
// token l%16.
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int K6_RB = 2;                  // 16-row blocks per wave
constexpr int K6_ROWS = 4 * 16 * K6_RB;   // rows per workgroup
constexpr int K6_KC = 4;                  // blocks per K chunk
constexpr int K6_NT = 2;                  // 16-token tiles per pass
constexpr int K6_AW = K6_KC * 4 + 1;      // words per LDS row (one pad against bank conflicts)

__device__ __forceinline__ uint4 decode_word_h(uint32_t q) {
  const uint32_t m = 0x000F000Fu, mag = 0x64006400u;
  uint4 r;
  r.x = and_or(q, m, mag);
  r.y = and_or(q >> 4, m, mag);
  r.z = and_or(q >> 8, m, mag);
  r.w = and_or(q >> 12, m, mag);
  return r;
}

template <int NM>
struct K6Buf {
  uint32_t A[NM][K6_ROWS][K6_AW];
  float S[NM][K6_ROWS][K6_KC];
  uint4 B[K6_NT * 16][K6_KC * 4][2];
  float X[K6_NT * 16][K6_KC];
};

template <int NM>
struct K6Regs {
  uint4 w[NM][2];
  float sc[NM][2];
  uint4 b[2][2];
  float4 xs;
};

template <bool GLU>
__global__ __launch_bounds__(256) void q4_mfma_kernel(GemvArgs a) {
  constexpr int NM = GLU ? 2 : 1;
  __shared__ K6Buf<NM> buf[2];
  __shared__ int lTok[K6_NT * 16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bucket = blockIdx.y;
  if (bucket >= a.meta[0]) return;
  const int slot = a.meta[2 + bucket];
  const int off = a.meta[2 + kMetaB + bucket];
  const int cnt = a.meta[2 + 2 * kMetaB + bucket];
  const uint8_t *rec = a.slots + (long long)slot * a.rec_bytes;
  const int row_base = blockIdx.x * K6_ROWS;
  const int words = a.nb * 4;
  const uint32_t *qb[NM];
  const __half *sb[NM];
  qb[0] = reinterpret_cast<const uint32_t *>(rec + a.off_q0);
  sb[0] = reinterpret_cast<const __half *>(rec + a.off_s0);
  if constexpr (GLU) {
    qb[NM - 1] = reinterpret_cast<const uint32_t *>(rec + a.off_q1);
    sb[NM - 1] = reinterpret_cast<const __half *>(rec + a.off_s1);
  }
  const int m = lane & 15, kg = lane >> 4;
  const int n_chunks = (a.nb + K6_KC - 1) / K6_KC;

  for (int g0 = 0; g0 < cnt; g0 += K6_NT * 16) {
    const int ntok = min(K6_NT * 16, cnt - g0);
    const int n_tiles = (ntok + 15) >> 4;
    if (tid < K6_NT * 16) {
      const int p = a.bucket_pair[off + g0 + min(tid, ntok - 1)];
      lTok[tid] = a.in_by_pair ? p : pair_row(a, p);
    }
    __syncthreads();
    // staging roles: items (row, block) = 128 x KC per matrix, 2 per thread;
    // (token, word) = 32 x 4*KC, 2 per thread; (token, block) = 32 x KC, 1 per thread
    auto load_chunk = [&](int c, K6Regs<NM> &r) {
      const int kc = c * K6_KC;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int it = tid + 256 * j;
        const int row = it >> 2, blk = min(kc + (it & 3), a.nb - 1);
        const long long gr = min(row_base + row, a.rows - 1);
#pragma unroll
        for (int q = 0; q < NM; ++q) {
          r.w[q][j] = *reinterpret_cast<const uint4 *>(qb[q] + gr * words + blk * 4);
          r.sc[q][j] = __half2float(sb[q][gr * a.nb + blk]);
        }
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int it = tid + 256 * j;
        const int t = it >> 4, w = it & 15;
        const int wq = min(kc * 4 + w, words - 1);
        const uint4 *src =
            reinterpret_cast<const uint4 *>(a.xp + ((long long)lTok[t] * words + wq) * 8);
        r.b[j][0] = src[0];
        r.b[j][1] = src[1];
      }
      {
        const int t = (tid >> 2) & 31, b = tid & 3;
        const int blk = min(kc + b, a.nb - 1);
        r.xs = *reinterpret_cast<const float4 *>(a.xsw + (long long)lTok[t] * words + blk * 4);
      }
    };
    auto store_chunk = [&](K6Buf<NM> &B, const K6Regs<NM> &r) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int it = tid + 256 * j;
        const int row = it >> 2, b = it & 3;
#pragma unroll
        for (int q = 0; q < NM; ++q) {
          B.A[q][row][b * 4 + 0] = r.w[q][j].x;
          B.A[q][row][b * 4 + 1] = r.w[q][j].y;
          B.A[q][row][b * 4 + 2] = r.w[q][j].z;
          B.A[q][row][b * 4 + 3] = r.w[q][j].w;
          B.S[q][row][b] = r.sc[q][j];
        }
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int it = tid + 256 * j;
        B.B[it >> 4][it & 15][0] = r.b[j][0];
        B.B[it >> 4][it & 15][1] = r.b[j][1];
      }
      if (tid < 128) B.X[tid >> 2][tid & 3] = (r.xs.x + r.xs.y) + (r.xs.z + r.xs.w);
    };

    floatx4 acc[NM][K6_RB][K6_NT];
#pragma unroll
    for (int q = 0; q < NM; ++q)
#pragma unroll
      for (int rb = 0; rb < K6_RB; ++rb)
#pragma unroll
        for (int t = 0; t < K6_NT; ++t) acc[q][rb][t] = floatx4{0.f, 0.f, 0.f, 0.f};

    K6Regs<NM> regs;
    load_chunk(0, regs);
    store_chunk(buf[0], regs);
    __syncthreads();
    for (int c = 0; c < n_chunks; ++c) {
      if (c + 1 < n_chunks) load_chunk(c + 1, regs);
      const K6Buf<NM> &B = buf[c & 1];
      const int kb_n = min(K6_KC, a.nb - c * K6_KC);
      for (int kb = 0; kb < kb_n; ++kb) {
        half8_t Bh[K6_NT], Bl[K6_NT];
        float o1032[K6_NT];
#pragma unroll
        for (int t = 0; t < K6_NT; ++t) {
          Bh[t] = __builtin_bit_cast(half8_t, B.B[t * 16 + m][kb * 4 + kg][0]);
          Bl[t] = __builtin_bit_cast(half8_t, B.B[t * 16 + m][kb * 4 + kg][1]);
          o1032[t] = 1032.0f * B.X[t * 16 + m][kb];
        }
#pragma unroll
        for (int rb = 0; rb < K6_RB; ++rb) {
          const int rw = wave * (16 * K6_RB) + rb * 16;
#pragma unroll
          for (int q = 0; q < NM; ++q) {
            const half8_t A = __builtin_bit_cast(half8_t, decode_word_h(B.A[q][rw + m][kb * 4 + kg]));
            float sc[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) sc[i] = B.S[q][rw + kg * 4 + i][kb];
#pragma unroll
            for (int t = 0; t < K6_NT; ++t) {
              if (t < n_tiles) {
                floatx4 cc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, Bh[t], floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                cc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, Bl[t], cc, 0, 0, 0);
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[q][rb][t][i] += sc[i] * (cc[i] - o1032[t]);
              }
            }
          }
        }
      }
      if (c + 1 < n_chunks) store_chunk(buf[(c + 1) & 1], regs);
      __syncthreads();
    }
    // C lane layout: rows rw + kg*4 + i, token column m of each tile
#pragma unroll
    for (int t = 0; t < K6_NT; ++t) {
      const int col = t * 16 + m;
      if (t < n_tiles && col < ntok) {
        const int p = a.bucket_pair[off + g0 + col];
        const float sc = a.xscale[lTok[col]];
#pragma unroll
        for (int rb = 0; rb < K6_RB; ++rb) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = row_base + wave * (16 * K6_RB) + rb * 16 + kg * 4 + i;
            if (r < a.rows) {
              const float v = GLU ? silu_f(acc[0][rb][t][i] * sc) * (acc[NM - 1][rb][t][i] * sc)
                                  : acc[0][rb][t][i] * sc;
              a.out[(long long)p * a.rows + r] = v;
            }
          }
        }
      }
    }
    __syncthreads();
  }
}

hipError_t launch_mfma(const GemvArgs &a, bool glu, int n_buckets, hipStream_t s) {
  if (n_buckets <= 0) return hipSuccess;
  const dim3 grid((a.rows + K6_ROWS - 1) / K6_ROWS, n_buckets);
  if (glu)
    hipLaunchKernelGGL(q4_mfma_kernel<true>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(q4_mfma_kernel<false>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

// One wave per row: scale, binary16 hi/lo pairs in the decoder's order, word sums.
__global__ __launch_bounds__(64) void prep_pairs_kernel(const float *__restrict__ in, int rows, int K,
                                                        uint32_t *__restrict__ xp,
                                                        float *__restrict__ xsw,
                                                        float *__restrict__ xscale) {
  const int r = blockIdx.x, lane = threadIdx.x;
  if (r >= rows) return;
  const float *xt = in + (long long)r * K;
  float m = 0.0f;
  for (int i = lane; i < K; i += 64) m = fmaxf(m, fabsf(xt[i]));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  int ex2 = 0;
  if (m > 0.0f && m <= 3.0e38f) {
    int fe;
    (void)frexpf(m, &fe);
    ex2 = max(0, fe - 14);
  }
  const float sc = ldexpf(1.0f, -ex2);
  if (lane == 0) xscale[r] = ldexpf(1.0f, ex2);
  const int words = K / 8;
  for (int j = lane; j < words; j += 64) {
    const int b = j >> 2, wq = j & 3;
    const float4 av = *reinterpret_cast<const float4 *>(xt + b * 32 + 4 * wq);
    const float4 cv = *reinterpret_cast<const float4 *>(xt + b * 32 + 16 + 4 * wq);
    const float e0 = av.x * sc, e1 = av.y * sc, e2 = av.z * sc, e3 = av.w * sc;
    const float f0 = cv.x * sc, f1 = cv.y * sc, f2 = cv.z * sc, f3 = cv.w * sc;
    const float he0 = (float)(_Float16)e0, he1 = (float)(_Float16)e1;
    const float he2 = (float)(_Float16)e2, he3 = (float)(_Float16)e3;
    const float hf0 = (float)(_Float16)f0, hf1 = (float)(_Float16)f1;
    const float hf2 = (float)(_Float16)f2, hf3 = (float)(_Float16)f3;
    uint4 hi, lo;
    hi.x = pack_h2(he0, he2);
    hi.y = pack_h2(hf0, hf2);
    hi.z = pack_h2(he1, he3);
    hi.w = pack_h2(hf1, hf3);
    lo.x = pack_h2(e0 - he0, e2 - he2);
    lo.y = pack_h2(f0 - hf0, f2 - hf2);
    lo.z = pack_h2(e1 - he1, e3 - he3);
    lo.w = pack_h2(f1 - hf1, f3 - hf3);
    uint4 *dst = reinterpret_cast<uint4 *>(xp + ((long long)r * words + j) * 8);
    dst[0] = hi;
    dst[1] = lo;
    xsw[(long long)r * words + j] = ((e0 + e1) + (e2 + e3)) + ((f0 + f1) + (f2 + f3));
  }
}

hipError_t launch_prep_pairs(const float *in, int rows, int K, uint32_t *xp, float *xsw,
                             float *xscale, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(prep_pairs_kernel, dim3(rows), dim3(64), 0, s, in, rows, K, xp, xsw, xscale);
  return hipGetLastError();
}

// ============================================================== slot fills
__global__ __launch_bounds__(256) void pull_kernel(PullList l) {
  const int e = blockIdx.x / l.per_expert, part = blockIdx.x % l.per_expert;
  if (e >= l.n) return;
  const long long per = (l.bytes16 + l.per_expert - 1) / l.per_expert;
  const long long b = part * per, end = min(b + per, l.bytes16);
  const uint4 *__restrict__ src = reinterpret_cast<const uint4 *>(l.src[e]);
  uint4 *__restrict__ dst = reinterpret_cast<uint4 *>(l.dst[e]);
  constexpr int U = 8;
  for (long long i = b + threadIdx.x; i < end; i += 256 * U) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const long long j = i + (long long)u * 256;
      if (j < end) v[u] = src[j];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const long long j = i + (long long)u * 256;
      if (j < end) dst[j] = v[u];
    }
  }
}

hipError_t launch_pull(const PullList &l, hipStream_t s) {
  if (l.n <= 0) return hipSuccess;
  hipLaunchKernelGGL(pull_kernel, dim3(l.n * l.per_expert), dim3(256), 0, s, l);
  return hipGetLastError();
}

// ============================================================== combine
__global__ __launch_bounds__(256) void combine_kernel(const float *__restrict__ y,
                                                      const float *__restrict__ w,
                                                      const int32_t *__restrict__ idx,
                                                      SlotView view, int all_gpu, int T, int k,
                                                      int d, int n_shared,
                                                      const float *__restrict__ host_part,
                                                      float *__restrict__ out,
                                                      float *__restrict__ dbg_gpu) {
  const int t = blockIdx.y;
  const int i = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= d) return;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < k; ++j) {
    const long long p = (long long)t * k + j;
    if (all_gpu || view.slot[idx[p]] >= 0) {
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

hipError_t launch_combine(const float *y, const float *w, const int32_t *idx,
                          const SlotView &view, int all_gpu, int T, int k, int d, int n_shared,
                          const float *host_part, float *out, float *dbg_gpu, hipStream_t s) {
  const dim3 grid((d / 4 + 255) / 256, T);
  hipLaunchKernelGGL(combine_kernel, grid, dim3(256), 0, s, y, w, idx, view, all_gpu, T, k, d,
                     n_shared, host_part, out, dbg_gpu);
  return hipGetLastError();
}

}  // namespace moe
