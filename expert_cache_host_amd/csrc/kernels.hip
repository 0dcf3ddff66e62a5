// gfx950 kernels of the routed-MoE layer served from per-layer expert slots.
//
// Wave64 throughout.  Q4 weights are read from the slot layout (layout.hpp):
// per matrix, row-major 16-byte nibble blocks and a separate binary16 scale
// array.  Element j of a block is the low nibble of byte j, element j+16 the
// high nibble; w = d * (q - 8).
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <algorithm>
#include <mutex>
#include <type_traits>

#include "kernels.hpp"
#include "workspace.hpp"

namespace moe {

// ============================================================== launches
// Every kernel goes out through launch_k.  A start / stop event pair set by
// set_launch_events is handed to the next launch of the same host thread,
// which records them at that kernel's own dispatch start and end
// (hipExtLaunchKernel): the pair then times the kernel alone, without the
// host's launch latency that events recorded around the call would include
// whenever the stream is idle.
static thread_local hipEvent_t t_ev_start = nullptr, t_ev_stop = nullptr;

void set_launch_events(hipEvent_t start, hipEvent_t stop) {
  t_ev_start = start;
  t_ev_stop = stop;
}

bool launch_events_pending() {
  const bool p = t_ev_start != nullptr;
  t_ev_start = t_ev_stop = nullptr;
  return p;
}

template <typename... KArgs, typename... Args>
static void launch_k(void (*kernel)(KArgs...), dim3 grid, dim3 blk, size_t lds, hipStream_t s,
                     Args... args) {
  hipEvent_t a = t_ev_start, b = t_ev_stop;
  t_ev_start = t_ev_stop = nullptr;
  hipExtLaunchKernelGGL(kernel, grid, blk, (uint32_t)lds, s, a, b, 0u, static_cast<KArgs>(args)...);
}


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

// Top-k order as one unsigned 64-bit comparison: the logit's bits mapped to an
// order-preserving integer (-0 taken as +0) above the complemented expert id,
// so that a larger value wins and, at equal values, the lower id.  0 is "no
// candidate": no logit maps to it.
__device__ __forceinline__ uint64_t topk_key(float v, int e) {
  uint32_t b = __builtin_bit_cast(uint32_t, v + 0.0f);
  b = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((uint64_t)b << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)e);
}

__device__ __forceinline__ float key_value(uint64_t k) {
  const uint32_t b = (uint32_t)(k >> 32);
  return __builtin_bit_cast(float, (b & 0x80000000u) ? (b & 0x7FFFFFFFu) : ~b);
}

__device__ __forceinline__ int key_id(uint64_t k) { return (int)(0xFFFFFFFFu - (uint32_t)k); }

__device__ __forceinline__ uint64_t kmax(uint64_t a, uint64_t b) { return a > b ? a : b; }

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_key(uint64_t k) {
  const uint32_t lo = (uint32_t)mov_dpp<CTRL>((int)(uint32_t)k);
  const uint32_t hi = (uint32_t)mov_dpp<CTRL>((int)(uint32_t)(k >> 32));
  return ((uint64_t)hi << 32) | lo;
}

// max(k, k of the partner lane) across 16-lane rows (ROWS = 16: rows 2j and
// 2j+1) or wave halves (ROWS = 32), with the gfx950 lane swaps: swapping a
// register with itself leaves, per lane, its own value in one result and the
// partner's in the other, so the larger of the two results is the pair maximum.
template <int ROWS>
__device__ __forceinline__ uint64_t swap_max_key(uint64_t k) {
  const uint32_t lo = (uint32_t)k, hi = (uint32_t)(k >> 32);
  uint32_t l0, l1, h0, h1;
  if constexpr (ROWS == 16) {
    const auto a = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
    const auto b = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
    l0 = a[0], l1 = a[1], h0 = b[0], h1 = b[1];
  } else {
    const auto a = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
    const auto b = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
    l0 = a[0], l1 = a[1], h0 = b[0], h1 = b[1];
  }
  return kmax(((uint64_t)h0 << 32) | l0, ((uint64_t)h1 << 32) | l1);
}

// Largest key over the wave, branch free: DPP within rows of 16 lanes (xor 1,
// xor 2, half-row mirror, row mirror), then lane swaps across rows and halves.
__device__ __forceinline__ uint64_t wave_max_key(uint64_t k) {
  k = kmax(k, dpp_key<0xB1>(k));   // quad_perm [1,0,3,2]
  k = kmax(k, dpp_key<0x4E>(k));   // quad_perm [2,3,0,1]
  k = kmax(k, dpp_key<0x141>(k));  // row_half_mirror
  k = kmax(k, dpp_key<0x140>(k));  // row_mirror
  k = swap_max_key<16>(k);
  k = swap_max_key<32>(k);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)k);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(k >> 32));
  return ((uint64_t)hi << 32) | lo;
}

// Digit planes of 8 values (elements g..g+3, g+16..g+19 of a block) at scale
// 1/inv, in the layout the decode GEMV multiplies (described there).
__device__ __forceinline__ uint4 digit_planes8(const float (&v)[8], float inv) {
  uint32_t z[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) z[i] = ((uint32_t)((int)rintf(v[i] * inv) + 0x8888) ^ 0x8888u) & 0xFFFFu;
  uint32_t p[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint32_t w = 0;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      w |= ((z[m] >> (4 * k)) & 15u) << (8 * m);
      w |= ((z[m + 4] >> (4 * k)) & 15u) << (8 * m + 4);
    }
    p[k] = w;
  }
  return make_uint4(p[0], p[1], p[2], p[3]);
}

// Publishes one router logit to the host: the value's bits with the call's
// sequence number above them, in one 8-byte store at system scope.  The host
// polls the words of a call until every one carries its sequence number; a
// word is written whole, so no fence is needed for the logit itself.
__device__ __forceinline__ void publish_logit(unsigned long long *h_z, long long i, float v,
                                              uint32_t seq) {
  const unsigned long long w =
      ((unsigned long long)seq << 32) | (unsigned long long)__builtin_bit_cast(uint32_t, v);
  __hip_atomic_store(h_z + i, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// Smallest block maximum the 16-bit encoding scales by: keeps 30000 / m finite
// (a block whose values all lie below it is encoded on this coarser scale).
constexpr float kMinBlockMax = 0x1p-100f;

// Digit planes of 8 values of one 32-element block with the block's own scale:
// the block's four units sit in four consecutive active lanes (u % 4 = lane % 4),
// which share their max through two xor shuffles.  X = rint(v * 30000 / m), the
// scale m / 30000 goes to sb (0 for an all-zero block).
__device__ __forceinline__ uint4 block_planes8(const float (&v)[8], float &sb) {
  float m = 0.0f;
#pragma unroll
  for (int q = 0; q < 8; ++q) m = fmaxf(m, fabsf(v[q]));
  m = fmaxf(m, __shfl_xor(m, 1, 64));
  m = fmaxf(m, __shfl_xor(m, 2, 64));
  const float ms = fmaxf(m, kMinBlockMax);
  sb = m > 0.0f ? ms / 30000.0f : 0.0f;
  return digit_planes8(v, m > 0.0f ? 30000.0f / ms : 0.0f);
}

// Exponent e of the power-of-two scale 2^-e that brings a row maximum m into
// [2^13, 2^14) before the binary16 hi/lo split (m = f 2^fe, f in [0.5, 1)), so
// that every row keeps the split's 22 significant bits whatever its magnitude.
// Clamped to [-126, 127] so that 2^e and 2^-e stay finite normal floats; 0 for
// m = 0 or a non-finite m.
__device__ __forceinline__ int pow2_exponent(float m) {
  if (!(m > 0.0f) || !(m <= 3.4e38f)) return 0;
  int fe;
  (void)frexpf(m, &fe);
  return min(127, max(-126, fe - 14));
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
                                                     float *__restrict__ xscale,
                                                     uint4 *__restrict__ xq,
                                                     float *__restrict__ xs,
                                                     unsigned long long *h_z, uint32_t seq) {
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
      if (tt < nt) {
        const float v = bias ? p[tt] + bias[e] : p[tt];
        z[(long long)(t0 + tt) * E + e] = v;
        if (h_z != nullptr) publish_logit(h_z, (long long)(t0 + tt) * E + e, v, seq);
      }
    }
  }
  if (xp == nullptr && xq == nullptr) return;
  const int words = d / 8;
  const int gid = e * 64 + lane, stride = E * 64;
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) {
    if (tt >= nt) break;
    float m = mx[tt];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    const int t = t0 + tt;
    const float *xt = x + (long long)t * d;
    if (xq != nullptr) {
      // decode GEMV input: digit planes with one scale per 32-element block.
      // The four units of a block are four consecutive lanes (j = gid + stride
      // * i, gid and stride multiples of 4 at lane 0, words a multiple of 8), all
      // active together, so two xor shuffles give the block's max.
      const int nbq = xs_units(d >> 5);
      for (int j = gid; j < words; j += stride) {
        const int b = j >> 2, wq = j & 3;
        const float4 a = *reinterpret_cast<const float4 *>(xt + b * 32 + 4 * wq);
        const float4 c = *reinterpret_cast<const float4 *>(xt + b * 32 + 16 + 4 * wq);
        const float v[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
        float sb;
        const uint4 pl = block_planes8(v, sb);
        if (wq == 0) xs[(long long)t * nbq * 4 + b] = sb;
        xq[(long long)t * words + j] = pl;
      }
      continue;
    }
    const int ex2 = pow2_exponent(m);
    const float sc = ldexpf(1.0f, -ex2);
    if (gid == 0) xscale[t] = ldexpf(1.0f, ex2);
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
    }
  }
}

// Decode router: one workgroup per expert for calls of up to four tokens.  The
// workgroup loads the expert's router row and the tokens' x in the pieces the
// decode GEMV's digit planes group (unit j: elements 32b + 4q .. +3 and
// 32b + 16 + 4q .. +3 of block b = j / 4, q = j % 4), all in flight together,
// rounds every product x_i * w_i to fp32 and stores it in LDS at index i.  Wave
// tt then adds token tt's products in the order of router_kernel (lane l:
// i = l, l + 64, ... ascending, the halving tree, the bias), so the logits are
// the same bits.  max|x| per token comes from the same loads, and workgroup e
// turns units 256 e .. 256 e + 255 into digit planes from the registers that
// loaded them, and, when h_x is given, copies those x values to page-locked
// host memory.  Needs tokens * d * 4 bytes of LDS (<= 64 KiB) and d / 8 <= 256 E.
template <int TT>
__global__ __launch_bounds__(256) void router_decode_kernel(const float *__restrict__ x, int T,
                                                            int d, const float *__restrict__ W,
                                                            const float *__restrict__ bias, int E,
                                                            float *__restrict__ z,
                                                            uint4 *__restrict__ xq,
                                                            float *__restrict__ xs, float *h_x,
                                                            unsigned long long *h_z,
                                                            uint32_t seq) {
#pragma clang fp contract(off)
  extern __shared__ float sprod[];  // [TT][d] products
  const int e = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int words = d >> 3;
  const float *wr = W + (long long)e * d;
  float px[TT][8];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) {
#pragma unroll
    for (int i = 0; i < 8; ++i) px[tt][i] = 0.0f;
  }
  constexpr int CH = 4;
  for (int u0 = 0; u0 < words; u0 += 256 * CH) {
    float4 wa[CH], wb[CH], xa[TT][CH], xb[TT][CH];
#pragma unroll
    for (int jj = 0; jj < CH; ++jj) {
      const int j = min(u0 + tid + 256 * jj, words - 1);
      const int o = (j >> 2) * 32 + (j & 3) * 4;
      wa[jj] = *reinterpret_cast<const float4 *>(wr + o);
      wb[jj] = *reinterpret_cast<const float4 *>(wr + o + 16);
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        const float *xr = x + (long long)min(tt, T - 1) * d + o;
        xa[tt][jj] = *reinterpret_cast<const float4 *>(xr);
        xb[tt][jj] = *reinterpret_cast<const float4 *>(xr + 16);
      }
    }
#pragma unroll
    for (int jj = 0; jj < CH; ++jj) {
      const int j = u0 + tid + 256 * jj;
      if (j < words) {
        const int o = (j >> 2) * 32 + (j & 3) * 4;
        const bool mine = u0 + 256 * jj == 256 * e;  // uniform
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
          if (tt < T) {
            const float4 a = xa[tt][jj], c = xb[tt][jj], p = wa[jj], q = wb[jj];
            float4 r, s;
            r.x = a.x * p.x;
            r.y = a.y * p.y;
            r.z = a.z * p.z;
            r.w = a.w * p.w;
            s.x = c.x * q.x;
            s.y = c.y * q.y;
            s.z = c.z * q.z;
            s.w = c.w * q.w;
            *reinterpret_cast<float4 *>(sprod + tt * d + o) = r;
            *reinterpret_cast<float4 *>(sprod + tt * d + o + 16) = s;
            if (mine) {
              px[tt][0] = a.x, px[tt][1] = a.y, px[tt][2] = a.z, px[tt][3] = a.w;
              px[tt][4] = c.x, px[tt][5] = c.y, px[tt][6] = c.z, px[tt][7] = c.w;
            }
          }
        }
      }
    }
  }
  __syncthreads();
  float zv = 0.0f;
  if (wave < T) {
    const float *pr = sprod + wave * d + lane;
    const int M = d >> 6;
    float p = 0.0f;
    for (int m = 0; m < M; ++m) p = p + pr[64 * m];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float o = __shfl_down(p, off, 64);
      if (lane < off) p = p + o;
    }
    zv = bias ? p + bias[e] : p;
    if (lane == 0) z[(long long)wave * E + e] = zv;
  }
  // decode GEMV input: digit planes with one scale per 32-element block (the
  // block's four units are four consecutive threads; words is a multiple of 8,
  // so they pass the test below together)
  const int j = tid + 256 * e;
  if (j < words) {
    const int nbq = xs_units(d >> 5);
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      if (tt >= T) break;
      float sb;
      const uint4 pl = block_planes8(px[tt], sb);
      if ((j & 3) == 0) xs[(long long)tt * nbq * 4 + (j >> 2)] = sb;
      xq[(long long)tt * words + j] = pl;
      if (h_x != nullptr) {
        const int o = (j >> 2) * 32 + (j & 3) * 4;
        float *hx = h_x + (long long)tt * d + o;
        *reinterpret_cast<float4 *>(hx) = make_float4(px[tt][0], px[tt][1], px[tt][2], px[tt][3]);
        *reinterpret_cast<float4 *>(hx + 16) =
            make_float4(px[tt][4], px[tt][5], px[tt][6], px[tt][7]);
      }
    }
    // every thread's copy of x reaches host memory before the workgroup
    // publishes its logits (the host reads x once it has every logit)
    if (h_x != nullptr) __threadfence_system();
  }
  if (h_z != nullptr) {
    __syncthreads();
    if (wave < T && lane == 0) publish_logit(h_z, (long long)wave * E + e, zv, seq);
  }
}

bool router_decode_fits(int T, int d, int E) {
  const int tt = T <= 1 ? 1 : (T <= 2 ? 2 : 4);
  return T >= 1 && T <= 4 && (size_t)tt * d * 4 <= 64 * 1024 && d / 8 <= 256 * E;
}

hipError_t launch_router(const float *x, int T, int d, const float *W, const float *bias, int E,
                         float *z, uint32_t *xp, float *xscale, uint4 *xq, float *xs,
                         hipStream_t s, float *h_x, unsigned long long *h_z, uint32_t seq) {
  const int tt = T <= 1 ? 1 : (T <= 2 ? 2 : 4);
  const size_t lds = (size_t)tt * d * 4;
  if (xq != nullptr && xp == nullptr && router_decode_fits(T, d, E)) {
    if (tt == 1)
      launch_k(router_decode_kernel<1>, dim3(E), dim3(256), lds, s, x, T, d, W, bias, E,
                         z, xq, xs, h_x, h_z, seq);
    else if (tt == 2)
      launch_k(router_decode_kernel<2>, dim3(E), dim3(256), lds, s, x, T, d, W, bias, E,
                         z, xq, xs, h_x, h_z, seq);
    else
      launch_k(router_decode_kernel<4>, dim3(E), dim3(256), lds, s, x, T, d, W, bias, E,
                         z, xq, xs, h_x, h_z, seq);
    return hipGetLastError();
  }
  if (h_x != nullptr) return hipErrorInvalidValue;
  const int gx = (E + 3) / 4;
  if (T <= 1) {
    launch_k((router_kernel<1, 32>), dim3(gx, T), dim3(256), 0, s, x, T, d, W, bias, E,
                       z, xp, xscale, xq, xs, h_z, seq);
  } else if (T <= 4) {
    launch_k((router_kernel<4, 16>), dim3(gx, 1), dim3(256), 0, s, x, T, d, W, bias, E,
                       z, xp, xscale, xq, xs, h_z, seq);
  } else {
    launch_k((router_kernel<8, 8>), dim3(gx, (T + 7) / 8), dim3(256), 0, s, x, T, d, W,
                       bias, E, z, xp, xscale, xq, xs, h_z, seq);
  }
  return hipGetLastError();
}

// ============================================================== top-k + softmax
// One wave per token; E <= 512, so each lane owns NC <= 8 logits (expert
// lane + 64c).  k rounds of a wave-wide maximum over the remaining keys; lane
// j < k ends with the j-th selection (my_e) and its gating weight (my_w).
template <int NC>
__device__ __forceinline__ void topk_token_nc(const float *z, int t, int E, int k, int norm_topk,
                                              int &my_e, float &my_w) {
  const int lane = threadIdx.x & 63;
  float v[NC];
  uint64_t key[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int e = lane + 64 * c;
    v[c] = e < E ? z[(long long)t * E + e] : 0.0f;
    key[c] = e < E ? topk_key(v[c], e) : 0ull;
  }
  my_e = 0;
  float my_v = 0.0f;
  for (int j = 0; j < k; ++j) {
    uint64_t m = key[0];
#pragma unroll
    for (int c = 1; c < NC; ++c) m = kmax(m, key[c]);
    m = wave_max_key(m);
#pragma unroll
    for (int c = 0; c < NC; ++c) key[c] = key[c] == m ? 0ull : key[c];
    if (lane == j) {
      my_e = key_id(m);
      my_v = key_value(m);
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
    for (int c = 0; c < NC; ++c)
      if (lane + 64 * c < E) denom += expf(v[c] - zmax);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) denom += __shfl_xor(denom, off, 64);
  my_w = ex / denom;
}

__device__ __forceinline__ void topk_token(const float *z, int t, int E, int k, int norm_topk,
                                           int &my_e, float &my_w) {
  if (E <= 64)
    topk_token_nc<1>(z, t, E, k, norm_topk, my_e, my_w);
  else if (E <= 128)
    topk_token_nc<2>(z, t, E, k, norm_topk, my_e, my_w);
  else if (E <= 256)
    topk_token_nc<4>(z, t, E, k, norm_topk, my_e, my_w);
  else
    topk_token_nc<8>(z, t, E, k, norm_topk, my_e, my_w);
}

__global__ __launch_bounds__(64) void topk_kernel(const float *__restrict__ z, int T, int E, int k,
                                                  int norm_topk, int32_t *__restrict__ idx,
                                                  float *__restrict__ w, int32_t *h_idx,
                                                  float *h_w) {
  const int t = blockIdx.x, lane = threadIdx.x;
  int my_e;
  float my_w;
  topk_token(z, t, E, k, norm_topk, my_e, my_w);
  if (lane < k) {
    const long long o = (long long)t * k + lane;
    idx[o] = my_e;
    w[o] = my_w;
    h_idx[o] = my_e;
    h_w[o] = my_w;
  }
}

// Decode calls (T <= 4 tokens, T*k + shared pairs <= 64): one workgroup, wave t
// selects token t's experts; then wave 0 maps every pair to its slot through
// `view` (shared pairs to shared_slot) and lists the buckets (pairs grouped by
// slot, a bucket per slot in order of its first pair, pairs ascending).  The
// host makes the same selection from the published logits, so nothing here
// goes to host memory.  Every thread of the workgroup (at least 64 * T) calls it.
__device__ void topk_decode_block(const float *z, int T, int E, const DecodeTopk &a) {
  __shared__ int sidx[kDecodeMaxPairs];
  const int t = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int k = a.k;
  if (t < T) {
    int my_e;
    float my_w;
    topk_token(z, t, E, k, a.norm_topk, my_e, my_w);
    if (lane < k) {
      const int o = t * k + lane;
      a.idx[o] = my_e;
      a.w[o] = my_w;
      sidx[o] = my_e;
    }
  }
  __syncthreads();
  if (t != 0) return;
  const int Pr = T * k;
  const int P = Pr + (a.shared_slot >= 0 ? T : 0);
  int s = -1;
  if (lane < P) s = lane < Pr ? (int)a.view.slot[sidx[lane]] : a.shared_slot;
  if (lane < Pr) a.pair_slot[lane] = s;
  // one pass per distinct slot, in order of its first pair: that pair's lane
  // leads, the ballot of equal slots gives the bucket's pairs
  const uint64_t below = (1ull << lane) - 1ull;
  uint64_t todo = __ballot(s >= 0);
  int nbk = 0;
  while (todo) {
    const int lead = __ffsll((unsigned long long)todo) - 1;
    const int slot = __builtin_amdgcn_readlane(s, lead);
    const uint64_t same = __ballot(s == slot);
    const int cnt = __popcll(same);
    int32_t *e = a.buckets + 1 + nbk * kBucketInts;
    if (s == slot) {
      const int rank = __popcll(same & below);
      e[2 + rank] = lane;
      if (rank == cnt - 1)
        for (int i = cnt; i < kDecodeMaxTokens; ++i) e[2 + i] = lane;
      if (rank == 0) {
        e[0] = slot;
        e[1] = cnt;
      }
    }
    todo &= ~same;
    nbk++;
  }
  if (lane == 0) a.buckets[0] = nbk;
}

__global__ __launch_bounds__(256) void topk_decode_kernel(const float *z, int T, int E,
                                                          DecodeTopk a) {
  topk_decode_block(z, T, E, a);
}

hipError_t launch_topk(const float *z, int T, int E, int k, int norm_topk, int32_t *idx, float *w,
                       int32_t *h_idx, float *h_w, hipStream_t s) {
  launch_k(topk_kernel, dim3(T), dim3(64), 0, s, z, T, E, k, norm_topk, idx, w, h_idx,
                     h_w);
  return hipGetLastError();
}

static bool decode_args_ok(int T, const DecodeTopk &a) {
  return T >= 1 && T <= kDecodeMaxTokens &&
         T * a.k + (a.shared_slot >= 0 ? T : 0) <= kDecodeMaxPairs;
}

hipError_t launch_topk_decode(const float *z, int T, int E, const DecodeTopk &a, hipStream_t s) {
  if (!decode_args_ok(T, a)) return hipErrorInvalidValue;
  launch_k(topk_decode_kernel, dim3(1), dim3(64 * T), 0, s, z, T, E, a);
  return hipGetLastError();
}


// ============================================================== remap + bucket
// One workgroup of 16 waves.  Counts pairs per slot, lays buckets out in slot
// order with their token passes, then places pairs stably (ascending pair id
// inside a bucket): wave w owns the slots s = w (mod 16) and walks the pairs,
// staged through LDS in runs of kRemapRun, with one ballot per 64 pairs.
constexpr int kRemapWaves = 16;
constexpr int kRemapRun = 4096;

__global__ __launch_bounds__(64 * kRemapWaves) void remap_kernel(
    const int32_t *__restrict__ idx, int T, int k, SlotView view, int shared_slot, int n_ids,
    int32_t *__restrict__ meta, int32_t *__restrict__ bucket_pair, int32_t *__restrict__ items) {
  __shared__ int cnt[kMetaB];
  __shared__ int base[kMetaB];
  __shared__ int16_t sl[kRemapRun];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int P_routed = T * k;
  const int P = P_routed + (shared_slot >= 0 ? T : 0);
  for (int s = tid; s < n_ids; s += 64 * kRemapWaves) cnt[s] = 0;
  __syncthreads();
  auto slot_of = [&](int p) -> int {
    return p < P_routed ? (int)view.slot[idx[p]] : shared_slot;
  };
  for (int p = tid; p < P; p += 64 * kRemapWaves) {
    const int s = slot_of(p);
    if (s >= 0) atomicAdd(&cnt[s], 1);
  }
  __syncthreads();
  if (wave == 0) {
    // each lane scans a run of slots; exclusive prefix of buckets, pairs and
    // token passes over the lanes
    const int chunk = (n_ids + 63) / 64;
    const int s0 = min(n_ids, lane * chunk), s1 = min(n_ids, s0 + chunk);
    int na = 0, np = 0, ni = 0;
    for (int s = s0; s < s1; ++s)
      if (cnt[s] > 0) {
        na++;
        np += cnt[s];
        ni += (cnt[s] + kGemmTokens - 1) / kGemmTokens;
      }
    int ia = na, ip = np, ii = ni;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int oa = __shfl_up(ia, off, 64), op = __shfl_up(ip, off, 64),
                oi = __shfl_up(ii, off, 64);
      if (lane >= off) {
        ia += oa;
        ip += op;
        ii += oi;
      }
    }
    int a = ia - na, q = ip - np, it = ii - ni;
    for (int s = s0; s < s1; ++s) {
      if (cnt[s] > 0) {
        meta[2 + a] = s;
        meta[2 + kMetaB + a] = q;
        meta[2 + 2 * kMetaB + a] = cnt[s];
        base[s] = q;
        for (int j = 0; j * kGemmTokens < cnt[s]; ++j) items[1 + it++] = a | (j << 16);
        q += cnt[s];
        a++;
      }
    }
    if (lane == 63) {
      meta[0] = ia;
      meta[1] = ip;
      items[0] = ii;
    }
  }
  __syncthreads();
  const uint64_t below = (1ull << lane) - 1ull;
  for (int c0 = 0; c0 < P; c0 += kRemapRun) {
    const int n = min(kRemapRun, P - c0);
    for (int i = tid; i < n; i += 64 * kRemapWaves) sl[i] = (int16_t)slot_of(c0 + i);
    __syncthreads();
    for (int s = wave; s < n_ids; s += kRemapWaves) {
      if (cnt[s] == 0) continue;
      int pos = base[s];  // wave-owned: the next free place of bucket s
      for (int i0 = 0; i0 < n; i0 += 64) {
        const int i = i0 + lane;
        const bool mine = i < n && sl[i] == s;
        const uint64_t m = __ballot(mine);
        if (mine) bucket_pair[pos + __popcll(m & below)] = c0 + i;
        pos += __popcll(m);
      }
      if (lane == 0) base[s] = pos;
    }
    __syncthreads();
  }
}

hipError_t launch_remap(const int32_t *idx, int T, int k, const SlotView &view, int shared_slot,
                        int n_slot_ids, int32_t *meta, int32_t *bucket_pair, int32_t *items,
                        hipStream_t s) {
  if (n_slot_ids < 1 || n_slot_ids > kMetaB) return hipErrorInvalidValue;
  launch_k(remap_kernel, dim3(1), dim3(64 * kRemapWaves), 0, s, idx, T, k, view,
                     shared_slot, n_slot_ids, meta, bucket_pair, items);
  return hipGetLastError();
}

// ============================================================== decode GEMV arithmetic
// Activations enter the decode GEMV as 16-bit fixed point: X = rint(v / s) with
// one scale per 32-element block, s = max|v over the block| / 30000 (for x and
// for h alike, so that one large channel costs only its own block), split into
// four signed base-16 digits c_0..c_3 in [-8, 7], X = sum_k 16^k c_k.  For
// X + 0x8888 the digit nibbles are those of ((X + 0x8888) ^ 0x8888), so no
// carry chain is needed.  A digit plane is laid out like the weights' nibble
// words: in word j of a block, nibble 2m holds element 4j+m and nibble 2m+1
// element 4j+m+16.  XOR with 0x88888888 turns a weight word's nibbles q into
// signed nibbles q - 8, so one v_dot8_i32_i4 per (word, plane) accumulates
// sum (q - 8) c_k exactly, and the four planes meet with shifts by 4 bits:
// I = sum_i (q_i - 8) X_i, |I| <= 32 * 8 * 34952 < 2^24, exact in int32 and in
// its float32 conversion.  A block then contributes d * s * I.

// sum over one block of (q - 8) * X, X given as digit planes P[word].{x,y,z,w}
__device__ __forceinline__ int dot_block_i4(const uint4 &w, const uint4 (&P)[4]) {
  const int w0 = (int)(w.x ^ 0x88888888u), w1 = (int)(w.y ^ 0x88888888u);
  const int w2 = (int)(w.z ^ 0x88888888u), w3 = (int)(w.w ^ 0x88888888u);
  int acc = __builtin_amdgcn_sdot8(w0, (int)P[0].w, 0, false);
  acc = __builtin_amdgcn_sdot8(w1, (int)P[1].w, acc, false);
  acc = __builtin_amdgcn_sdot8(w2, (int)P[2].w, acc, false);
  acc = __builtin_amdgcn_sdot8(w3, (int)P[3].w, acc, false);
  acc <<= 4;
  acc = __builtin_amdgcn_sdot8(w0, (int)P[0].z, acc, false);
  acc = __builtin_amdgcn_sdot8(w1, (int)P[1].z, acc, false);
  acc = __builtin_amdgcn_sdot8(w2, (int)P[2].z, acc, false);
  acc = __builtin_amdgcn_sdot8(w3, (int)P[3].z, acc, false);
  acc <<= 4;
  acc = __builtin_amdgcn_sdot8(w0, (int)P[0].y, acc, false);
  acc = __builtin_amdgcn_sdot8(w1, (int)P[1].y, acc, false);
  acc = __builtin_amdgcn_sdot8(w2, (int)P[2].y, acc, false);
  acc = __builtin_amdgcn_sdot8(w3, (int)P[3].y, acc, false);
  acc <<= 4;
  acc = __builtin_amdgcn_sdot8(w0, (int)P[0].x, acc, false);
  acc = __builtin_amdgcn_sdot8(w1, (int)P[1].x, acc, false);
  acc = __builtin_amdgcn_sdot8(w2, (int)P[2].x, acc, false);
  acc = __builtin_amdgcn_sdot8(w3, (int)P[3].x, acc, false);
  return acc;
}

__device__ __forceinline__ float silu_f(float v) { return v / (1.0f + expf(-v)); }

__device__ __forceinline__ int pair_row(const GemvArgs &a, int p) {
  return p < a.T * a.k ? p / a.k : p - a.T * a.k;
}

// Expert weights are read once per launch and not again for many calls (other
// layers' experts pass through the caches in between), so the GEMV loads them
// with the nontemporal hint: they stream past the caches' retained lines (the
// activations, scales and router rows) instead of replacing them.  About 5%
// faster for both GEMV kernels at 6144 x 2048 experts.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ldnt(const uint4 *p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
// ============================================================== bucket lookup
// The expert record and pairs of bucket b on the decode path, from the list the
// decode top-k kernel wrote (BK_LIST; workgroup-uniform, so scalar loads) or
// from a host-built table passed by value (BK_TABLE).  pairs[i] for i >= cnt
// repeats the last pair.
template <int TT>
struct Bucket {
  int cnt;
  int pairs[TT];
  const uint8_t *src;
};

enum { BK_LIST = 1, BK_TABLE = 2 };

// a[i] for a runtime i without indexing a register array (no scratch)
template <int N>
__device__ __forceinline__ int pick(const int (&a)[N], int i) {
  int r = a[0];
#pragma unroll
  for (int q = 1; q < N; ++q) r = i == q ? a[q] : r;
  return r;
}

// Pair tt of bucket b for a lane-varying tt: a select chain for TT <= 2; above
// that the compiler turns selects back into an indexed register array (which
// lives in scratch), so the pair is read again from the list or the table.
template <int TT, int MODE>
__device__ __forceinline__ int pair_at(const GemvArgs &a, const BucketTable &tab, int b,
                                       const Bucket<TT> &bk, int tt) {
  if constexpr (TT <= 2) {
    return pick(bk.pairs, tt);
  } else if constexpr (MODE == BK_TABLE) {
    return tab.pairs[b][min(tt, bk.cnt - 1)];
  } else {
    return a.bt[1 + b * kBucketInts + 2 + tt];
  }
}

template <int TT, int MODE>
__device__ __forceinline__ bool find_bucket(const GemvArgs &a, const BucketTable &tab, int b,
                                            Bucket<TT> &bk) {
  if constexpr (MODE == BK_TABLE) {
    if (b >= tab.n) return false;
    bk.src = tab.src[b];
    bk.cnt = tab.cnt[b];
#pragma unroll
    for (int i = 0; i < TT; ++i) bk.pairs[i] = tab.pairs[b][min(i, bk.cnt - 1)];
    return true;
  }
  if (b >= a.bt[0]) return false;
  const int32_t *e = a.bt + 1 + b * kBucketInts;
  bk.src = a.slots + (long long)e[0] * a.rec_bytes;
  bk.cnt = e[1];
#pragma unroll
  for (int i = 0; i < TT; ++i) bk.pairs[i] = e[2 + i];
  return true;
}

// ============================================================== decode Q4 GEMV
// Workgroup = 4 waves, one bucket (blockIdx.y) and a tile of rows (blockIdx.x).
// G lanes share a row, RW = 64/G rows side by side, R row steps per lane; the
// K blocks of a row are split over KS waves (block j = gl + G*(ks + KS*it)), so a
// wave instruction reads G consecutive 16-byte nibble blocks of each of RW rows.
// The bucket's activation planes (x for gate/up, h for down, up to TT tokens)
// sit in LDS; their global loads are issued before the weight loads, so waiting
// for them never waits for HBM.  The next step's weights are loaded before the
// current step is multiplied.  Partial sums meet across the G lanes with xor
// shuffles and across the KS waves in LDS, in a fixed order.
constexpr int kStageChunks = 6;  // 16-byte staging chunks per thread and round
constexpr int kHUnits = 2;       // down prologue: h words per thread and round
constexpr int kScaleChunks = 2;  // down prologue: scale chunks per thread and round

// Bytes of the row scales a workgroup stages: rows [r0, r0 + n) of nb binary16
// scales, in 16-byte chunks.  r0 is a multiple of the workgroup's row count
// (>= 8) and a section holds rows * nb * 2 bytes, a multiple of 16 (nb and
// rows even, one of them a multiple of 8 for every shape the cache admits), so
// chunks start aligned and never pass the section's end.
__device__ __forceinline__ int scale_chunks(int rows_here, int nb) {
  return (rows_here * nb * 2 + 15) / 16;
}

// gate/up + SwiGLU.  LDS: the bucket's x planes [TT][nb][4], its x block scales
// [TT][4 * xs_units(nb)], then the gate and the up scales of the workgroup's rows.
template <int G, int KS, int R, int TT, int MODE, int NW, int PF>
__global__ __launch_bounds__(64 * NW) void q4_gateup_kernel(GemvArgs a, BucketTable tab) {
  constexpr int RW = 64 / G;
  constexpr int RWG = (NW / KS) * RW * R;
  constexpr int NT = 64 * NW;
  extern __shared__ uint4 sx[];
  __shared__ float red[NW][RW * R][TT][2];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, tid = threadIdx.x;
  const int ks = wave % KS, rg = wave / KS;
  Bucket<TT> bk;
  if (!find_bucket<TT, MODE>(a, tab, blockIdx.y, bk)) return;
  const uint8_t *rec = bk.src;
  const int nb = a.nb;
  const int gl = lane % G;
  const int r0 = blockIdx.x * RWG;
  const int rows_here = min(RWG, a.rows - r0);
  const int rbase = r0 + rg * RW * R + lane / G;
  const uint4 *q0 = reinterpret_cast<const uint4 *>(rec + a.off_q0);
  const uint4 *q1 = reinterpret_cast<const uint4 *>(rec + a.off_q1);
  const uint4 *c0 = reinterpret_cast<const uint4 *>(rec + a.off_s0 + (long long)r0 * nb * 2);
  const uint4 *c1 = reinterpret_cast<const uint4 *>(rec + a.off_s1 + (long long)r0 * nb * 2);
  int tok[TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) tok[tt] = pair_row(a, bk.pairs[tt]);
  // rows past the end read the last row and are never written
  int rl[R];  // row within the workgroup's staged scales
  long long ro[R];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int r = min(rbase + RW * i, a.rows - 1);
    rl[i] = (r - r0) * nb;
    ro[i] = (long long)r * nb;
  }
  const int NI = (nb + G * KS - 1) / (G * KS);
  auto blk_of = [&](int it) { return min(gl + G * (ks + KS * it), nb - 1); };
  // staging: x planes, x block scales, gate scales, up scales, as one run of
  // 16-byte units
  const int nbq = xs_units(nb);
  const int n_x = TT * nb * 4, n_xs = TT * nbq, n_s = scale_chunks(rows_here, nb);
  const int n_stage = n_x + n_xs + 2 * n_s;
  const uint4 *xs4 = reinterpret_cast<const uint4 *>(a.xs);
  auto row_of = [&](int tt) {
    return TT <= 2 ? pick(tok, tt) : pair_row(a, pair_at<TT, MODE>(a, tab, blockIdx.y, bk, tt));
  };
  auto stage_ld = [&](int u) -> uint4 {
    u = min(u, n_stage - 1);
    if (u < n_x) {
      const int tt = u / (nb * 4);
      return a.xq[(long long)row_of(tt) * nb * 4 + (u - tt * nb * 4)];
    }
    u -= n_x;
    if (u < n_xs) {
      const int tt = u / nbq;
      return xs4[(long long)row_of(tt) * nbq + (u - tt * nbq)];
    }
    u -= n_xs;
    return u < n_s ? c0[u] : c1[u - n_s];
  };
  uint4 xv[kStageChunks];
#pragma unroll
  for (int c = 0; c < kStageChunks; ++c) xv[c] = stage_ld(tid + NT * c);
  // keep the weight loads behind the staging loads
  __builtin_amdgcn_sched_barrier(0);
  // weights of the first PF K steps in flight before the staging completes
  uint4 wg[PF][R], wu[PF][R];
#pragma unroll
  for (int f = 0; f < PF; ++f) {
    const int j = blk_of(min(f, NI - 1));
#pragma unroll
    for (int i = 0; i < R; ++i) {
      wg[f][i] = ldnt(&q0[ro[i] + j]);
      wu[f][i] = ldnt(&q1[ro[i] + j]);
    }
  }
#pragma unroll
  for (int c = 0; c < kStageChunks; ++c)
    if (tid + NT * c < n_stage) sx[tid + NT * c] = xv[c];
  for (int u0 = NT * kStageChunks; u0 < n_stage; u0 += NT * kStageChunks) {
    uint4 yv[kStageChunks];
#pragma unroll
    for (int c = 0; c < kStageChunks; ++c) yv[c] = stage_ld(u0 + tid + NT * c);
#pragma unroll
    for (int c = 0; c < kStageChunks; ++c)
      if (u0 + tid + NT * c < n_stage) sx[u0 + tid + NT * c] = yv[c];
  }
  __syncthreads();
  const float *sxs = reinterpret_cast<const float *>(sx + n_x);
  const _Float16 *sg = reinterpret_cast<const _Float16 *>(sx + n_x + n_xs);
  const _Float16 *su = reinterpret_cast<const _Float16 *>(sx + n_x + n_xs + n_s);
  float ag[R][TT], au[R][TT];
#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      ag[i][tt] = 0.0f;
      au[i][tt] = 0.0f;
    }
  for (int it0 = 0; it0 < NI; it0 += PF) {
#pragma unroll
    for (int f = 0; f < PF; ++f) {
      const int it = it0 + f;
      if (it < NI) {
        const int j0 = gl + G * (ks + KS * it);
        const bool ok = j0 < nb;
        const int j = min(j0, nb - 1);
        uint4 cw[R], cv[R];
#pragma unroll
        for (int i = 0; i < R; ++i) {
          cw[i] = wg[f][i];
          cv[i] = wu[f][i];
        }
        if (it + PF < NI) {
          const int jn = blk_of(it + PF);
#pragma unroll
          for (int i = 0; i < R; ++i) {
            wg[f][i] = ldnt(&q0[ro[i] + jn]);
            wu[f][i] = ldnt(&q1[ro[i] + jn]);
          }
        }
        float dg[R], du[R];
#pragma unroll
        for (int i = 0; i < R; ++i) {
          dg[i] = ok ? (float)sg[rl[i] + j] : 0.0f;
          du[i] = ok ? (float)su[rl[i] + j] : 0.0f;
        }
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
          uint4 P[4];
#pragma unroll
          for (int w = 0; w < 4; ++w) P[w] = sx[(tt * nb + j) * 4 + w];
          const float se = sxs[tt * nbq * 4 + j];
#pragma unroll
          for (int i = 0; i < R; ++i) {
            ag[i][tt] = __builtin_fmaf((float)dot_block_i4(cw[i], P) * se, dg[i], ag[i][tt]);
            au[i][tt] = __builtin_fmaf((float)dot_block_i4(cv[i], P) * se, du[i], au[i][tt]);
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
        ag[i][tt] += __shfl_xor(ag[i][tt], o, 64);
        au[i][tt] += __shfl_xor(au[i][tt], o, 64);
      }
    }
  if (gl == 0) {
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        red[wave][lane / G + RW * i][tt][0] = ag[i][tt];
        red[wave][lane / G + RW * i][tt][1] = au[i][tt];
      }
  }
  __syncthreads();
  for (int o = tid; o < (NW / KS) * RW * R * TT; o += NT) {
    const int g = o / (RW * R * TT), rr = (o / TT) % (RW * R), tt = o % TT;
    const int r = r0 + g * RW * R + rr;
    if (r < a.rows && tt < bk.cnt) {
      float gg = 0.0f, uu = 0.0f;
#pragma unroll
      for (int q = 0; q < KS; ++q) {
        gg += red[g * KS + q][rr][tt][0];
        uu += red[g * KS + q][rr][tt][1];
      }
      const int p = pair_at<TT, MODE>(a, tab, blockIdx.y, bk, tt);
      a.out[(long long)p * a.rows + r] = silu_f(gg) * uu;
    }
  }
}

// down: y = D h.  The prologue turns the bucket's h rows (fp32, by pair) into
// digit planes with one scale per 32-element block (thread = one word of one
// block; the block's four threads share its max through two xor shuffles) and
// stages the workgroup's row scales.  LDS: planes [TT][nb][4], block scales
// [TT][nb] (fp32), row scales.
template <int G, int KS, int R, int TT, int MODE, int NW, int PF>
__global__ __launch_bounds__(64 * NW) void q4_down_kernel(GemvArgs a, BucketTable tab) {
  constexpr int RW = 64 / G;
  constexpr int RWG = (NW / KS) * RW * R;
  constexpr int NT = 64 * NW;
  extern __shared__ uint4 sh[];
  __shared__ float red[NW][RW * R][TT];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, tid = threadIdx.x;
  const int ks = wave % KS, rg = wave / KS;
  Bucket<TT> bk;
  if (!find_bucket<TT, MODE>(a, tab, blockIdx.y, bk)) return;
  const uint8_t *rec = bk.src;
  const int nb = a.nb;
  const int n_units = TT * nb * 4;
  float *sscale = reinterpret_cast<float *>(sh + n_units);
  uint4 *srow = sh + n_units + (TT * nb + 3) / 4;
  const int gl = lane % G;
  const int r0 = blockIdx.x * RWG;
  const int rows_here = min(RWG, a.rows - r0);
  const int rbase = r0 + rg * RW * R + lane / G;
  const uint4 *q0 = reinterpret_cast<const uint4 *>(rec + a.off_q0);
  const uint4 *c0 = reinterpret_cast<const uint4 *>(rec + a.off_s0 + (long long)r0 * nb * 2);
  int rl[R];
  long long ro[R];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int r = min(rbase + RW * i, a.rows - 1);
    rl[i] = (r - r0) * nb;
    ro[i] = (long long)r * nb;
  }
  const int NI = (nb + G * KS - 1) / (G * KS);
  auto blk_of = [&](int it) { return min(gl + G * (ks + KS * it), nb - 1); };
  const int n_s = scale_chunks(rows_here, nb);
  auto load_units = [&](int u0, float4 (&v0)[kHUnits], float4 (&v1)[kHUnits]) {
#pragma unroll
    for (int c = 0; c < kHUnits; ++c) {
      if (u0 + NT * c >= n_units) break;  // uniform
      const int u = min(u0 + tid + NT * c, n_units - 1);
      const int tt = u / (nb * 4), rem = u - tt * nb * 4;
      const int b = rem >> 2, j = rem & 3;
      const float *hr =
          a.in + (long long)pair_at<TT, MODE>(a, tab, blockIdx.y, bk, tt) * nb * 32 + b * 32 + 4 * j;
      v0[c] = *reinterpret_cast<const float4 *>(hr);
      v1[c] = *reinterpret_cast<const float4 *>(hr + 16);
    }
  };
  auto put_units = [&](int u0, const float4 (&v0)[kHUnits], const float4 (&v1)[kHUnits]) {
#pragma unroll
    for (int c = 0; c < kHUnits; ++c) {
      const int u = u0 + tid + NT * c;
      if (u0 + NT * c >= n_units) break;  // uniform
      const float v[8] = {v0[c].x, v0[c].y, v0[c].z, v0[c].w, v1[c].x, v1[c].y, v1[c].z, v1[c].w};
      float sb;
      const uint4 pl = block_planes8(v, sb);
      if (u < n_units) {
        sh[u] = pl;
        if ((u & 3) == 0) sscale[u >> 2] = sb;
      }
    }
  };
  float4 hv0[kHUnits], hv1[kHUnits];
  load_units(0, hv0, hv1);
  static_assert(kScaleChunks == 2, "row scale staging is written out for 2 chunks");
  const uint4 sv0 = c0[min(tid, n_s - 1)], sv1 = c0[min(tid + NT, n_s - 1)];
  // keep the weight loads behind the staging loads
  __builtin_amdgcn_sched_barrier(0);
  // weights of the first PF K steps in flight before the prologue runs
  uint4 wd[PF][R];
#pragma unroll
  for (int f = 0; f < PF; ++f) {
    const int j = blk_of(min(f, NI - 1));
#pragma unroll
    for (int i = 0; i < R; ++i) wd[f][i] = ldnt(&q0[ro[i] + j]);
  }
  if (tid < n_s) srow[tid] = sv0;
  if (tid + NT < n_s) srow[tid + NT] = sv1;
  for (int u0 = NT * kScaleChunks; u0 < n_s; u0 += NT) {
    if (u0 + tid < n_s) srow[u0 + tid] = c0[u0 + tid];
  }
  put_units(0, hv0, hv1);
  for (int u0 = NT * kHUnits; u0 < n_units; u0 += NT * kHUnits) {
    float4 gv0[kHUnits], gv1[kHUnits];
    load_units(u0, gv0, gv1);
    put_units(u0, gv0, gv1);
  }
  __syncthreads();
  const _Float16 *sd = reinterpret_cast<const _Float16 *>(srow);
  float ac[R][TT];
#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) ac[i][tt] = 0.0f;
  for (int it0 = 0; it0 < NI; it0 += PF) {
#pragma unroll
    for (int f = 0; f < PF; ++f) {
      const int it = it0 + f;
      if (it < NI) {
        const int j0 = gl + G * (ks + KS * it);
        const bool ok = j0 < nb;
        const int j = min(j0, nb - 1);
        uint4 cw[R];
#pragma unroll
        for (int i = 0; i < R; ++i) cw[i] = wd[f][i];
        if (it + PF < NI) {
          const int jn = blk_of(it + PF);
#pragma unroll
          for (int i = 0; i < R; ++i) wd[f][i] = ldnt(&q0[ro[i] + jn]);
        }
        float dd[R];
#pragma unroll
        for (int i = 0; i < R; ++i) dd[i] = ok ? (float)sd[rl[i] + j] : 0.0f;
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
          uint4 P[4];
#pragma unroll
          for (int w = 0; w < 4; ++w) P[w] = sh[(tt * nb + j) * 4 + w];
          const float se = sscale[tt * nb + j];
#pragma unroll
          for (int i = 0; i < R; ++i)
            ac[i][tt] = __builtin_fmaf((float)dot_block_i4(cw[i], P) * se, dd[i], ac[i][tt]);
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
#pragma unroll
      for (int o = G / 2; o >= 1; o >>= 1) ac[i][tt] += __shfl_xor(ac[i][tt], o, 64);
    }
  if (gl == 0) {
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) red[wave][lane / G + RW * i][tt] = ac[i][tt];
  }
  __syncthreads();
  for (int o = tid; o < (NW / KS) * RW * R * TT; o += NT) {
    const int g = o / (RW * R * TT), rr = (o / TT) % (RW * R), tt = o % TT;
    const int r = r0 + g * RW * R + rr;
    if (r < a.rows && tt < bk.cnt) {
      float v = 0.0f;
#pragma unroll
      for (int q = 0; q < KS; ++q) v += red[g * KS + q][rr][tt];
      a.out[(long long)pair_at<TT, MODE>(a, tab, blockIdx.y, bk, tt) * a.rows + r] = v;
    }
  }
}

template <bool GLU, int G, int KS, int R, int TT, int MODE, int PF>
static void launch_one(const GemvArgs &a, const BucketTable &tab, int nbk, size_t lds,
                       hipStream_t s) {
  constexpr int NW = 4;
  constexpr int RWG = (NW / KS) * (64 / G) * R;
  const dim3 grid((a.rows + RWG - 1) / RWG, nbk);
  if constexpr (GLU)
    launch_k((q4_gateup_kernel<G, KS, R, TT, MODE, NW, PF>), grid, dim3(64 * NW), lds, s,
                       a, tab);
  else
    launch_k((q4_down_kernel<G, KS, R, TT, MODE, NW, PF>), grid, dim3(64 * NW), lds, s,
                       a, tab);
}

template <bool GLU, int G, int KS, int R, int PF = 1>
static void launch_tt(const GemvArgs &a, const BucketTable &tab, int nbk, int TT, size_t lds,
                      hipStream_t s) {
  const bool t = tab.n >= 0;
  switch (TT) {
    case 1:
      t ? launch_one<GLU, G, KS, R, 1, BK_TABLE, PF>(a, tab, nbk, lds, s)
        : launch_one<GLU, G, KS, R, 1, BK_LIST, PF>(a, tab, nbk, lds, s);
      break;
    case 2:
      t ? launch_one<GLU, G, KS, R, 2, BK_TABLE, PF>(a, tab, nbk, lds, s)
        : launch_one<GLU, G, KS, R, 2, BK_LIST, PF>(a, tab, nbk, lds, s);
      break;
    default:
      t ? launch_one<GLU, G, KS, R, 4, BK_TABLE, PF>(a, tab, nbk, lds, s)
        : launch_one<GLU, G, KS, R, 4, BK_LIST, PF>(a, tab, nbk, lds, s);
      break;
  }
}

hipError_t launch_gemv(const GemvArgs &a, const BucketTable *tab, const GemvShape &sh, bool glu,
                       int n_buckets, hipStream_t s) {
  if (n_buckets <= 0) return hipSuccess;
  if (!tab && !a.bt) return hipErrorInvalidValue;
  BucketTable none;
  none.n = -1;
  const BucketTable &t = tab ? *tab : none;
  const size_t lds = gemv_lds_bytes(glu, a.nb, sh.TT);
  const int key = (glu ? 1000 : 0) + sh.G * 100 + sh.KS * 10 + sh.R;
  switch (key) {
    case 1000 + 1600 + 40 + 2: launch_tt<true, 16, 4, 2>(a, t, n_buckets, sh.TT, lds, s); break;
    case 1000 + 800 + 40 + 1:
      // a launch of one or two buckets (the fills of a call) is latency bound:
      // all three K steps of a Gemma-sized row in flight at once
      if (n_buckets <= 2)
        launch_tt<true, 8, 4, 1, 3>(a, t, n_buckets, sh.TT, lds, s);
      else
        launch_tt<true, 8, 4, 1>(a, t, n_buckets, sh.TT, lds, s);
      break;
    case 1000 + 800 + 10 + 2: launch_tt<true, 8, 1, 2>(a, t, n_buckets, sh.TT, lds, s); break;
    case 800 + 40 + 4: launch_tt<false, 8, 4, 4>(a, t, n_buckets, sh.TT, lds, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t o) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(m), "v"(o));
  return r;
}

// ============================================================== prefill MFMA GEMM
// Per workgroup: 8 waves over one pass of up to 32 of a bucket's tokens (one or
// two 16-token tiles, a compile-time count) and a tile of weight rows of the
// bucket's expert.  Each wave owns 32 rows (two groups of 16) of one matrix:
// for the fused GLU, waves 0-3 take 128 rows of the gate projection and waves
// 4-7 the same rows of the up projection (the gate sums reach the up waves
// through LDS at the end); the down GEMM gives its 8 waves 256 rows.
// The MFMA takes the tokens as its A operand and the weight rows as its B
// operand, so that a lane's accumulators (C: lane l = tokens 4*(l/16)+i, weight
// row l%16) all belong to one weight row and each block scale is one register
// value; both row groups of a wave share every activation fragment read.
// A wave streams its rows through registers: for each group, lane l loads the
// whole 16-byte nibble block 4c + l/16 of row l%16 for K chunk c (4 blocks),
// two chunks ahead of the one it multiplies.  A 4 x 4 word transpose across the
// four 16-lane rows of the wave (two rounds of gfx950 lane swaps) turns "block
// per lane row" into the operand layout (lane l: row l%16, word l/16 of each of
// the 4 blocks).  Block scales: rows of a multiple of 32 blocks take them in
// windows of 32 blocks through a wave-private LDS table; other rows load each
// chunk's scales beside its weights, and the same lane swaps gather the four
// scales of a row into every lane of that row.  The activation tiles (binary16
// hi/lo pairs for the chunk's 4 blocks and the pass's tokens) are staged per
// chunk for the whole workgroup in two LDS buffers, with one barrier per chunk.
// A lane turns its nibble word into binary16 q - 8 exactly: the exponent trick
// puts q (or 16 q, for the nibbles at bits 4-7 of each half) in the mantissa of
// 1024, and one packed subtract (or multiply-add by 1/16) leaves q - 8.  Each
// 32-weight block is one pair of v_mfma_f32_16x16x32_f16 (x hi, x lo) per token
// tile and row group, and the block scale d multiplies the pair's result into
// the fp32 accumulators.  Operand lanes: weights lane l = row l%16 and the 8 K
// values of word l/16 of the block (elements g, g+2, g+16, g+18, g+1, g+3,
// g+17, g+19 with g = 4*(l/16)); tokens lane l = token l%16 and the same 8 K
// values.
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int K6_WAVES = 8;
constexpr int K6_KC = 4;                // blocks per K chunk
constexpr int K6_TOK = kGemmTokens;     // tokens per pass (two tiles of 16)
constexpr int K6_PD = 2;                // K chunks in flight per wave

// weight rows per workgroup
constexpr int k6_rows(bool glu) { return glu ? 32 * K6_WAVES / 2 : 32 * K6_WAVES; }

// binary16 pairs of (q - 8) for the 8 nibbles of word w, in the operand order
__device__ __forceinline__ half8_t decode_word_h(uint32_t w) {
  const uint32_t m = 0x000F000Fu, m16 = 0x00F000F0u, mag = 0x64006400u;
  const half2_t off = {(_Float16)1032.0f, (_Float16)1032.0f};
  const half2_t sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  const half2_t off16 = {(_Float16)-72.0f, (_Float16)-72.0f};
  const uint32_t w8 = w >> 8;
  // 1024 + q - 1032, and (1024 + 16 q) / 16 - 72: both exact in binary16
  const half2_t p0 = __builtin_bit_cast(half2_t, and_or(w, m, mag)) - off;
  const half2_t p1 = __builtin_elementwise_fma(__builtin_bit_cast(half2_t, and_or(w, m16, mag)),
                                               sixteenth, off16);
  const half2_t p2 = __builtin_bit_cast(half2_t, and_or(w8, m, mag)) - off;
  const half2_t p3 = __builtin_elementwise_fma(__builtin_bit_cast(half2_t, and_or(w8, m16, mag)),
                                               sixteenth, off16);
  half8_t r;
  r[0] = p0[0];
  r[1] = p0[1];
  r[2] = p1[0];
  r[3] = p1[1];
  r[4] = p2[0];
  r[5] = p2[1];
  r[6] = p3[0];
  r[7] = p3[1];
  return r;
}

// 4 x 4 transpose of 32-bit words over the wave's four 16-lane rows: on entry
// row g holds (w0..w3) of block g, on exit row g holds word g of blocks 0..3.
// Round 1 swaps the off-diagonal 2 x 2 quarters between lane halves 0-31 and
// 32-63, round 2 the off-diagonal entries between rows 2j and 2j+1.
__device__ __forceinline__ uint4 transpose_rows(uint4 v) {
  const auto a = __builtin_amdgcn_permlane32_swap(v.x, v.z, false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(v.y, v.w, false, false);
  const auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
  const auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
  return make_uint4(c[0], c[1], d[0], d[1]);
}

// All-gather over the wave's four 16-lane rows: on entry row g holds s_g, on
// exit every row holds (s_0, s_1, s_2, s_3).  permlane32_swap exchanges the
// upper half of its first operand with the lower half of its second, so after
// it each lane holds (s_{g mod 2}, s_{g mod 2 + 2}); permlane16_swap then does
// the same between rows 2j + 1 and 2j.
__device__ __forceinline__ uint4 gather_rows(uint32_t s) {
  const auto a = __builtin_amdgcn_permlane32_swap(s, s, false, false);
  const auto b = __builtin_amdgcn_permlane16_swap(a[0], a[0], false, false);
  const auto c = __builtin_amdgcn_permlane16_swap(a[1], a[1], false, false);
  return make_uint4(b[0], b[1], c[0], c[1]);
}

struct K6Lds {
  // [buf][token][word * 2 + hi/lo]; one spare entry per token row staggers the
  // rows over the banks (row stride 528 B = 16 B mod 128 B).  After the last
  // chunk the buffers hold the gate sums for the up waves.
  uint4 B[2][K6_TOK][K6_KC * 8 + 1];
  // block scales of windows of 32 blocks, two buffers, wave-private: [buffer]
  // [wave][row group][row][16 binary16 pairs + 2 spare] (row stride 72 B: the
  // 16 rows' 8-byte reads fall on distinct banks)
  uint32_t SC[2][K6_WAVES][2][16][18];
  int tok[K6_TOK];
};

// The pass body for NT token tiles of 16 (a pass of up to 16 tokens stages and
// multiplies half the activation rows).
template <bool GLU, int NT, bool SW>
__device__ __forceinline__ void mfma_pass(const GemvArgs &a, K6Lds &L, int item, int tile);

template <bool GLU>
__global__ __launch_bounds__(64 * K6_WAVES, 4) void q4_mfma_kernel(GemvArgs a) {
  __shared__ K6Lds L;
  // XCD-aware order: workgroup l of the grid runs on XCD l % 8; each XCD takes a
  // contiguous run of the (item, row tile) work, so that the row tiles of one
  // item, which read the same activations, share that XCD's L2.  Workgroups past
  // their XCD's run exit.
  const int gx = gridDim.x;
  const int n_work = a.items[0] * gx;
  const int lin = blockIdx.y * gx + blockIdx.x;
  const int xcd = lin & 7, r = lin >> 3;
  const int q8 = n_work >> 3, rem = n_work & 7;
  if (r >= q8 + (xcd < rem ? 1 : 0)) return;
  const int work = xcd * q8 + min(xcd, rem) + r;
  const int item = a.items[1 + work / gx];
  const int tile = work % gx;
  const int ntok = min(K6_TOK, a.meta[2 + 2 * kMetaB + (item & 0xFFFF)] - (item >> 16) * K6_TOK);
  // rows of a multiple of 32 blocks take their scales in windows of 32 blocks
  // (two 16-byte loads per lane and window); other rows per chunk
  const bool sw = (a.nb & 31) == 0;
  if (ntok > 16) {
    if (sw)
      mfma_pass<GLU, 2, true>(a, L, item, tile);
    else
      mfma_pass<GLU, 2, false>(a, L, item, tile);
  } else {
    if (sw)
      mfma_pass<GLU, 1, true>(a, L, item, tile);
    else
      mfma_pass<GLU, 1, false>(a, L, item, tile);
  }
}

template <bool GLU, int NT, bool SW>
__device__ __forceinline__ void mfma_pass(const GemvArgs &a, K6Lds &L, int item, int tile) {
  constexpr int NTH = 64 * K6_WAVES;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = GLU ? wave / (K6_WAVES / 2) : 0;             // matrix of this wave
  const int rw = GLU ? wave % (K6_WAVES / 2) : wave;        // its 32-row slice
  const int bucket = item & 0xFFFF;
  const int g0 = (item >> 16) * K6_TOK;
  const int slot = a.meta[2 + bucket];
  const int off = a.meta[2 + kMetaB + bucket];
  const int cnt = a.meta[2 + 2 * kMetaB + bucket];
  const uint8_t *rec = a.slots + (long long)slot * a.rec_bytes;
  const int nb = a.nb, words = nb * 4;
  const int lr = lane & 15, lg = lane >> 4;
  const int row0 = tile * k6_rows(GLU) + rw * 32;
  const long long rowA = min(row0 + lr, a.rows - 1), rowB = min(row0 + 16 + lr, a.rows - 1);
  const uint4 *q = reinterpret_cast<const uint4 *>(rec + (m ? a.off_q1 : a.off_q0));
  const uint16_t *sc = reinterpret_cast<const uint16_t *>(rec + (m ? a.off_s1 : a.off_s0));
  const uint4 *qA = q + rowA * nb, *qB = q + rowB * nb;
  const uint16_t *sA = sc + rowA * nb, *sB = sc + rowB * nb;
  const int nch = (nb + K6_KC - 1) / K6_KC;
  const int ntok = min(K6_TOK, cnt - g0);
  if (tid < NT * 16) {
    const int p = a.bucket_pair[off + g0 + min(tid, ntok - 1)];
    L.tok[tid] = a.in_by_pair ? p : pair_row(a, p);
  }
  __syncthreads();

  // activation staging of chunk c: per token 16 words x (hi, lo) = 512
  // contiguous bytes in 32 units of 16 B; thread tid stages unit tid % 32 of
  // tokens tid / 32 (and + 16 for two tiles).  The loads of chunk c + 1 are
  // issued at the start of step c and stored to LDS at its end (they mostly hit
  // the L2: every row tile of the pass reads the same activations); one
  // register set instead of two leaves room for the scale windows.
  static_assert(NTH == 16 * 32, "one staging unit per thread and tile");
  const int sv = tid & 31, st = tid >> 5;
  const uint4 *bsrc0 = reinterpret_cast<const uint4 *>(a.xp + (long long)L.tok[st] * words * 8) +
                       (sv & 1);
  const uint4 *bsrc1 = NT == 2 ? reinterpret_cast<const uint4 *>(
                                     a.xp + (long long)L.tok[st + 16] * words * 8) +
                                     (sv & 1)
                               : bsrc0;
  auto load_b = [&](int c, uint4 &o0, uint4 &o1) __attribute__((always_inline)) {
    const int wd = min(c * 16 + (sv >> 1), words - 1);
    o0 = bsrc0[2 * wd];
    if constexpr (NT == 2) o1 = bsrc1[2 * wd];
  };
  auto store_b = [&](int buf, const uint4 &o0, const uint4 &o1) __attribute__((always_inline)) {
    L.B[buf][st][sv] = o0;
    if constexpr (NT == 2) L.B[buf][st + 16][sv] = o1;
  };
  // this lane's weight blocks of chunk c (one per row group) and, without scale
  // windows, their scales (group A, group B) as loaded: packing them here would
  // make the loads' wait immediate.  Unconditional loads (clamped block) keep
  // the code straight.
  auto load_a = [&](int c, uint4 &wA, uint4 &wB, uint2 &s) __attribute__((always_inline)) {
    const int bc = min(c * K6_KC + lg, nb - 1);
    wA = qA[bc];
    wB = qB[bc];
    if constexpr (!SW) s = make_uint2(sA[bc], sB[bc]);
  };
  // Scale windows (SW: nb is a multiple of 32, so every window is whole and the
  // chunk count a multiple of 8).  Half h of window k holds row group h's
  // scales of blocks 32k ... 32k + 31: lane (lr, lg) loads the 8 of row lr
  // from block 32k + 8 lg (each load reads 64 contiguous bytes of 16 rows).
  // Window k + 1 arrives during window k, both halves inside the same loop
  // trip: half 0 is loaded at chunk 8k and written at chunk 8k + 3, half 1
  // loaded at 8k + 3 and written at 8k + 6, to table buffer (k + 1) % 2, which
  // window k - 1 has left.  (A load in one trip consumed in the next made the
  // compiler's wait at the trip's start cover every load in flight, the next
  // chunk's weights too.)  Each chunk reads its 4 blocks' scales of row lr for
  // both groups (8 bytes each) from buffer (c / 8) % 2; window 0 is written
  // before the loop.
  const int nwin = nb >> 5;
  uint4 swin = make_uint4(0u, 0u, 0u, 0u);
  auto load_w = [&](int k, int h) __attribute__((always_inline)) {
    swin = *reinterpret_cast<const uint4 *>((h ? sB : sA) + min(k, nwin - 1) * 32 + 8 * lg);
  };
  auto store_w = [&](int buf, int h) __attribute__((always_inline)) {
    uint32_t *dst = &L.SC[buf][wave][h][lr][4 * lg];
    *reinterpret_cast<uint2 *>(dst) = make_uint2(swin.x, swin.y);
    *reinterpret_cast<uint2 *>(dst + 2) = make_uint2(swin.z, swin.w);
  };
  static_assert(K6_PD == 2, "the chunk ring is written out for two chunks");
  uint4 wa0, wa1, wb0, wb1;
  uint2 sa = make_uint2(0u, 0u), sb = sa;
  uint4 xa0, xa1;
  if constexpr (SW) {
    load_w(0, 0);
    store_w(0, 0);
    load_w(0, 1);
    store_w(0, 1);
  }
  load_b(0, xa0, xa1);
  load_a(0, wa0, wa1, sa);
  load_a(1, wb0, wb1, sb);
  store_b(0, xa0, xa1);
  __syncthreads();

  // accumulators [row group][token tile]
  floatx4 acc00 = {0.f, 0.f, 0.f, 0.f}, acc01 = acc00, acc10 = acc00, acc11 = acc00;

  // one K chunk: stage-load chunk c + 1, transpose, gather scales, refill the
  // ring slot with chunk c + 2, multiply, store chunk c + 1's activations,
  // barrier.  (wA, wB, s): this chunk's ring slot.
  auto step = [&](auto first, int c, uint4 &wA, uint4 &wB, uint2 &s)
      __attribute__((always_inline)) {
    // keep the scheduler from pulling the next step's transposes (and so the
    // wait for its weights) into this one: that would shorten the prefetch
    __builtin_amdgcn_sched_barrier(0);
    const int cur = c & 1;
    load_b(min(c + 1, nch - 1), xa0, xa1);
    const uint4 tA = transpose_rows(wA);
    const uint4 tB = transpose_rows(wB);
    // the chunk's scales: (sAl, sAh) = row lr of group A, blocks 0-1 / 2-3 as
    // binary16 pairs, (sBl, sBh) the same for group B
    uint32_t sAl, sAh, sBl, sBh;
    if constexpr (SW) {
      const int k = c >> 3;
      if constexpr (decltype(first)::value == 1) {  // chunk 8k
        load_w(k + 1, 0);
      } else if constexpr (decltype(first)::value == 2) {  // chunk 8k + 3
        store_w((k + 1) & 1, 0);
        load_w(k + 1, 1);
      } else if constexpr (decltype(first)::value == 3) {  // chunk 8k + 6
        store_w((k + 1) & 1, 1);
      }
      const uint2 pA = *reinterpret_cast<const uint2 *>(&L.SC[k & 1][wave][0][lr][2 * (c & 7)]);
      const uint2 pB = *reinterpret_cast<const uint2 *>(&L.SC[k & 1][wave][1][lr][2 * (c & 7)]);
      sAl = pA.x;
      sAh = pA.y;
      sBl = pB.x;
      sBh = pB.y;
    } else {
      // lane row g holds (group A, group B) of block g (zero past the row end,
      // also for every block of a chunk c >= nch): gather all four, then
      // regroup per row group
      const bool live = c * K6_KC + lg < nb;
      const uint4 sg = gather_rows(live ? (s.x | (s.y << 16)) : 0u);
      sAl = __builtin_amdgcn_perm(sg.y, sg.x, 0x05040100u);
      sAh = __builtin_amdgcn_perm(sg.w, sg.z, 0x05040100u);
      sBl = __builtin_amdgcn_perm(sg.y, sg.x, 0x07060302u);
      sBh = __builtin_amdgcn_perm(sg.w, sg.z, 0x07060302u);
    }
    // Loads past the last chunk re-read it (clamped) so that the code stays
    // straight and the waits exact.
    load_a(c + K6_PD, wA, wB, s);
#pragma unroll
    for (int b = 0; b < K6_KC; ++b) {
      const uint32_t awA = b == 0 ? tA.x : b == 1 ? tA.y : b == 2 ? tA.z : tA.w;
      const uint32_t awB = b == 0 ? tB.x : b == 1 ? tB.y : b == 2 ? tB.z : tB.w;
      const half2_t hA = __builtin_bit_cast(half2_t, b < 2 ? sAl : sAh);
      const half2_t hB = __builtin_bit_cast(half2_t, b < 2 ? sBl : sBh);
      const float dA = (float)hA[b & 1], dB = (float)hB[b & 1];
      const half8_t WA = decode_word_h(awA);
      const half8_t WB = decode_word_h(awB);
      const half8_t Xh0 = __builtin_bit_cast(half8_t, L.B[cur][lr][(b * 4 + lg) * 2]);
      const half8_t Xl0 = __builtin_bit_cast(half8_t, L.B[cur][lr][(b * 4 + lg) * 2 + 1]);
      const floatx4 z = {0.f, 0.f, 0.f, 0.f};
      floatx4 cA0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(Xh0, WA, z, 0, 0, 0);
      floatx4 cB0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(Xh0, WB, z, 0, 0, 0);
      cA0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(Xl0, WA, cA0, 0, 0, 0);
      cB0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(Xl0, WB, cB0, 0, 0, 0);
      if constexpr (NT == 2) {
        const half8_t Xh1 = __builtin_bit_cast(half8_t, L.B[cur][16 + lr][(b * 4 + lg) * 2]);
        const half8_t Xl1 =
            __builtin_bit_cast(half8_t, L.B[cur][16 + lr][(b * 4 + lg) * 2 + 1]);
        floatx4 cA1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(Xh1, WA, z, 0, 0, 0);
        floatx4 cB1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(Xh1, WB, z, 0, 0, 0);
        cA1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(Xl1, WA, cA1, 0, 0, 0);
        cB1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(Xl1, WB, cB1, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc01[i] = __builtin_fmaf(dA, cA1[i], acc01[i]);
          acc11[i] = __builtin_fmaf(dB, cB1[i], acc11[i]);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc00[i] = __builtin_fmaf(dA, cA0[i], acc00[i]);
        acc10[i] = __builtin_fmaf(dB, cB0[i], acc10[i]);
      }
    }
    store_b(cur ^ 1, xa0, xa1);  // buffer cur ^ 1 is idle until the barrier
    __syncthreads();
  };
  // steps in pairs (in fours with scale windows), unconditionally (straight
  // code keeps the load waits exact); for an odd chunk count the last step is a
  // chunk past the row end, whose blocks all have a zero scale
  const std::integral_constant<int, 0> nowin;
  const std::integral_constant<int, 1> win0;
  const std::integral_constant<int, 2> win3;
  const std::integral_constant<int, 3> win6;
  if constexpr (SW) {
    for (int c0 = 0; c0 < nch; c0 += 8) {
      step(win0, c0, wa0, wa1, sa);
      step(nowin, c0 + 1, wb0, wb1, sb);
      step(nowin, c0 + 2, wa0, wa1, sa);
      step(win3, c0 + 3, wb0, wb1, sb);
      step(nowin, c0 + 4, wa0, wa1, sa);
      step(nowin, c0 + 5, wb0, wb1, sb);
      step(win6, c0 + 6, wa0, wa1, sa);
      step(nowin, c0 + 7, wb0, wb1, sb);
    }
  } else {
    for (int c0 = 0; c0 < nch; c0 += K6_PD) {
      step(nowin, c0, wa0, wa1, sa);
      step(nowin, c0 + 1, wb0, wb1, sb);
    }
  }
  // C lane layout: token column t*16 + 4*lg + i, weight row row0 + 16*g + lr.
  // The GLU's gate waves hand their sums to the up waves of the same rows
  // through the (now idle) activation buffers.
  floatx4 *xg = reinterpret_cast<floatx4 *>(&L.B[0][0][0]) + rw * 4 * 64 + lane;
  if constexpr (GLU) {
    if (m == 0) {
      xg[0] = acc00;
      xg[64] = acc10;
      if constexpr (NT == 2) {
        xg[128] = acc01;
        xg[192] = acc11;
      }
    }
    __syncthreads();
    if (m == 0) return;
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) {
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const int r = row0 + 16 * g + lr;
      const floatx4 u = g == 0 ? (t == 0 ? acc00 : acc01) : (t == 0 ? acc10 : acc11);
      floatx4 gt = u;
      if constexpr (GLU) gt = xg[(t * 2 + g) * 64];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int col = t * 16 + 4 * lg + i;
        if (col < ntok && r < a.rows) {
          const int p = a.bucket_pair[off + g0 + col];
          const float s = a.xscale[L.tok[col]];
          const float v = GLU ? silu_f(gt[i] * s) * (u[i] * s) : u[i] * s;
          a.out[(long long)p * a.rows + r] = v;
        }
      }
    }
  }
}

hipError_t launch_mfma(const GemvArgs &a, bool glu, int n_items, hipStream_t s) {
  if (n_items <= 0) return hipSuccess;
  if (n_items > 65535) return hipErrorInvalidValue;
  const int rows_wg = k6_rows(glu);
  const dim3 grid((a.rows + rows_wg - 1) / rows_wg, n_items);
  if (glu)
    launch_k(q4_mfma_kernel<true>, grid, dim3(64 * K6_WAVES), 0, s, a);
  else
    launch_k(q4_mfma_kernel<false>, grid, dim3(64 * K6_WAVES), 0, s, a);
  return hipGetLastError();
}

// One wave per row: scale, binary16 hi/lo pairs in the decoder's order, word sums.
__global__ __launch_bounds__(64) void prep_pairs_kernel(const float *__restrict__ in, int rows, int K,
                                                        uint32_t *__restrict__ xp,
                                                        float *__restrict__ xscale) {
  const int r = blockIdx.x, lane = threadIdx.x;
  if (r >= rows) return;
  const float *xt = in + (long long)r * K;
  float m = 0.0f;
  for (int i = lane; i < K; i += 64) m = fmaxf(m, fabsf(xt[i]));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  const int ex2 = pow2_exponent(m);
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
  }
}

hipError_t launch_prep_pairs(const float *in, int rows, int K, uint32_t *xp, float *xscale,
                             hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  launch_k(prep_pairs_kernel, dim3(rows), dim3(64), 0, s, in, rows, K, xp, xscale);
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
  // two 16-B loads in flight per lane.  Measured on page-locked records: more
  // requests in flight (more loads per lane, or more workgroups per expert)
  // lowers the PCIe read rate; 32 workgroups x 256 lanes x 2 is near the best.
  // A load past the end is skipped, not clamped, so no host byte is read twice.
#pragma unroll 1
  for (long long i = b + threadIdx.x; i < end; i += 512) {
    const uint4 v0 = src[i];
    const bool k1 = i + 256 < end;
    uint4 v1;
    if (k1) v1 = src[i + 256];
    dst[i] = v0;
    if (k1) dst[i + 256] = v1;
  }
}

hipError_t launch_pull(const PullList &l, hipStream_t s) {
  if (l.n <= 0) return hipSuccess;
  launch_k(pull_kernel, dim3(l.n * l.per_expert), dim3(256), 0, s, l);
  return hipGetLastError();
}

// ============================================================== combine
// out[t] = sum_j [pair on GPU] w * y (j ascending) + shared + host part.  A pair
// is on the GPU when all_gpu, else when pair_slot[p] >= 0 (decode: the decode
// top-k kernel's table), else when view.slot[idx[p]] >= 0.  The loads of 8
// pairs are issued together; pairs off the GPU are skipped by select, since
// their y rows were never written.
__global__ __launch_bounds__(256) void combine_kernel(const float *__restrict__ y,
                                                      const float *__restrict__ w,
                                                      const int32_t *__restrict__ idx,
                                                      SlotView view, int all_gpu,
                                                      const int32_t *__restrict__ pair_slot,
                                                      int T, int k, int d, int n_shared,
                                                      const float *__restrict__ host_part,
                                                      float *__restrict__ out,
                                                      float *__restrict__ dbg_gpu) {
  const int t = blockIdx.y;
  const int i = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= d) return;
  // the host partial sits in page-locked host memory: its read crosses PCIe,
  // so it goes out first and its latency overlaps the expert outputs' reads
  float4 hv = make_float4(0.f, 0.f, 0.f, 0.f);
  if (host_part) hv = *reinterpret_cast<const float4 *>(host_part + (long long)t * d + i);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j0 = 0; j0 < k; j0 += 8) {
    float4 yv[8];
    float wv[8];
    bool on[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = min(j0 + u, k - 1);
      const long long p = (long long)t * k + j;
      bool g = j0 + u < k;
      if (g && !all_gpu) g = pair_slot ? pair_slot[p] >= 0 : view.slot[idx[p]] >= 0;
      on[u] = g;
      wv[u] = w[p];
      yv[u] = *reinterpret_cast<const float4 *>(y + p * d + i);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (on[u]) {
        acc.x += wv[u] * yv[u].x;
        acc.y += wv[u] * yv[u].y;
        acc.z += wv[u] * yv[u].z;
        acc.w += wv[u] * yv[u].w;
      }
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
    acc.x += hv.x;
    acc.y += hv.y;
    acc.z += hv.z;
    acc.w += hv.w;
  }
  *reinterpret_cast<float4 *>(out + (long long)t * d + i) = acc;
}

hipError_t launch_combine(const float *y, const float *w, const int32_t *idx,
                          const SlotView &view, int all_gpu, const int32_t *pair_slot, int T,
                          int k, int d, int n_shared, const float *host_part, float *out,
                          float *dbg_gpu, hipStream_t s) {
  const dim3 grid((d / 4 + 255) / 256, T);
  launch_k(combine_kernel, grid, dim3(256), 0, s, y, w, idx, view, all_gpu, pair_slot,
                     T, k, d, n_shared, host_part, out, dbg_gpu);
  return hipGetLastError();
}

// ============================================================== fixed scratch
// The workspace of moe_layer_forward_noalloc, for callers that may not
// allocate: one array per device, loaded with the code object and held until
// the process ends.  Every call on a device shares it.
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

hipError_t noalloc_scratch(void **ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex m;
  static void *addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> g(m);
  if (addr[dev] == nullptr) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

}  // namespace moe
