// Decode path decision, GEMV shapes and the per-call device workspace (plain
// C++; see workspace.hpp).
#include "workspace.hpp"

#include <algorithm>
#include <cmath>
#include <vector>

namespace moe {

// Shapes measured on MI355X for one token per bucket over the decode shapes
// d x f = 6144 x 2048 and 2816 x 704: gate/up rows of >= 128 blocks run best
// with 16 lanes per row and 2 rows per lane, rows of 32-127 blocks with 8 lanes
// and 1 row per lane, K split over the 4 waves; down rows with 8 lanes per row,
// 4 rows per lane and K split over the 4 waves (at 64 blocks per row 4% faster
// than 16 lanes with whole K per wave: the four waves read a row's K range
// together).  Rows of fewer than 32 gate/up blocks keep K in one wave.
GemvShape choose_gemv(bool glu, int nb, int tokens) {
  GemvShape sh{};
  sh.TT = tokens <= 1 ? 1 : (tokens <= 2 ? 2 : 4);
  if (glu) {
    sh.R = 2;
    if (nb >= 128) {
      sh.G = 16;
      sh.KS = 4;
    } else if (nb >= 32) {
      sh.G = 8;
      sh.KS = 4;
      sh.R = 1;
    } else {
      sh.G = 8;
      sh.KS = 1;
    }
  } else {
    sh.R = 4;
    sh.G = 8;
    sh.KS = 4;
  }
  sh.NW = 4;
  sh.rows_wg = (sh.NW / sh.KS) * (64 / sh.G) * sh.R;
  return sh;
}

size_t gemv_lds_bytes(bool glu, int nb, int tokens) {
  const GemvShape sh = choose_gemv(glu, nb, tokens);
  const size_t row_scales = ((size_t)sh.rows_wg * nb * 2 + 15) / 16 * 16;
  if (glu) return (size_t)sh.TT * nb * 64 + (size_t)sh.TT * xs_units(nb) * 16 + 2 * row_scales;
  return (size_t)sh.TT * nb * 64 + ((size_t)sh.TT * nb + 3) / 4 * 16 + row_scales;
}


bool decode_path(const WsParams &p) {
  if (p.T < 1 || p.T > kDecodeMaxTokens) return false;
  if ((int64_t)p.T * (p.k + p.n_shared) > kDecodeMaxPairs) return false;
  return gemv_lds_bytes(true, p.d / 32, p.T) <= kDecodeLdsBudget &&
         gemv_lds_bytes(false, p.f / 32, p.T) <= kDecodeLdsBudget;
}

namespace {

size_t up(size_t v) { return (v + kWsAlign - 1) / kWsAlign * kWsAlign; }

// Places a region of `bytes` at the running offset.
WsRegion take(size_t &o, size_t bytes) {
  WsRegion r;
  r.off = o;
  r.bytes = bytes;
  o = up(o + bytes);
  return r;
}

}  // namespace

WsLayout ws_layout(const WsParams &p) {
  WsLayout L;
  const size_t T = (size_t)p.T, E = (size_t)p.E, k = (size_t)p.k, d = (size_t)p.d,
               f = (size_t)p.f;
  L.decode = decode_path(p);
  L.pairs = p.T * p.k + p.T * p.n_shared;
  const size_t P = (size_t)L.pairs;
  size_t o = 0;
  L.z = take(o, T * E * 4);
  L.idx = take(o, T * k * 4);
  L.w = take(o, T * k * 4);
  L.h = take(o, P * f * 4);
  L.y = take(o, P * d * 4);
  if (L.decode) {
    L.xq = take(o, T * d * 2);  // [T][d/32 blocks][4 words] x 16 bytes
    L.xs = take(o, T * (size_t)xs_units(p.d / 32) * 16);
    // at most one bucket per pair (the decode path has at most kDecodeMaxPairs)
    L.buckets = take(o, (1 + P * kBucketInts) * 4);
    L.pair_slot = take(o, T * k * 4);
  } else {
    L.meta = take(o, (size_t)kMetaInts * 4);
    L.bucket_pair = take(o, P * 4);
    L.items = take(o, ((size_t)gemm_items_bound(kMetaB, (int)P) + 1) * 4);
    L.xp = take(o, T * (d / 8) * 8 * 4);  // [T][d/8 words][hi, lo x 4 pairs]
    L.xscale = take(o, T * 4);
    L.hp = take(o, P * (f / 8) * 8 * 4);
    L.hscale = take(o, P * 4);
  }
  L.total = o;
  return L;
}

const char *ws_check(const WsLayout &L, const WsParams &p) {
  // What each launch of the call reads or writes, restated from the kernels'
  // contracts (element counts x element bytes).
  struct Need {
    const char *name;
    const WsRegion *r;
    double bytes;
  };
  const double T = p.T, E = p.E, k = p.k, d = p.d, f = p.f;
  const double P = T * k + T * p.n_shared;
  const bool dec = decode_path(p);
  if (dec != L.decode || (int)P != L.pairs) return "path";
  Need common[] = {
      {"z", &L.z, T * E * 4},     // router logits [T][E]
      {"idx", &L.idx, T * k * 4},  // top-k ids [T][k]
      {"w", &L.w, T * k * 4},      // gating weights [T][k]
      {"h", &L.h, P * f * 4},      // gate/up output by pair [P][f]
      {"y", &L.y, P * d * 4},      // down output by pair [P][d]
  };
  Need decode[] = {
      {"xq", &L.xq, T * (d / 32) * 4 * 16},  // digit planes: 4 words x 16 B per block
      {"xs", &L.xs, T * xs_units(p.d / 32) * 4 * 4},  // block scales, padded rows
      {"buckets", &L.buckets, (1.0 + P * kBucketInts) * 4},  // count + one entry per bucket
      {"pair_slot", &L.pair_slot, T * k * 4},
  };
  Need gemm[] = {
      {"meta", &L.meta, (2.0 + 3.0 * kMetaB) * 4},
      {"bucket_pair", &L.bucket_pair, P * 4},
      // the remap kernel lists at most one item per bucket (<= kMetaB slot ids)
      // plus one per started 32-token pass
      {"items", &L.items, (1.0 + kMetaB + std::ceil(P / kGemmTokens)) * 4},
      {"xp", &L.xp, T * d * 4},        // hi/lo binary16 pairs: 4 bytes per element
      {"xscale", &L.xscale, T * 4},
      {"hp", &L.hp, P * f * 4},
      {"hscale", &L.hscale, P * 4},
  };
  std::vector<const Need *> used;
  for (const Need &n : common) used.push_back(&n);
  if (dec)
    for (const Need &n : decode) used.push_back(&n);
  else
    for (const Need &n : gemm) used.push_back(&n);
  if (dec && P > kDecodeMaxPairs) return "pairs";
  for (const Need *n : used) {
    if ((double)n->r->bytes < n->bytes) return n->name;
    if (n->r->off % kWsAlign) return n->name;
    if (n->r->off + n->r->bytes > L.total) return n->name;
  }
  for (size_t i = 0; i < used.size(); ++i)
    for (size_t j = i + 1; j < used.size(); ++j) {
      const WsRegion &a = *used[i]->r, &b = *used[j]->r;
      if (a.bytes && b.bytes && a.off < b.off + b.bytes && b.off < a.off + a.bytes)
        return used[j]->name;
    }
  return nullptr;
}

}  // namespace moe
