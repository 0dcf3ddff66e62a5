// Slot layout of one expert, shared by the host arena and the device slots.
//
// The interchange layout keeps each 32-weight block as 18 contiguous bytes
// (binary16 scale, then 16 bytes of nibbles), so blocks sit at 2-byte
// alignment.  The slot layout separates the two parts so that GPU lanes read
// nibbles with aligned 16-byte loads and scales as a contiguous array:
//
//   [gate nibbles][up nibbles][down nibbles][gate scales][up scales][down scales]
//
// nibbles: rows x blocks x 16 bytes (byte j: element j low, element j+16 high);
// scales: rows x blocks binary16; each section starts on a 256-byte boundary and
// the record is padded to 4096 bytes.  One expert is one contiguous record, so a
// slot fill is a single host->device copy, as the pages' caches copy whole
// experts into slots.
#pragma once
#include <cstddef>
#include <cstdint>
#include <cstring>

namespace moe {

struct RecordLayout {
  int64_t d = 0, f = 0;
  int64_t nb_gu = 0;  // blocks per gate/up row (d / 32)
  int64_t nb_dn = 0;  // blocks per down row (f / 32)
  int64_t off_gq = 0, off_uq = 0, off_dq = 0;
  int64_t off_gs = 0, off_us = 0, off_ds = 0;
  int64_t bytes = 0;  // record stride
  int64_t interchange_bytes = 0;

  static int64_t align(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

  static RecordLayout make(int64_t d_model, int64_t d_ff) {
    RecordLayout L;
    L.d = d_model;
    L.f = d_ff;
    L.nb_gu = d_model / 32;
    L.nb_dn = d_ff / 32;
    const int64_t gq = d_ff * L.nb_gu * 16, dq = d_model * L.nb_dn * 16;
    const int64_t gs = d_ff * L.nb_gu * 2, ds = d_model * L.nb_dn * 2;
    int64_t o = 0;
    L.off_gq = o; o = align(o + gq, 256);
    L.off_uq = o; o = align(o + gq, 256);
    L.off_dq = o; o = align(o + dq, 256);
    L.off_gs = o; o = align(o + gs, 256);
    L.off_us = o; o = align(o + gs, 256);
    L.off_ds = o; o = align(o + ds, 256);
    L.bytes = align(o, 4096);
    L.interchange_bytes = 3 * d_model * d_ff / 32 * 18;
    return L;
  }
};

// Splits one matrix of 18-byte blocks into nibble and scale sections.
inline void repack_matrix(const uint8_t *src, int64_t n_blocks, uint8_t *q, uint8_t *s) {
  for (int64_t b = 0; b < n_blocks; ++b) {
    const uint8_t *blk = src + b * 18;
    s[2 * b] = blk[0];
    s[2 * b + 1] = blk[1];
    std::memcpy(q + 16 * b, blk + 2, 16);
  }
}

// One expert: interchange bytes -> slot record (padding zeroed).
inline void repack_expert(const uint8_t *src, const RecordLayout &L, uint8_t *dst) {
  std::memset(dst, 0, (size_t)L.bytes);
  const int64_t n_gu = L.f * L.nb_gu, n_dn = L.d * L.nb_dn;
  repack_matrix(src, n_gu, dst + L.off_gq, dst + L.off_gs);
  repack_matrix(src + n_gu * 18, n_gu, dst + L.off_uq, dst + L.off_us);
  repack_matrix(src + 2 * n_gu * 18, n_dn, dst + L.off_dq, dst + L.off_ds);
}

}  // namespace moe
