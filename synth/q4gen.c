/*
 * Seeded synthetic expert weights in the Q4_0 interchange layout.
 *
 * This file generates INPUT DATA only.  It is shared by the oracle side and the
 * library side as the one source of synthetic weights; it implements none of
 * the layer's arithmetic (no dequantisation, no matrix products, no routing).
 *
 * Weight values: w ~ N(0, sigma^2), drawn per element from a counter-based
 * stream (splitmix64 finaliser over a per-matrix key and the element index),
 * turned into a normal deviate through a 65536-entry inverse-CDF table that the
 * caller supplies (its entries are Phi^-1((u + 0.5) / 65536)).
 *
 * Quantisation into 18-byte blocks of 32 weights (the GGML Q4_0 block the
 * calculator page counts at 18/32 bytes per parameter, "Memory placement"):
 *   m  = the element of largest |x| in the block (first one on a tie)
 *   d  = fp16 round-to-nearest-even of m / -8
 *   q  = clamp(floor(x / d + 8.5), 0, 15)      (q = 8 when d == 0)
 *   bytes 0-1: d little-endian; byte 2 + j: (q[j] & 15) | (q[j + 16] << 4)
 *
 * Interchange layout of one expert: gate rows [f][d], up rows [f][d], down
 * rows [d][f]; every row quantised along its reduction dimension, blocks in
 * K order, no padding.  Experts follow one another; layers follow one another.
 */
#include <stdint.h>
#include <string.h>
#include <math.h>
#include <pthread.h>

static inline uint64_t mix64(uint64_t z) {
  z += 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

/* float -> IEEE binary16 bits, round to nearest even (overflow -> inf). */
static uint16_t f32_to_f16_rne(float v) {
  uint32_t x;
  memcpy(&x, &v, 4);
  uint32_t sign = (x >> 16) & 0x8000u;
  uint32_t ax = x & 0x7FFFFFFFu;
  if (ax >= 0x7F800000u) return (uint16_t)(sign | (ax > 0x7F800000u ? 0x7E00u : 0x7C00u));
  int32_t exp = (int32_t)(ax >> 23) - 127 + 15;
  uint32_t mant = ax & 0x7FFFFFu;
  if (exp >= 31) return (uint16_t)(sign | 0x7C00u);
  if (exp <= 0) {
    if (exp < -10) return (uint16_t)sign;
    mant |= 0x800000u;
    uint32_t shift = (uint32_t)(14 - exp);
    uint32_t half = mant >> shift;
    uint32_t rem = mant & ((1u << shift) - 1u);
    uint32_t mid = 1u << (shift - 1u);
    if (rem > mid || (rem == mid && (half & 1u))) half++;
    return (uint16_t)(sign | half);
  }
  uint32_t h = ((uint32_t)exp << 10) | (mant >> 13);
  uint32_t rem = mant & 0x1FFFu;
  if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) h++;
  return (uint16_t)(sign | h);
}

static float f16_bits_to_f32(uint16_t h) {
  uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
  uint32_t exp = (h >> 10) & 0x1Fu, mant = h & 0x3FFu, x;
  if (exp == 0) {
    if (mant == 0) x = sign;
    else {
      exp = 127 - 15 + 1;
      while (!(mant & 0x400u)) { mant <<= 1; exp--; }
      x = sign | (exp << 23) | ((mant & 0x3FFu) << 13);
    }
  } else if (exp == 31) x = sign | 0x7F800000u | (mant << 13);
  else x = sign | ((exp - 15 + 127) << 23) | (mant << 13);
  float f;
  memcpy(&f, &x, 4);
  return f;
}

/* One matrix [rows][cols] (cols % 32 == 0) -> rows * cols/32 blocks at dst
 * (when dst != NULL) and/or the unquantised values at vals (when != NULL). */
static void gen_matrix(uint8_t *dst, float *vals, uint64_t key, int64_t rows, int64_t cols,
                       float sigma, const float *table) {
  float x[32];
  const int64_t nb = cols / 32;
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t b = 0; b < nb; ++b) {
      const uint64_t base = (uint64_t)(r * cols + b * 32);
      for (int i = 0; i < 32; i += 4) {
        uint64_t u = mix64(key ^ ((base + (uint64_t)i) >> 2) * 0xD1B54A32D192ED03ull);
        x[i + 0] = sigma * table[(u >> 0) & 0xFFFF];
        x[i + 1] = sigma * table[(u >> 16) & 0xFFFF];
        x[i + 2] = sigma * table[(u >> 32) & 0xFFFF];
        x[i + 3] = sigma * table[(u >> 48) & 0xFFFF];
      }
      if (vals) memcpy(vals + base, x, sizeof(x));
      if (!dst) continue;
      float amax = 0.0f, m = 0.0f;
      for (int i = 0; i < 32; ++i) {
        float a = fabsf(x[i]);
        if (a > amax) { amax = a; m = x[i]; }
      }
      uint16_t dh = f32_to_f16_rne(m / -8.0f);
      float d = f16_bits_to_f32(dh);
      uint8_t q[32];
      for (int i = 0; i < 32; ++i) {
        int qi = 8;
        if (d != 0.0f) {
          float t = floorf(x[i] / d + 8.5f);
          qi = t < 0.0f ? 0 : (t > 15.0f ? 15 : (int)t);
        }
        q[i] = (uint8_t)qi;
      }
      uint8_t *blk = dst + (r * nb + b) * 18;
      blk[0] = (uint8_t)(dh & 0xFF);
      blk[1] = (uint8_t)(dh >> 8);
      for (int j = 0; j < 16; ++j) blk[2 + j] = (uint8_t)((q[j] & 15) | (q[j + 16] << 4));
    }
  }
}

typedef struct {
  uint8_t *dst;
  float *vals;
  uint64_t seed;
  int64_t e0, e1, d, f;
  float sigma;
  const float *table;
} job_t;

static void *run_job(void *p) {
  job_t *j = (job_t *)p;
  const int64_t mat_gu = j->f * (j->d / 32) * 18;
  const int64_t mat_dn = j->d * (j->f / 32) * 18;
  const int64_t eb = 2 * mat_gu + mat_dn;
  const int64_t n_gu = j->f * j->d;
  for (int64_t e = j->e0; e < j->e1; ++e) {
    uint8_t *ex = j->dst ? j->dst + (e - j->e0) * eb : 0;
    float *vx = j->vals ? j->vals + (e - j->e0) * 3 * n_gu : 0;
    uint64_t ke = mix64(j->seed ^ mix64((uint64_t)e + 0x1234567ull));
    gen_matrix(ex, vx, mix64(ke ^ 1), j->f, j->d, j->sigma, j->table);
    gen_matrix(ex ? ex + mat_gu : 0, vx ? vx + n_gu : 0, mix64(ke ^ 2), j->f, j->d, j->sigma, j->table);
    gen_matrix(ex ? ex + 2 * mat_gu : 0, vx ? vx + 2 * n_gu : 0, mix64(ke ^ 3), j->d, j->f, j->sigma,
               j->table);
  }
  return 0;
}

/*
 * Writes experts [e_begin, e_end) of the stream keyed by `seed` into dst (which
 * receives (e_end - e_begin) * eb bytes), split over n_threads threads.
 * Returns 0, or -1 on a bad argument.
 */
static int run_all(uint8_t *dst, float *vals, uint64_t seed, int64_t e_begin, int64_t e_end,
                   int64_t d, int64_t f, float sigma, const float *table, int n_threads) {
  if ((!dst && !vals) || !table || d <= 0 || f <= 0 || d % 32 || f % 32 || e_end < e_begin) return -1;
  if (n_threads < 1) n_threads = 1;
  if (n_threads > 256) n_threads = 256;
  const int64_t n = e_end - e_begin;
  if (n == 0) return 0;
  if (n_threads > n) n_threads = (int)n;
  const int64_t eb = 3 * d * f / 32 * 18;
  pthread_t th[256];
  job_t jobs[256];
  int64_t per = n / n_threads, extra = n % n_threads, e = e_begin;
  for (int t = 0; t < n_threads; ++t) {
    int64_t c = per + (t < extra ? 1 : 0);
    jobs[t].dst = dst ? dst + (e - e_begin) * eb : 0;
    jobs[t].vals = vals ? vals + (e - e_begin) * 3 * d * f : 0;
    jobs[t].seed = seed;
    jobs[t].e0 = e;
    jobs[t].e1 = e + c;
    jobs[t].d = d;
    jobs[t].f = f;
    jobs[t].sigma = sigma;
    jobs[t].table = table;
    e += c;
  }
  int started = 0;
  for (int t = 1; t < n_threads; ++t) {
    if (pthread_create(&th[t], 0, run_job, &jobs[t]) != 0) break;
    started = t;
  }
  run_job(&jobs[0]);
  for (int t = started + 1; t < n_threads; ++t) run_job(&jobs[t]);
  for (int t = 1; t <= started; ++t) pthread_join(th[t], 0);
  return 0;
}

int q4gen_experts(uint8_t *dst, uint64_t seed, int64_t e_begin, int64_t e_end,
                  int64_t d, int64_t f, float sigma, const float *table, int n_threads) {
  if (!dst) return -1;
  return run_all(dst, 0, seed, e_begin, e_end, d, f, sigma, table, n_threads);
}

/* The unquantised values behind q4gen_experts: per expert gate [f][d], up
 * [f][d], down [d][f] as float32 (3*d*f floats per expert). */
int q4gen_values(float *vals, uint64_t seed, int64_t e_begin, int64_t e_end,
                 int64_t d, int64_t f, float sigma, const float *table, int n_threads) {
  if (!vals) return -1;
  return run_all(0, vals, seed, e_begin, e_end, d, f, sigma, table, n_threads);
}
