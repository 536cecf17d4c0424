/* synth_rng.h - counter-based generator for the seeded synthetic workloads.
 *
 * Input generation only: nothing here belongs to the sparse-FFN method.  The
 * same header is compiled for the host (gcc, C99) and for the device (hipcc),
 * and every function uses only integer arithmetic, one IEEE multiply and
 * IEEE round-to-nearest-even conversions, so a given (seed, tag, layer, row,
 * col) yields the same stored bits on both sides.
 *
 * Hash: the SplitMix64 output function (Steele, Lea and Flood, "Fast
 * splittable pseudorandom number generators", OOPSLA 2014) applied to a
 * counter built from the coordinates.
 *
 * Values: sum of four 16-bit uniforms taken from one 64-bit hash (the
 * Irwin-Hall distribution with n = 4), centred and scaled to unit variance.
 * It is an approximately Gaussian, bounded (|v| <= 2*sqrt(3)) distribution
 * that is reproducible bit for bit without transcendental functions.
 */
#ifndef SYNTH_RNG_H
#define SYNTH_RNG_H
#include <stdint.h>

#if defined(__HIPCC__)
#define SX_FN __host__ __device__ static inline
#else
#define SX_FN static inline
#endif

SX_FN uint64_t sx_mix64(uint64_t z) {
  z += 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

/* Per-row stream key: hash of (seed, tag, layer, row).  The element hash is
 * sx_mix64(rowkey ^ col). */
SX_FN uint64_t sx_rowkey(uint64_t seed, uint32_t tag, uint32_t layer, uint64_t row) {
  uint64_t h = sx_mix64(seed ^ (((uint64_t)tag << 40) | ((uint64_t)layer << 8)));
  return sx_mix64(h ^ (row * 0xD1B54A32D192ED03ull));
}
SX_FN uint64_t sx_hash(uint64_t rowkey, uint64_t col) { return sx_mix64(rowkey ^ (col * 0xA24BAED4963EE407ull)); }

/* Irwin-Hall(4) integer: sum of the four 16-bit fields minus 131070, i.e.
 * 65536 * (sum of four uniforms on (0,1) centred at 2).  Range [-131070, 131070]. */
SX_FN int32_t sx_ih4(uint64_t h) {
  int32_t s = (int32_t)(h & 0xFFFFu) + (int32_t)((h >> 16) & 0xFFFFu) +
              (int32_t)((h >> 32) & 0xFFFFu) + (int32_t)(h >> 48);
  return s - 131070;
}
/* Scale that maps sx_ih4 to a value of standard deviation sigma:
 * sqrt(3) * sigma / 65536 (the variance of a sum of four uniforms is 1/3).
 * Callers compute it once on the host and pass the same double to both sides. */

/* Uniform on (0,1) from the top 53 bits. */
SX_FN double sx_u01(uint64_t h) { return ((double)(h >> 11) + 0.5) * (1.0 / 9007199254740992.0); }

/* IEEE binary16 bits of a double, round to nearest even, overflow to inf. */
SX_FN uint16_t sx_f64_to_f16(double v) {
  uint16_t sign = 0;
  if (v < 0 || (v == 0 && 1.0 / v < 0)) { sign = 0x8000u; v = -v; }
  if (v != v) return (uint16_t)(sign | 0x7E00u);
  if (v >= 65520.0) return (uint16_t)(sign | 0x7C00u);
  if (v < 5.9604644775390625e-08 * 0.5) {        /* below half the smallest subnormal */
    return sign;                                  /* (exactly half rounds to even = 0) */
  }
  /* find exponent e with 2^e <= v < 2^(e+1) */
  int e = 0;
  double m = v;
  while (m >= 2.0) { m *= 0.5; ++e; }
  while (m < 1.0) { m *= 2.0; --e; }
  if (e < -14) {
    /* subnormal: units of 2^-24 */
    double q = v * 16777216.0;                    /* exact (power of two scaling) */
    double fl = (double)(int64_t)q;               /* floor, q >= 0 */
    double rem = q - fl;                          /* exact */
    int64_t n = (int64_t)fl;
    if (rem > 0.5 || (rem == 0.5 && (n & 1))) ++n;
    return (uint16_t)(sign | (uint16_t)n);        /* n == 1024 gives the smallest normal */
  }
  /* normal: 10 fraction bits */
  double q = m * 1024.0;                          /* in [1024, 2048), exact */
  double fl = (double)(int64_t)q;
  double rem = q - fl;
  int64_t n = (int64_t)fl;
  if (rem > 0.5 || (rem == 0.5 && (n & 1))) ++n;
  if (n == 2048) { n = 1024; ++e; }
  if (e > 15) return (uint16_t)(sign | 0x7C00u);
  return (uint16_t)(sign | (uint16_t)((e + 15) << 10) | (uint16_t)(n - 1024));
}

/* Widen binary16 bits to double (exact). */
SX_FN double sx_f16_to_f64(uint16_t h) {
  int e = (h >> 10) & 0x1F, f = h & 0x3FF;
  double s = (h & 0x8000u) ? -1.0 : 1.0;
  if (e == 0) return s * (double)f * 5.9604644775390625e-08;        /* f * 2^-24 */
  if (e == 31) return f ? (0.0 / 0.0) : s * (1.0 / 0.0);
  double m = 1.0 + (double)f / 1024.0;
  double p = 1.0;
  int k = e - 15;
  while (k > 0) { p *= 2.0; --k; }
  while (k < 0) { p *= 0.5; ++k; }
  return s * m * p;
}

/* Tags: one independent stream per synthetic tensor. */
enum {
  SX_TAG_P1 = 1, SX_TAG_P2 = 2, SX_TAG_W1 = 3, SX_TAG_W2 = 4, SX_TAG_WUP = 5,
  SX_TAG_X = 6, SX_TAG_YC = 7, SX_TAG_PERM = 8, SX_TAG_PROF = 9, SX_TAG_LAYER = 10
};

/* Storage formats written by the fill routines. */
enum { SX_F32 = 0, SX_F16 = 1, SX_I4G128 = 2 };

#endif
