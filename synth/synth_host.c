/* synth_host.c - host side of the seeded synthetic-workload generator.
 *
 * Input generation only (weights, inputs, permutations, simulated profiling
 * counts).  Contains none of the sparse-FFN method's arithmetic.  The element
 * values come from synth_rng.h, which the device generator compiles too, so a
 * row generated here has the same bits as the row generated on the GPU.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include "synth_rng.h"

/* One row of `cols` synthetic values v = ih4 * k, stored as dtype.
 * f32: float; f16: binary16 bits; i4g128: symmetric int4, one fp16 scale per
 * 128 consecutive elements, scale = f16(max|v| / 7), q = clamp(rne(v/scale)),
 * two elements per byte with the even element in the low nibble. */
static void fill_one_row(void* out_row, uint16_t* scales_row, int dtype, uint64_t rk, int64_t cols, double k) {
  if (dtype == SX_F32) {
    float* o = (float*)out_row;
    for (int64_t c = 0; c < cols; ++c) o[c] = (float)((double)sx_ih4(sx_hash(rk, (uint64_t)c)) * k);
  } else if (dtype == SX_F16) {
    uint16_t* o = (uint16_t*)out_row;
    for (int64_t c = 0; c < cols; ++c) o[c] = sx_f64_to_f16((double)sx_ih4(sx_hash(rk, (uint64_t)c)) * k);
  } else {
    uint8_t* o = (uint8_t*)out_row;
    double v[128];
    for (int64_t g = 0; g < cols / 128; ++g) {
      double mx = 0.0;
      for (int j = 0; j < 128; ++j) {
        v[j] = (double)sx_ih4(sx_hash(rk, (uint64_t)(g * 128 + j))) * k;
        double a = v[j] < 0 ? -v[j] : v[j];
        if (a > mx) mx = a;
      }
      uint16_t s16 = sx_f64_to_f16(mx / 7.0);
      double s = sx_f16_to_f64(s16);
      scales_row[g] = s16;
      for (int j = 0; j < 128; j += 2) {
        int q[2];
        for (int t = 0; t < 2; ++t) {
          double r = s > 0 ? rint(v[j + t] / s) : 0.0;
          if (r > 7) r = 7;
          if (r < -8) r = -8;
          q[t] = (int)r;
        }
        o[(g * 128 + j) / 2] = (uint8_t)((q[0] & 0xF) | ((q[1] & 0xF) << 4));
      }
    }
  }
}

static size_t row_bytes(int dtype, int64_t cols) {
  return dtype == SX_F32 ? (size_t)cols * 4 : dtype == SX_F16 ? (size_t)cols * 2 : (size_t)cols / 2;
}

/* Fill nrows rows.  Row r takes global id row_ids[r] if row_ids != NULL, else
 * row0 + r.  Scales (i4g128 only) are [nrows x cols/128]. */
void sx_fill_rows(void* out, uint16_t* scales, int dtype, uint64_t seed, uint32_t tag, uint32_t layer,
                  const int32_t* row_ids, int64_t row0, int64_t nrows, int64_t cols, double k) {
  size_t rb = row_bytes(dtype, cols);
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < nrows; ++r) {
    int64_t id = row_ids ? (int64_t)row_ids[r] : row0 + r;
    uint64_t rk = sx_rowkey(seed, tag, layer, (uint64_t)id);
    fill_one_row((char*)out + (size_t)r * rb, scales ? scales + (size_t)r * (cols / 128) : NULL, dtype, rk, cols, k);
  }
}

/* Per-row sum and sum of squares of the STORED values (f32 or f16) of rows
 * row0..row0+nrows-1, without materialising the matrix. */
void sx_row_stats(double* sum, double* sumsq, int dtype, uint64_t seed, uint32_t tag, uint32_t layer,
                  int64_t row0, int64_t nrows, int64_t cols, double k) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < nrows; ++r) {
    uint64_t rk = sx_rowkey(seed, tag, layer, (uint64_t)(row0 + r));
    double s = 0, s2 = 0;
    for (int64_t c = 0; c < cols; ++c) {
      double v = (double)sx_ih4(sx_hash(rk, (uint64_t)c)) * k;
      double w = dtype == SX_F32 ? (double)(float)v : sx_f16_to_f64(sx_f64_to_f16(v));
      s += w;
      s2 += w * w;
    }
    sum[r] = s;
    sumsq[r] = s2;
  }
}

/* Seeded Fisher-Yates permutation of 0..n-1 (index j drawn as hash mod (i+1)). */
void sx_perm(uint64_t seed, uint32_t tag, uint32_t layer, int32_t n, int32_t* out) {
  for (int32_t i = 0; i < n; ++i) out[i] = i;
  uint64_t rk = sx_rowkey(seed, tag, layer, 0);
  for (int32_t i = n - 1; i > 0; --i) {
    uint64_t h = sx_hash(rk, (uint64_t)i);
    int32_t j = (int32_t)(h % (uint64_t)(i + 1));
    int32_t t = out[i]; out[i] = out[j]; out[j] = t;
  }
}

/* Simulated offline profiling: for each neuron i, count over ntok tokens the
 * events u(seed, PROF, layer, token, i) < p[i], i.e. a Binomial(ntok, p_i)
 * draw, which is the distribution of the number of profiling tokens on which
 * a neuron with activation probability p_i fires. */
void sx_profile_counts(uint64_t seed, uint32_t layer, int32_t n, const double* p, int32_t ntok, int32_t* counts) {
#pragma omp parallel for schedule(static)
  for (int32_t i = 0; i < n; ++i) {
    int32_t c = 0;
    for (int32_t t = 0; t < ntok; ++t) {
      uint64_t rk = sx_rowkey(seed, SX_TAG_PROF, layer, (uint64_t)t);
      if (sx_u01(sx_hash(rk, (uint64_t)i)) < p[i]) ++c;
    }
    counts[i] = c;
  }
}

/* Simulated activation events for the generator's own self-check: out[t*n+i]
 * = 1 if u(seed, PROF, layer, token, i) < p[i]. */
uint16_t sx_f16_bits(double v) { return sx_f64_to_f16(v); }
double sx_f16_value(uint16_t h) { return sx_f16_to_f64(h); }
int32_t sx_ih4_at(uint64_t seed, uint32_t tag, uint32_t layer, uint64_t row, uint64_t col) {
  return sx_ih4(sx_hash(sx_rowkey(seed, tag, layer, row), col));
}
