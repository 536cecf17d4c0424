/* oracle.c - plain, slow CPU oracle for the neuron-aware sparse FFN.
 * TEST INFRASTRUCTURE ONLY (see oracle.h for the sources it follows). */
#include "oracle.h"
#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static int g_threads = 0;
void or_set_threads(int n) { g_threads = n; }
int or_get_threads(void) {
#ifdef _OPENMP
  return g_threads > 0 ? g_threads : omp_get_max_threads();
#else
  return 1;
#endif
}
#define OR_NT or_get_threads()

/* IEEE 754 binary16: sign, 5-bit exponent (bias 15), 10-bit fraction;
 * exponent 0 encodes subnormals f * 2^-24. */
double or_f16_to_double(uint16_t h) {
  int sign = (h >> 15) & 1, e = (h >> 10) & 31, f = h & 1023;
  double v;
  if (e == 0) v = ldexp((double)f, -24);
  else if (e == 31) v = f ? NAN : INFINITY;
  else v = ldexp(1024.0 + (double)f, e - 25);
  return sign ? -v : v;
}

/* int4 group 128: byte (row*cols + col)/2, even column in the low nibble,
 * two's-complement nibble q in [-8, 7], value q * scale[row, col/128]. */
double or_mat_at(or_mat m, int64_t row, int64_t col) {
  switch (m.dtype) {
    case OR_F32: return (double)((const float*)m.data)[row * m.cols + col];
    case OR_F16: return or_f16_to_double(((const uint16_t*)m.data)[row * m.cols + col]);
    default: {
      uint8_t byte = ((const uint8_t*)m.data)[(row * m.cols + col) / 2];
      int nib = (col & 1) ? (byte >> 4) : (byte & 15);
      int q = nib >= 8 ? nib - 16 : nib;
      return (double)q * or_f16_to_double(m.scales[row * (m.cols / 128) + col / 128]);
    }
  }
}

double or_vec_at(or_vec v, int64_t i) {
  if (!v.data) return 0.0;
  return v.dtype == OR_F32 ? (double)((const float*)v.data)[i] : or_f16_to_double(((const uint16_t*)v.data)[i]);
}

static double dot_row(or_mat m, int64_t row, const float* x, int64_t n) {
  double s = 0.0;
  for (int64_t k = 0; k < n; ++k) s += or_mat_at(m, row, k) * (double)x[k];
  return s;
}

void or_predict(int B, int d, int H, int N, const float* x, or_mat P1, or_vec c1,
                or_mat P2, or_vec c2, double* h_out, double* logits) {
  double* h = (double*)malloc(sizeof(double) * (size_t)B * H);
#pragma omp parallel for collapse(2) schedule(static) num_threads(OR_NT)
  for (int b = 0; b < B; ++b)
    for (int m = 0; m < H; ++m) {
      double z = dot_row(P1, m, x + (size_t)b * d, d) + or_vec_at(c1, m);
      h[(size_t)b * H + m] = z > 0.0 ? z : 0.0;
    }
#pragma omp parallel for collapse(2) schedule(static) num_threads(OR_NT)
  for (int b = 0; b < B; ++b)
    for (int i = 0; i < N; ++i) {
      double s = 0.0;
      for (int m = 0; m < H; ++m) s += or_mat_at(P2, i, m) * h[(size_t)b * H + m];
      logits[(size_t)b * N + i] = s + or_vec_at(c2, i);
    }
  if (h_out)
    for (size_t t = 0; t < (size_t)B * H; ++t) h_out[t] = h[t];
  free(h);
}

void or_compact(int B, int N, const double* logits, float tau, const int32_t* T_g, int n_g,
                int32_t* A_g, int32_t* K, const int32_t* T_c, int n_c, int32_t* A_c, int32_t* K_c) {
  unsigned char* M = (unsigned char*)calloc((size_t)N, 1);
  for (int i = 0; i < N; ++i)
    for (int b = 0; b < B; ++b)
      if ((float)logits[(size_t)b * N + i] > tau) { M[i] = 1; break; }
  int k = 0;
  for (int s = 0; s < n_g; ++s)
    if (M[T_g[s]]) A_g[k++] = s;
  *K = k;
  if (T_c) {
    int kc = 0;
    for (int c = 0; c < n_c; ++c)
      if (M[T_c[c]]) A_c[kc++] = c;
    *K_c = kc;
  }
  free(M);
}

static double neuron_act(int kind, const float* xb, int d, or_mat W1, or_vec b1, or_mat Wup, int64_t r) {
  double z = dot_row(W1, r, xb, d) + or_vec_at(b1, r);
  double a = z > 0.0 ? z : 0.0;
  if (kind == OR_GATED_RELU) a *= dot_row(Wup, r, xb, d);
  return a;
}

void or_sparse_ffn(int B, int d, int kind, const float* x, or_mat W1, or_vec b1, or_mat Wup,
                   or_mat W2, const int32_t* rows, int K, double* a_out, double* y) {
  double* a = (double*)malloc(sizeof(double) * ((size_t)B * K + 1));
#pragma omp parallel for collapse(2) schedule(static) num_threads(OR_NT)
  for (int b = 0; b < B; ++b)
    for (int j = 0; j < K; ++j)
      a[(size_t)b * K + j] = neuron_act(kind, x + (size_t)b * d, d, W1, b1, Wup, rows[j]);
#pragma omp parallel for collapse(2) schedule(static) num_threads(OR_NT)
  for (int b = 0; b < B; ++b)
    for (int c = 0; c < d; ++c) {
      double s = 0.0;
      for (int j = 0; j < K; ++j) s += a[(size_t)b * K + j] * or_mat_at(W2, rows[j], c);
      y[(size_t)b * d + c] = s;
    }
  if (a_out)
    for (size_t t = 0; t < (size_t)B * K; ++t) a_out[t] = a[t];
  free(a);
}

void or_dense_ffn(int B, int d, int n, int kind, const float* x, or_mat W1, or_vec b1, or_mat Wup,
                  or_mat W2, or_vec b2, double* y) {
  int32_t* rows = (int32_t*)malloc(sizeof(int32_t) * ((size_t)n + 1));
  for (int i = 0; i < n; ++i) rows[i] = i;
  or_sparse_ffn(B, d, kind, x, W1, b1, Wup, W2, rows, n, NULL, y);
  for (int b = 0; b < B; ++b)
    for (int c = 0; c < d; ++c) y[(size_t)b * d + c] += or_vec_at(b2, c);
  free(rows);
}

void or_merge(int B, int d, const double* y_g, const double* y_c, int K_c, or_vec b2, double* y) {
  for (int b = 0; b < B; ++b)
    for (int c = 0; c < d; ++c) {
      size_t t = (size_t)b * d + c;
      double v = y_g[t];
      if (y_c && K_c != 0) v += y_c[t];
      y[t] = v + or_vec_at(b2, c);
    }
}

void or_layer_norm(int B, int d, const float* y, double eps, double* x) {
  for (int b = 0; b < B; ++b) {
    const float* r = y + (size_t)b * d;
    double mu = 0.0, var = 0.0;
    for (int k = 0; k < d; ++k) mu += (double)r[k];
    mu /= (double)d;
    for (int k = 0; k < d; ++k) var += ((double)r[k] - mu) * ((double)r[k] - mu);
    var /= (double)d;
    const double sd = sqrt(var + eps);
    for (int k = 0; k < d; ++k) x[(size_t)b * d + k] = ((double)r[k] - mu) / sd;
  }
}

uint16_t or_double_to_f16(double v) {
  const uint16_t sign = signbit(v) ? 0x8000u : 0u;
  if (isnan(v)) return 0x7e00u;
  const double a = fabs(v);
  if (a >= 65520.0) return sign | 0x7c00u;   /* at or past the midpoint above 65504: infinity */
  int e = 0;
  (void)frexp(a, &e);                        /* a = m 2^e, m in [0.5, 1) */
  if (a != 0.0 && e - 1 >= -14) {            /* normal: a = (1 + f / 1024) 2^E */
    int E = e - 1;
    double r = nearbyint(ldexp(a, 10 - E));  /* in [1024, 2048], ties to even */
    if (r >= 2048.0) { r = 1024.0; E += 1; }
    if (E > 15) return sign | 0x7c00u;
    return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | (uint16_t)((int)r - 1024));
  }
  const double r = nearbyint(ldexp(a, 24));  /* subnormal: k 2^-24, ties to even */
  if (r >= 1024.0) return (uint16_t)(sign | 0x0400u);
  return (uint16_t)(sign | (uint16_t)r);
}

void or_attn_decode(int d, int n_heads, int d_h, int Ha, int t, const float* x, or_mat Pa1, or_vec ca1,
                    or_mat Pa2, or_vec ca2, float tau, or_mat Wq, or_vec bq, or_mat Wk, or_vec bk, or_mat Wv,
                    or_vec bv, or_mat WoT, or_vec bo, const uint16_t* Kc, const uint16_t* Vc, int L_max,
                    double* head_logits, int32_t* heads, int32_t* n_active, uint16_t* k_new, uint16_t* v_new,
                    double* y) {
  /* the head predictor is the FFN predictor's MLP with one output per head */
  or_predict(1, d, Ha, n_heads, x, Pa1, ca1, Pa2, ca2, NULL, head_logits);
  int na = 0;
  for (int h = 0; h < n_heads; ++h)
    if ((float)head_logits[h] > tau) heads[na++] = h;
  *n_active = na;
  /* this token's cache entry, every head */
#pragma omp parallel for schedule(static) num_threads(OR_NT)
  for (int r = 0; r < d; ++r) {
    k_new[r] = or_double_to_f16(dot_row(Wk, r, x, d) + or_vec_at(bk, r));
    v_new[r] = or_double_to_f16(dot_row(Wv, r, x, d) + or_vec_at(bv, r));
  }
  /* the active heads' outputs */
  double* o = (double*)calloc((size_t)n_heads * d_h, sizeof(double));
  const double scale = 1.0 / sqrt((double)d_h);
#pragma omp parallel for schedule(dynamic) num_threads(OR_NT)
  for (int a = 0; a < na; ++a) {
    const int h = heads[a];
    double* q = (double*)malloc(sizeof(double) * (size_t)d_h);
    double* e = (double*)malloc(sizeof(double) * (size_t)(t + 1));
    for (int i = 0; i < d_h; ++i) q[i] = dot_row(Wq, (int64_t)h * d_h + i, x, d) + or_vec_at(bq, (int64_t)h * d_h + i);
    double mx = -INFINITY;
    for (int j = 0; j <= t; ++j) {
      double s = 0.0;
      for (int i = 0; i < d_h; ++i) {
        const uint16_t kb = j < t ? Kc[((size_t)h * L_max + j) * d_h + i] : k_new[(size_t)h * d_h + i];
        s += q[i] * or_f16_to_double(kb);
      }
      e[j] = s * scale;
      if (e[j] > mx) mx = e[j];
    }
    double z = 0.0;
    for (int j = 0; j <= t; ++j) { e[j] = exp(e[j] - mx); z += e[j]; }
    for (int i = 0; i < d_h; ++i) {
      double acc = 0.0;
      for (int j = 0; j <= t; ++j) {
        const uint16_t vb = j < t ? Vc[((size_t)h * L_max + j) * d_h + i] : v_new[(size_t)h * d_h + i];
        acc += e[j] * or_f16_to_double(vb);
      }
      o[(size_t)h * d_h + i] = acc / z;
    }
    free(q);
    free(e);
  }
#pragma omp parallel for schedule(static) num_threads(OR_NT)
  for (int c = 0; c < d; ++c) {
    double s = or_vec_at(bo, c);
    for (int a = 0; a < na; ++a) {
      const int h = heads[a];
      for (int i = 0; i < d_h; ++i) s += o[(size_t)h * d_h + i] * or_mat_at(WoT, (int64_t)h * d_h + i, c);
    }
    y[c] = s;
  }
  free(o);
}
