// pi_host.cpp - libpi_host: the FFN over the CPU-resident (cold) neurons, on
// the host, for the pages' GPU-CPU hybrid layer.
//
// FC1: each listed neuron's row is read once and dotted with every batch row
// of x (threads take fixed ranges of the list).  FC2 over the neurons with a
// non-zero output, in list order: when they are few, each thread streams its
// fixed column slice of every such row into its slice of y_c; when they are
// many, they are cut into chunks of a size fixed by their count alone, a
// thread streams whole W2 rows of a chunk into that chunk's partial y (each
// row one contiguous run, which the hardware prefetchers follow), and y_c is
// the sum of the chunks' partials in chunk order.  A dot product keeps 32 partial sums
// (4 x 8 lanes, k = 32 i + 8 q + l) and adds them in one fixed tree, with fused
// multiply-adds; the AVX2 path and the scalar path follow the same order, so
// the bits are the same on either and for any thread count.
#include <immintrin.h>
#include <omp.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <vector>

#include "../../include/pi_host.h"

namespace {

// IEEE binary16 -> binary32 (exact).
inline float half_to_float(uint16_t h) {
  const uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
  const uint32_t exp = (h >> 10) & 0x1Fu;
  uint32_t man = h & 0x3FFu;
  uint32_t bits;
  if (exp == 0) {
    if (man == 0) {
      bits = sign;
    } else {                      // subnormal: m * 2^-24, renormalised
      int shift = 0;
      while (!(man & 0x400u)) { man <<= 1; ++shift; }
      bits = sign | ((uint32_t)(113 - shift) << 23) | ((man & 0x3FFu) << 13);
    }
  } else if (exp == 31) {
    bits = sign | 0x7F800000u | (man << 13);
  } else {
    bits = sign | ((exp + 112u) << 23) | (man << 13);
  }
  float f;
  memcpy(&f, &bits, 4);
  return f;
}

constexpr int64_t kFc1PrefetchBytes = 2048;   // FC1: leading bytes of the next row requested early
constexpr int64_t kRowPrefetchBytes = 2048;   // distance of the software prefetch inside a row
constexpr int64_t kFc2ChunkMinRows = 128;   // FC2: fewer contributing rows take column ranges
constexpr int64_t kFc2ChunkRows = 16;   // FC2: fewest rows per chunk
constexpr int64_t kFc2MaxChunks = 64;   // FC2: most chunks (bounds the partials at 64 x B x d floats)

struct Rows {
  const char* data;
  const uint16_t* scales;
  int dt;
  int64_t rb;      // bytes per row
  int64_t groups;  // int4 scale groups per row
  const char* row(int64_t r) const { return data + r * rb; }
};

int64_t row_bytes(int dt, int64_t d) { return dt == PI_F32 ? d * 4 : dt == PI_F16 ? d * 2 : d / 2; }

// Eight consecutive weights k0 .. k0 + 7 of row r as floats (k0 a multiple of 8).
inline void load8_scalar(const Rows& w, int64_t r, int64_t k0, float* out) {
  const char* p = w.row(r);
  if (w.dt == PI_F32) {
    memcpy(out, p + k0 * 4, 32);
  } else if (w.dt == PI_F16) {
    uint16_t h[8];
    memcpy(h, p + k0 * 2, 16);
    for (int l = 0; l < 8; ++l) out[l] = half_to_float(h[l]);
  } else {
    const float s = half_to_float(w.scales[r * w.groups + k0 / 128]);
    uint8_t b[4];
    memcpy(b, p + k0 / 2, 4);
    for (int l = 0; l < 8; ++l) {
      const int nib = (l & 1) ? (b[l / 2] >> 4) : (b[l / 2] & 0xF);
      out[l] = (float)(nib >= 8 ? nib - 16 : nib) * s;
    }
  }
}

float bias_at(const pi_vector& v, int64_t i) {
  if (!v.data) return 0.f;
  if (v.dtype == PI_F32) return static_cast<const float*>(v.data)[i];
  return half_to_float(static_cast<const uint16_t*>(v.data)[i]);
}

// The fixed tree over the 32 partial sums: lanes of the 4 groups, then halves.
inline float tree32(const float (&acc)[4][8]) {
  float t[8];
  for (int l = 0; l < 8; ++l) t[l] = (acc[0][l] + acc[1][l]) + (acc[2][l] + acc[3][l]);
  float u[4];
  for (int l = 0; l < 4; ++l) u[l] = t[l] + t[l + 4];
  return (u[0] + u[2]) + (u[1] + u[3]);
}

// dot[b] = W[r] . x_b for b < B (scalar path).
void dots_scalar(const Rows& w, int64_t r, const float* x, int B, int64_t d, float* dot) {
  for (int b = 0; b < B; ++b) {
    const float* xb = x + (int64_t)b * d;
    float acc[4][8] = {};
    float wv[8];
    for (int64_t k0 = 0; k0 < d; k0 += 32)
      for (int q = 0; q < 4 && k0 + 8 * q < d; ++q) {
        load8_scalar(w, r, k0 + 8 * q, wv);
        for (int l = 0; l < 8; ++l) acc[q][l] = std::fma(wv[l], xb[k0 + 8 * q + l], acc[q][l]);
      }
    dot[b] = tree32(acc);
  }
}

// y[b, c0 .. c1) += a[b] * W[r, c0 .. c1) for the b with a[b] != 0 (scalar path).
void axpy_scalar(const Rows& w, int64_t r, const float* a, int B, int64_t d, int64_t c0, int64_t c1, float* y) {
  float wv[8];
  for (int64_t c = c0; c < c1; c += 8) {
    load8_scalar(w, r, c, wv);
    for (int b = 0; b < B; ++b) {
      if (a[b] == 0.f) continue;
      float* yb = y + (int64_t)b * d + c;
      for (int l = 0; l < 8; ++l) yb[l] = std::fma(a[b], wv[l], yb[l]);
    }
  }
}

#define PI_AVX2 __attribute__((target("avx2,fma,f16c")))

PI_AVX2 inline __m256 load8_avx2(const Rows& w, int64_t r, int64_t k0) {
  const char* p = w.row(r);
  if (w.dt == PI_F32) return _mm256_loadu_ps(reinterpret_cast<const float*>(p) + k0);
  if (w.dt == PI_F16) return _mm256_cvtph_ps(_mm_loadu_si128(reinterpret_cast<const __m128i*>(p + k0 * 2)));
  float f[8];
  load8_scalar(w, r, k0, f);
  return _mm256_loadu_ps(f);
}

PI_AVX2 float tree32_avx2(__m256 a0, __m256 a1, __m256 a2, __m256 a3) {
  const __m256 t = _mm256_add_ps(_mm256_add_ps(a0, a1), _mm256_add_ps(a2, a3));
  const __m128 u = _mm_add_ps(_mm256_castps256_ps128(t), _mm256_extractf128_ps(t, 1));   // t[l] + t[l+4]
  // (u0 + u2) + (u1 + u3)
  const __m128 v = _mm_add_ps(u, _mm_movehl_ps(u, u));                                  // [u0+u2, u1+u3, ...]
  return _mm_cvtss_f32(_mm_add_ss(v, _mm_shuffle_ps(v, v, 1)));
}

// NB batch rows of one row's dot (NB a compile-time count, so the 4 * NB accumulators stay in
// registers instead of a stack array reloaded and stored around every fma).
template <int NB>
PI_AVX2 inline void dots_avx2_nb(const Rows& w, int64_t r, const float* x, int64_t d, float* dot) {
  __m256 acc[NB][4];
  for (int i = 0; i < NB; ++i)
    for (int q = 0; q < 4; ++q) acc[i][q] = _mm256_setzero_ps();
  const char* rowp = w.row(r);
  // the row's lines kRowPrefetchBytes ahead (the hardware prefetchers stop at page ends); 32
  // columns are pstep bytes of every format (128, 64 or 16), so the offset advances by addition
  const int64_t pstep = w.rb * 32 / d;
  int64_t po = kRowPrefetchBytes;
  int64_t k0 = 0;
  // whole 32-column blocks, every index known at compile time
  for (; k0 + 32 <= d; k0 += 32, po += pstep) {
    if (po < w.rb) _mm_prefetch(rowp + po, _MM_HINT_T0);
    __m256 wv[4];
    for (int q = 0; q < 4; ++q) wv[q] = load8_avx2(w, r, k0 + 8 * q);
    for (int i = 0; i < NB; ++i)
      for (int q = 0; q < 4; ++q)
        acc[i][q] = _mm256_fmadd_ps(wv[q], _mm256_loadu_ps(x + (int64_t)i * d + k0 + 8 * q), acc[i][q]);
  }
  // a tail of 8, 16 or 24 columns (d is a multiple of 8) into the first accumulators
  if (k0 < d) {
    const int nq = (int)((d - k0) / 8);
    for (int q = 0; q < 3; ++q) {
      if (q < nq) {
        const __m256 wq = load8_avx2(w, r, k0 + 8 * q);
        for (int i = 0; i < NB; ++i)
          acc[i][q] = _mm256_fmadd_ps(wq, _mm256_loadu_ps(x + (int64_t)i * d + k0 + 8 * q), acc[i][q]);
      }
    }
  }
  for (int i = 0; i < NB; ++i) dot[i] = tree32_avx2(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
}

PI_AVX2 void dots_avx2(const Rows& w, int64_t r, const float* x, int B, int64_t d, float* dot) {
  for (int b0 = 0; b0 < B; b0 += 4) {
    const float* xb = x + (int64_t)b0 * d;
    switch (B - b0 < 4 ? B - b0 : 4) {
      case 1: dots_avx2_nb<1>(w, r, xb, d, dot + b0); break;
      case 2: dots_avx2_nb<2>(w, r, xb, d, dot + b0); break;
      case 3: dots_avx2_nb<3>(w, r, xb, d, dot + b0); break;
      default: dots_avx2_nb<4>(w, r, xb, d, dot + b0); break;
    }
  }
}

PI_AVX2 void axpy_avx2(const Rows& w, int64_t r, const float* a, int B, int64_t d, int64_t c0, int64_t c1, float* y) {
  const char* rowp = w.row(r);
  const int64_t end = c1 * w.rb / d;
  // one line per 32 columns of fp16 (two of fp32): the first multiple of 32 at or after c0, then
  // pstep bytes (128, 64 or 16) per 32 columns, by addition
  const int64_t pstep = w.rb * 32 / d;
  int64_t po = ((c0 + 31) & ~(int64_t)31) * w.rb / d + kRowPrefetchBytes;
  for (int64_t c = c0; c < c1; c += 8) {
    if ((c & 31) == 0) {
      if (po < end) _mm_prefetch(rowp + po, _MM_HINT_T0);
      po += pstep;
    }
    const __m256 wv = load8_avx2(w, r, c);
    for (int b = 0; b < B; ++b) {
      if (a[b] == 0.f) continue;
      float* yb = y + (int64_t)b * d + c;
      _mm256_storeu_ps(yb, _mm256_fmadd_ps(_mm256_set1_ps(a[b]), wv, _mm256_loadu_ps(yb)));
    }
  }
}

bool have_avx2() {
  static const bool ok = __builtin_cpu_supports("avx2") && __builtin_cpu_supports("fma") &&
                         __builtin_cpu_supports("f16c");
  return ok;
}

bool valid_dtype(int dt) { return dt == PI_F32 || dt == PI_F16 || dt == PI_I4G128; }

}  // namespace

extern "C" int pi_host_vector_path(void) { return have_avx2() ? 1 : 0; }

namespace {

// XOR of the 64-byte lines [l0, l1) of p, four 32-byte accumulators.
PI_AVX2 uint64_t xor_lines_avx2(const uint8_t* p, int64_t l0, int64_t l1) {
  __m256i s0 = _mm256_setzero_si256(), s1 = s0, s2 = s0, s3 = s0;
  int64_t l = l0;
  for (; l + 2 <= l1; l += 2) {
    const __m256i* q = reinterpret_cast<const __m256i*>(p + l * 64);
    s0 = _mm256_xor_si256(s0, _mm256_load_si256(q));
    s1 = _mm256_xor_si256(s1, _mm256_load_si256(q + 1));
    s2 = _mm256_xor_si256(s2, _mm256_load_si256(q + 2));
    s3 = _mm256_xor_si256(s3, _mm256_load_si256(q + 3));
  }
  if (l < l1) {
    const __m256i* q = reinterpret_cast<const __m256i*>(p + l * 64);
    s0 = _mm256_xor_si256(s0, _mm256_load_si256(q));
    s1 = _mm256_xor_si256(s1, _mm256_load_si256(q + 1));
  }
  const __m256i s = _mm256_xor_si256(_mm256_xor_si256(s0, s1), _mm256_xor_si256(s2, s3));
  alignas(32) uint64_t w[4];
  _mm256_store_si256(reinterpret_cast<__m256i*>(w), s);
  return w[0] ^ w[1] ^ w[2] ^ w[3];
}

uint64_t xor_lines_scalar(const uint8_t* p, int64_t l0, int64_t l1) {
  const uint64_t* q = reinterpret_cast<const uint64_t*>(p);
  uint64_t s = 0;
  for (int64_t i = l0 * 8; i < l1 * 8; ++i) s ^= q[i];
  return s;
}

}  // namespace

extern "C" int pi_host_read_probe(const void* buf, size_t bytes, int32_t threads, uint64_t* out) {
  if (!buf || !out || bytes == 0 || bytes % 64 != 0 || (reinterpret_cast<uintptr_t>(buf) & 63) != 0)
    return PI_EINVAL;
  const int nt = threads > 0 ? threads : omp_get_max_threads();
  const uint8_t* p = static_cast<const uint8_t*>(buf);
  const int64_t lines = (int64_t)(bytes / 64);
  const bool vec = have_avx2();
  uint64_t acc = 0;
#pragma omp parallel for schedule(static) num_threads(nt) reduction(^ : acc)
  for (int t = 0; t < nt; ++t) {
    const int64_t l0 = lines * t / nt, l1 = lines * (t + 1) / nt;
    acc ^= vec ? xor_lines_avx2(p, l0, l1) : xor_lines_scalar(p, l0, l1);
  }
  *out = acc;
  return PI_OK;
}

extern "C" int pi_cold_ffn_ex(int32_t B, int32_t d, int32_t n_c, int32_t kind, const float* x, pi_matrix W1,
                              pi_vector b1, pi_matrix Wup, pi_matrix W2, const int32_t* A_c, int32_t K_c, float* y_c,
                              int32_t threads, int32_t path) {
  if (B < 1 || B > PI_MAX_BATCH || d <= 0 || K_c < 0 || n_c < K_c || !x || !y_c) return PI_EINVAL;
  if (path < -1 || path > 1) return PI_EINVAL;
  if (path == 1 && !have_avx2()) return PI_EUNSUPPORTED;
  if (kind != PI_RELU && kind != PI_GATED_RELU) return PI_EINVAL;
  const bool gated = kind == PI_GATED_RELU;
  if (!valid_dtype(W1.dtype) || !valid_dtype(W2.dtype) || (gated && !valid_dtype(Wup.dtype))) return PI_EINVAL;
  if (d % (W1.dtype == PI_I4G128 ? 128 : 8) != 0) return PI_EINVAL;
  if (b1.data && b1.dtype != PI_F32 && b1.dtype != PI_F16) return PI_EINVAL;
  if (K_c > 0 && (!A_c || !W1.data || !W2.data || (gated && !Wup.data))) return PI_EINVAL;
  if (W2.dtype != W1.dtype || (gated && Wup.dtype != W1.dtype)) return PI_EUNSUPPORTED;
  if (W1.dtype == PI_I4G128 && (!W1.scales || !W2.scales || (gated && !Wup.scales))) return PI_EINVAL;
  for (int32_t j = 0; j < K_c; ++j)
    if (A_c[j] < 0 || A_c[j] >= n_c) return PI_EINVAL;

  const int64_t dd = d;
  const int64_t rb = row_bytes(W1.dtype, dd);
  const Rows w1{static_cast<const char*>(W1.data), W1.scales, W1.dtype, rb, dd / 128};
  const Rows wu{static_cast<const char*>(gated ? Wup.data : W1.data), gated ? Wup.scales : W1.scales, W1.dtype, rb,
                dd / 128};
  const Rows w2{static_cast<const char*>(W2.data), W2.scales, W2.dtype, rb, dd / 128};
  const bool vec = path == -1 ? have_avx2() : path == 1;
  const int nt = threads > 0 ? threads : omp_get_max_threads();

  // One parallel region for the whole call: FC1, the list of contributing neurons, FC2 (and the
  // chunk sum), separated by barriers rather than a fork and a join per phase.
  std::vector<float> a((size_t)K_c * B);               // FC1 outputs, a[j * B + b]
  std::vector<int32_t> act;                              // neurons with a != 0, in list order
  act.reserve((size_t)K_c);
  static thread_local std::vector<float> part;           // the calling thread's, reused between calls
  std::vector<float>* const partp = &part;
  const int64_t nvec = dd / 8;
  const int64_t plane = (int64_t)B * dd;
  int64_t R = 0, crows = 0, nch = 0;
  float* pp = nullptr;
#pragma omp parallel num_threads(nt)
  {
#pragma omp for schedule(static)
    for (int32_t j = 0; j < K_c; ++j) {
      const int64_t c = A_c[j];
      // the next listed row starts a new stream: request its first lines before this row's dot
      if (j + 1 < K_c) {
        const char* pn = w1.row(A_c[j + 1]);
        for (int64_t o = 0; o < kFc1PrefetchBytes && o < rb; o += 64) _mm_prefetch(pn + o, _MM_HINT_T0);
      }
      float z[PI_MAX_BATCH], u[PI_MAX_BATCH];
      if (vec) dots_avx2(w1, c, x, B, dd, z);
      else dots_scalar(w1, c, x, B, dd, z);
      if (gated) {
        if (vec) dots_avx2(wu, c, x, B, dd, u);
        else dots_scalar(wu, c, x, B, dd, u);
      }
      const float bias = bias_at(b1, c);
      for (int b = 0; b < B; ++b) {
        float v = z[b] + bias;
        v = v > 0.f ? v : 0.f;
        if (gated) v *= u[b];
        a[(size_t)j * B + b] = v;
      }
    }
    // FC2.  Few contributing rows: every thread takes a fixed range of columns over all the rows
    // (all threads busy).  Many: chunks of whole rows (at least kFc2ChunkRows, at most
    // kFc2MaxChunks chunks), each into its own partial [B x d], then the partials summed in chunk
    // order (contiguous runs the hardware prefetchers follow).  Which one depends on the row count
    // only.
#pragma omp single
    {
      for (int32_t j = 0; j < K_c; ++j) {
        bool any = false;
        for (int b = 0; b < B; ++b) any = any || a[(size_t)j * B + b] != 0.f;
        if (any) act.push_back(j);
      }
      R = (int64_t)act.size();
      if (R >= kFc2ChunkMinRows) {
        crows = (R + kFc2MaxChunks - 1) / kFc2MaxChunks;
        crows = crows < kFc2ChunkRows ? kFc2ChunkRows : crows;
        nch = (R + crows - 1) / crows;
        if ((int64_t)partp->size() < nch * plane) partp->resize((size_t)(nch * plane));
        pp = partp->data();
      }
    }
    if (R < kFc2ChunkMinRows) {
#pragma omp for schedule(static)
      for (int t = 0; t < nt; ++t) {
        const int64_t c0 = nvec * t / nt * 8, c1 = nvec * (t + 1) / nt * 8;
        for (int b = 0; b < B; ++b)
          for (int64_t c = c0; c < c1; ++c) y_c[(int64_t)b * dd + c] = 0.f;
        if (c0 == c1) continue;
        for (int64_t q = 0; q < R; ++q) {
          const int32_t j = act[(size_t)q];
          if (vec) axpy_avx2(w2, A_c[j], &a[(size_t)j * B], B, dd, c0, c1, y_c);
          else axpy_scalar(w2, A_c[j], &a[(size_t)j * B], B, dd, c0, c1, y_c);
        }
      }
    } else {
#pragma omp for schedule(static)
      for (int64_t ch = 0; ch < nch; ++ch) {
        float* yp = pp + ch * plane;
        std::fill(yp, yp + plane, 0.f);
        const int64_t q1 = (ch + 1) * crows < R ? (ch + 1) * crows : R;
        for (int64_t q = ch * crows; q < q1; ++q) {
          const int32_t j = act[(size_t)q];
          if (vec) axpy_avx2(w2, A_c[j], &a[(size_t)j * B], B, dd, 0, dd, yp);
          else axpy_scalar(w2, A_c[j], &a[(size_t)j * B], B, dd, 0, dd, yp);
        }
      }
#pragma omp for schedule(static)
      for (int t = 0; t < nt; ++t) {
        const int64_t c0 = nvec * t / nt * 8, c1 = nvec * (t + 1) / nt * 8;
        for (int b = 0; b < B; ++b) {
          float* yb = y_c + (int64_t)b * dd;
          for (int64_t c = c0; c < c1; ++c) yb[c] = 0.f;
          for (int64_t ch = 0; ch < nch; ++ch) {
            const float* pb = pp + ch * plane + (int64_t)b * dd;
            for (int64_t c = c0; c < c1; ++c) yb[c] += pb[c];
          }
        }
      }
    }
  }
  return PI_OK;
}

extern "C" int pi_cold_ffn(int32_t B, int32_t d, int32_t n_c, int32_t kind, const float* x, pi_matrix W1,
                           pi_vector b1, pi_matrix Wup, pi_matrix W2, const int32_t* A_c, int32_t K_c, float* y_c,
                           int32_t threads) {
  return pi_cold_ffn_ex(B, d, n_c, kind, x, W1, b1, Wup, W2, A_c, K_c, y_c, threads, -1);
}
