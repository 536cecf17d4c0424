// sanitize_host.cpp - host code under AddressSanitizer and UndefinedBehaviorSanitizer.
//
// Test infrastructure (built and run by tests/test_host_sanitizers.py with g++
// -fsanitize=address,undefined; host code only, no GPU code).  It drives the CPU
// side of the hybrid layer (pi_cold_ffn_ex on both code paths and several thread
// counts, pi_host_read_probe) and the oracle's functions over seeded inputs of
// small, ragged shapes, and checks the host operator against the oracle on the
// same rows.  Exit status 0 = clean and within bounds.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "../include/pi_host.h"
extern "C" {
#include "../oracle/oracle.h"
}

namespace {

uint64_t g_state = 0x9E3779B97F4A7C15ull;
uint64_t next_u64() {   // xorshift64*
  g_state ^= g_state >> 12;
  g_state ^= g_state << 25;
  g_state ^= g_state >> 27;
  return g_state * 2685821657736338717ull;
}
float uniform_pm1() { return (float)((next_u64() >> 11) * (1.0 / 9007199254740992.0)) * 2.f - 1.f; }

uint16_t to_f16(float f) {   // round to nearest even, normal range only (|f| < 65504, inputs here are small)
  uint32_t u;
  memcpy(&u, &f, 4);
  const uint32_t sign = (u >> 16) & 0x8000u;
  int32_t e = (int32_t)((u >> 23) & 0xFF) - 127 + 15;
  uint32_t m = u & 0x7FFFFFu;
  if (e <= 0) return (uint16_t)sign;   // flush tiny values to zero
  uint32_t r = m >> 13, rem = m & 0x1FFFu;
  if (rem > 0x1000u || (rem == 0x1000u && (r & 1u))) ++r;
  if (r == 0x400u) { r = 0; ++e; }
  return (uint16_t)(sign | ((uint32_t)e << 10) | r);
}

struct HostMat {
  std::vector<uint8_t> data;
  std::vector<uint16_t> scales;
  int dtype;
};

// rows x cols values in [-s, s] in the given storage format
HostMat make_mat(int rows, int cols, int dtype, float s) {
  HostMat m;
  m.dtype = dtype;
  if (dtype == PI_F32) {
    m.data.resize((size_t)rows * cols * 4);
    float* p = reinterpret_cast<float*>(m.data.data());
    for (size_t i = 0; i < (size_t)rows * cols; ++i) p[i] = uniform_pm1() * s;
  } else if (dtype == PI_F16) {
    m.data.resize((size_t)rows * cols * 2);
    uint16_t* p = reinterpret_cast<uint16_t*>(m.data.data());
    for (size_t i = 0; i < (size_t)rows * cols; ++i) p[i] = to_f16(uniform_pm1() * s);
  } else {
    m.data.resize((size_t)rows * cols / 2);
    m.scales.resize((size_t)rows * cols / 128);
    for (auto& b : m.data) b = (uint8_t)(next_u64() & 0xFF);
    for (auto& v : m.scales) v = to_f16(s / 7.f);
  }
  return m;
}

pi_matrix pm(const HostMat& m) { return pi_matrix{m.data.data(), m.scales.empty() ? nullptr : m.scales.data(), m.dtype}; }
or_mat om(const HostMat& m, int cols) {
  return or_mat{m.data.data(), m.scales.empty() ? nullptr : m.scales.data(), m.dtype, cols};
}

int g_fail = 0;
void check(bool ok, const char* what) {
  if (!ok) {
    fprintf(stderr, "FAIL: %s\n", what);
    ++g_fail;
  }
}

void cold_ffn_case(int B, int d, int n_c, int kind, int dtype, int K_c) {
  HostMat W1 = make_mat(n_c, d, dtype, 1.f / sqrtf((float)d)), W2 = make_mat(n_c, d, dtype, 0.05f);
  HostMat Wup = kind == PI_GATED_RELU ? make_mat(n_c, d, dtype, 1.f / sqrtf((float)d)) : HostMat{{}, {}, dtype};
  std::vector<uint16_t> b1(n_c);
  for (auto& v : b1) v = to_f16(uniform_pm1() * 0.5f);
  std::vector<float> x((size_t)B * d);
  for (auto& v : x) v = uniform_pm1();
  // ascending distinct listed rows
  std::vector<int32_t> A;
  for (int r = 0; r < n_c && (int)A.size() < K_c; ++r)
    if ((next_u64() & 3u) != 0u || n_c - r <= K_c - (int)A.size()) A.push_back(r);
  const int K = (int)A.size();
  std::vector<double> y_or((size_t)B * d);
  or_sparse_ffn(B, d, kind, x.data(), om(W1, d), or_vec{b1.data(), OR_F16},
                kind == PI_GATED_RELU ? om(Wup, d) : or_mat{nullptr, nullptr, OR_F32, d}, om(W2, d), A.data(), K,
                nullptr, y_or.data());
  std::vector<float> ref;
  for (int path = 0; path <= (pi_host_vector_path() ? 1 : 0); ++path) {
    for (int threads : {1, 3, 8}) {
      std::vector<float> y((size_t)B * d, -1.f);
      const int st = pi_cold_ffn_ex(B, d, n_c, kind, x.data(), pm(W1), pi_vector{b1.data(), PI_F16},
                                    kind == PI_GATED_RELU ? pm(Wup) : pi_matrix{nullptr, nullptr, dtype}, pm(W2),
                                    A.data(), K, y.data(), threads, path);
      check(st == PI_OK, "pi_cold_ffn_ex status");
      double worst = 0.0, norm = 0.0;
      for (size_t i = 0; i < y.size(); ++i) {
        worst = fmax(worst, fabs((double)y[i] - y_or[i]));
        norm = fmax(norm, fabs(y_or[i]));
      }
      check(worst <= 1e-4 * fmax(norm, 1e-30) + 1e-30, "pi_cold_ffn_ex against the oracle");
      if (ref.empty()) ref = y;
      else check(memcmp(ref.data(), y.data(), y.size() * 4) == 0, "pi_cold_ffn_ex bits across paths and threads");
    }
  }
}

void oracle_cases() {
  const int B = 3, d = 136, H = 24, N = 200;
  HostMat P1 = make_mat(H, d, PI_F16, 1.f / sqrtf((float)d)), P2 = make_mat(N, H, PI_F32, 0.3f);
  std::vector<float> x((size_t)B * d);
  for (auto& v : x) v = uniform_pm1();
  std::vector<double> h((size_t)B * H), logits((size_t)B * N);
  or_predict(B, d, H, N, x.data(), om(P1, d), or_vec{nullptr, OR_F32}, om(P2, H), or_vec{nullptr, OR_F32}, h.data(),
             logits.data());
  std::vector<int32_t> T_g, T_c;
  for (int i = 0; i < N; ++i) (i % 3 ? T_g : T_c).push_back(i);
  std::vector<int32_t> A_g(T_g.size()), A_c(T_c.size());
  int32_t K = -1, K_c = -1;
  or_compact(B, N, logits.data(), 0.f, T_g.data(), (int)T_g.size(), A_g.data(), &K, T_c.data(), (int)T_c.size(),
             A_c.data(), &K_c);
  check(K >= 0 && K <= (int)T_g.size() && K_c >= 0 && K_c <= (int)T_c.size(), "or_compact counts");
  HostMat W1 = make_mat(N, d, PI_F32, 0.1f), W2 = make_mat(N, d, PI_F32, 0.1f);
  std::vector<double> y((size_t)B * d), yd((size_t)B * d), ym((size_t)B * d);
  or_dense_ffn(B, d, N, OR_RELU, x.data(), om(W1, d), or_vec{nullptr, OR_F32}, or_mat{nullptr, nullptr, OR_F32, d},
               om(W2, d), or_vec{nullptr, OR_F32}, yd.data());
  or_merge(B, d, yd.data(), nullptr, 0, or_vec{nullptr, OR_F32}, ym.data());
  std::vector<float> yf((size_t)B * d);
  for (size_t i = 0; i < yf.size(); ++i) yf[i] = (float)ym[i];
  std::vector<double> xn((size_t)B * d);
  or_layer_norm(B, d, yf.data(), 1e-5, xn.data());
  check(isfinite(xn[0]), "or_layer_norm");
}

}  // namespace

int main() {
  for (int dtype : {PI_F32, PI_F16, PI_I4G128})
    for (int kind : {PI_RELU, PI_GATED_RELU})
      for (int B : {1, 3}) {
        const int d = dtype == PI_I4G128 ? 384 : 264;
        cold_ffn_case(B, d, 300, kind, dtype, 5);      // few listed rows: column slices
        cold_ffn_case(B, d, 700, kind, dtype, 400);    // many: row chunks
        cold_ffn_case(B, d, 50, kind, dtype, 0);       // none
      }
  // the host streaming read over a 64-byte aligned buffer
  const size_t nb = 1 << 20;
  void* buf = aligned_alloc(64, nb);
  memset(buf, 0x5A, nb);
  uint64_t out = 0;
  check(pi_host_read_probe(buf, nb, 4, &out) == PI_OK, "pi_host_read_probe");
  free(buf);
  oracle_cases();
  if (g_fail) return 1;
  puts("sanitized host run clean");
  return 0;
}
