// pi_abi.hip - the C ABI of libpi: argument validation, workspace layout and
// kernel launches.  Declarations and their sources: include/pi.h.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "../../include/pi.h"
#include "pi_internal.h"

namespace {

thread_local int32_t g_last_hip_error = 0;

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_dtype(int32_t dt) { return dt == PI_F32 || dt == PI_F16 || dt == PI_I4G128; }

// A matrix whose rows have `cols` elements is usable by the kernels.
bool valid_matrix(const pi_matrix& m, int64_t cols) {
  if (!m.data || !aligned16(m.data) || !valid_dtype(m.dtype) || cols <= 0) return false;
  if (m.dtype == PI_I4G128) return cols % 128 == 0 && m.scales != nullptr;
  return cols % 8 == 0;
}

bool valid_vector(const pi_vector& v) { return !v.data || v.dtype == PI_F32 || v.dtype == PI_F16; }

bool valid_batch(int32_t B) { return B >= 1 && B <= PI_MAX_BATCH; }

int hip_status(hipError_t e) {
  if (e == hipSuccess) return PI_OK;
  g_last_hip_error = (int32_t)e;
  return PI_EHIP;
}

struct FfnWs {
  float* a;
  float* partials;
  uint32_t* counters;
  size_t bytes;
};

FfnWs ffn_ws_layout(void* ws, int32_t B, int32_t d, int32_t n_g, int32_t dt) {
  FfnWs w{};
  const size_t a_bytes = align_up((size_t)B * (size_t)(n_g > 0 ? n_g : 1) * 4);
  const size_t p_bytes = align_up((size_t)pi::kFc2Chunks * B * (size_t)d * 4);
  const size_t c_bytes = align_up((size_t)pi::fc2_tiles(dt, d) * 4);
  char* base = static_cast<char*>(ws);
  w.a = reinterpret_cast<float*>(base);
  w.partials = reinterpret_cast<float*>(base + a_bytes);
  w.counters = reinterpret_cast<uint32_t*>(base + a_bytes + p_bytes);
  w.bytes = a_bytes + p_bytes + c_bytes;
  return w;
}

}  // namespace

namespace pi {
hipError_t launch_rowdot_ex(const RowdotArgs& a, int64_t n_rows, uint32_t* zero_ptr, int zero_n, hipStream_t s);
}

extern "C" {

int32_t pi_abi_version(void) { return PI_ABI_VERSION; }

int32_t pi_last_hip_error(void) { return g_last_hip_error; }

const char* pi_status_string(int32_t status) {
  switch (status) {
    case PI_OK: return "PI_OK: success";
    case PI_EINVAL: return "PI_EINVAL: invalid argument";
    case PI_EWORKSPACE: return "PI_EWORKSPACE: workspace too small";
    case PI_EUNSUPPORTED: return "PI_EUNSUPPORTED: unsupported combination of arguments";
    case PI_EHIP: return "PI_EHIP: HIP launch failed (see pi_last_hip_error)";
    default: return "unknown pi status";
  }
}

size_t pi_workspace_bytes(int32_t op, int32_t B, int32_t d, int32_t H, int32_t N, int32_t n_g) {
  (void)N;
  if (B < 1) B = 1;
  switch (op) {
    case PI_OP_PREDICT: return H > 0 ? align_up((size_t)B * (size_t)H * 4) : 0;
    case PI_OP_SPARSE_FFN: {
      if (d <= 0) return 0;
      // the largest layout over the three storage types
      size_t m = 0;
      for (int32_t dt = PI_F32; dt <= PI_I4G128; ++dt) {
        const size_t b = ffn_ws_layout(nullptr, B, d, n_g, dt).bytes;
        if (b > m) m = b;
      }
      return m;
    }
    default: return 0;
  }
}

int pi_predict(void* stream, int32_t B, int32_t d, int32_t H, int32_t N, const float* x, pi_matrix P1,
               pi_vector c1, pi_matrix P2, pi_vector c2, float* logits, void* ws, size_t ws_bytes) {
  if (!valid_batch(B) || d <= 0 || H <= 0 || N <= 0) return PI_EINVAL;
  if (!x || !aligned16(x) || !logits || !valid_matrix(P1, d) || !valid_matrix(P2, H)) return PI_EINVAL;
  if (!valid_vector(c1) || !valid_vector(c2)) return PI_EINVAL;
  if (!ws || !aligned16(ws)) return ws_bytes ? PI_EINVAL : PI_EWORKSPACE;
  if (ws_bytes < pi_workspace_bytes(PI_OP_PREDICT, B, d, H, N, 0)) return PI_EWORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* h = static_cast<float*>(ws);
  pi::RowdotArgs a{};
  a.W = P1.data; a.Ws = P1.scales; a.dt = P1.dtype; a.cols = d;
  a.count_max = H; a.x = x; a.B = B; a.bias = c1.data; a.bias_dt = c1.dtype;
  a.relu = 1; a.out = h; a.out_stride = H;
  int st = hip_status(pi::launch_rowdot(a, s));
  if (st != PI_OK) return st;
  pi::RowdotArgs b{};
  b.W = P2.data; b.Ws = P2.scales; b.dt = P2.dtype; b.cols = H;
  b.count_max = N; b.x = h; b.B = B; b.bias = c2.data; b.bias_dt = c2.dtype;
  b.relu = 0; b.out = logits; b.out_stride = N;
  return hip_status(pi::launch_rowdot(b, s));
}

int pi_compact(void* stream, int32_t B, int32_t N, const float* logits, float tau, const int32_t* T_g,
               int32_t n_g, int32_t* A_g, int32_t* K, const int32_t* T_c, int32_t n_c, int32_t* A_c,
               int32_t* K_c, void* ws, size_t ws_bytes) {
  (void)ws; (void)ws_bytes;
  if (!valid_batch(B) || N <= 0 || n_g < 0 || !logits || !K) return PI_EINVAL;
  if (n_g > 0 && (!T_g || !A_g)) return PI_EINVAL;
  if (T_c && (n_c < 0 || !A_c || !K_c)) return PI_EINVAL;
  if (!T_c) n_c = 0;
  return hip_status(pi::launch_compact(B, N, logits, tau, T_g, n_g, A_g, K, T_c, n_c, A_c, K_c,
                                       static_cast<hipStream_t>(stream)));
}

int pi_sparse_ffn(void* stream, int32_t B, int32_t d, int32_t n_g, int32_t kind, const float* x, pi_matrix W1,
                  pi_vector b1, pi_matrix Wup, pi_matrix W2, const int32_t* A_g, const int32_t* K, float* y_g,
                  void* ws, size_t ws_bytes) {
  if (!valid_batch(B) || d <= 0 || n_g < 0) return PI_EINVAL;
  if (kind != PI_RELU && kind != PI_GATED_RELU) return PI_EINVAL;
  if (!x || !aligned16(x) || !y_g || !aligned16(y_g) || !K) return PI_EINVAL;
  if (n_g > 0 && !A_g) return PI_EINVAL;
  if (!valid_matrix(W1, d) || !valid_matrix(W2, d) || !valid_vector(b1)) return PI_EINVAL;
  if (kind == PI_GATED_RELU) {
    if (!valid_matrix(Wup, d)) return PI_EINVAL;
    if (Wup.dtype != W1.dtype) return PI_EUNSUPPORTED;
  }
  if (W2.dtype != W1.dtype) return PI_EUNSUPPORTED;
  if (!ws || !aligned16(ws)) return PI_EWORKSPACE;
  const FfnWs w = ffn_ws_layout(ws, B, d, n_g, W1.dtype);
  if (ws_bytes < w.bytes) return PI_EWORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int tiles = pi::fc2_tiles(W1.dtype, d);
  pi::RowdotArgs a{};
  a.W = W1.data; a.Ws = W1.scales; a.dt = W1.dtype; a.cols = d;
  a.gated = kind == PI_GATED_RELU;
  if (a.gated) { a.Wup = Wup.data; a.Wups = Wup.scales; }
  a.list = A_g; a.count_dev = K; a.count_max = n_g;
  a.x = x; a.B = B; a.bias = b1.data; a.bias_dt = b1.dtype; a.relu = 1;
  a.out = w.a; a.out_stride = n_g > 0 ? n_g : 1;
  int st = hip_status(pi::launch_rowdot_ex(a, n_g, w.counters, tiles, s));
  if (st != PI_OK) return st;
  pi::Fc2Args f{};
  f.W2 = W2.data; f.W2s = W2.scales; f.dt = W2.dtype; f.d = d; f.n_g = n_g;
  f.list = A_g; f.K = K; f.a = w.a; f.B = B; f.partials = w.partials; f.counters = w.counters; f.y = y_g;
  return hip_status(pi::launch_fc2(f, s));
}

int pi_merge(void* stream, int32_t B, int32_t d, float* y, const float* y_c, const int32_t* K_c, pi_vector b2) {
  if (!valid_batch(B) || d <= 0 || !y || !valid_vector(b2)) return PI_EINVAL;
  if (!y_c && !b2.data) return PI_OK;  // nothing to add
  return hip_status(pi::launch_merge(B, d, y, y_c, K_c, b2.data, b2.dtype, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
