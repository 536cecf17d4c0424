// pi_abi.hip - the C ABI of libpi: argument validation, workspace layout and
// kernel launches.  Declarations and their sources: include/pi.h.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>
#include <stdlib.h>
#include <atomic>
#include <cmath>
#include "../../include/pi.h"
#include "pi_internal.h"
#include "pi_attn.h"

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

// Two byte ranges [a, a + na) and [b, b + nb) share a byte (compared as integer addresses).
bool ranges_overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return na && nb && x < y + nb && y < x + na;
}

int hip_status(hipError_t e) {
  if (e == hipSuccess) return PI_OK;
  g_last_hip_error = (int32_t)e;
  return PI_EHIP;
}

// Carve a workspace into 256-byte aligned regions.
struct Carver {
  char* base;
  size_t off = 0;
  template <class T>
  T* take(size_t bytes) {
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += align_up(bytes);
    return p;
  }
};

struct FfnWs {
  float* a;
  float* partials;
  size_t bytes;
};

// Partial sums of the batched matrix-core GEMMs, bounded over the weight dtypes
// (workspace sizes are asked for without them).
// The smallest batches that take the matrix-core GEMMs: kMmRowMinBatch / kMmAxpyMinBatch, or
// both raised to PI_MATRIX_CORE_MIN_BATCH when that is set (read once; a value above the largest
// batch keeps every batch on the VALU kernels, for comparisons).
int mm_min_batch_env() {
  static const int v = [] {
    const char* e = getenv("PI_MATRIX_CORE_MIN_BATCH");
    if (!e || !*e) return 0;
    const long n = strtol(e, nullptr, 10);
    return n < 1 ? 0 : (n > 1000 ? 1000 : (int)n);
  }();
  return v;
}
bool use_mm_row(int32_t B) {
  const int e = mm_min_batch_env();
  return B >= (e > pi::kMmRowMinBatch ? e : pi::kMmRowMinBatch);
}
bool use_mm_axpy(int32_t B) {
  const int e = mm_min_batch_env();
  return B >= (e > pi::kMmAxpyMinBatch ? e : pi::kMmAxpyMinBatch);
}
// Rows of an activation buffer (h, a): B, or the padded batch 16 * nbt when the
// matrix-core kernels keep it neuron-major (a in fp16 also pads the neurons to 32).
size_t act_rows(int32_t B) {
  if (!use_mm_row(B)) return (size_t)B;
  const size_t p = (size_t)16 * pi::mm_nbt(B);
  return p > (size_t)B ? p : (size_t)B;
}
size_t act_bytes(int32_t B, int32_t n) {
  const size_t n1 = (size_t)(n > 0 ? n : 1);
  const size_t f32 = act_rows(B) * n1 * 4, f16 = act_rows(B) * ((n1 + 31) / 32 * 32) * 2;
  return f32 > f16 ? f32 : f16;
}
// h: [B x H] fp32, neuron-major fp32, or two fp16 parts (hi, then lo) in the fp16 layout
size_t h_bytes(int32_t B, int32_t H) {
  const size_t f32 = act_rows(B) * (size_t)H * 4, f16 = 2 * act_rows(B) * (((size_t)H + 31) / 32 * 32) * 2;
  return f32 > f16 ? f32 : f16;
}
float* h_lo_part(float* h, int32_t B, int32_t H) {
  return reinterpret_cast<float*>(reinterpret_cast<char*>(h) + act_rows(B) * (((size_t)H + 31) / 32 * 32) * 2);
}
size_t mm_row_partial_bytes(int32_t B, int64_t rows, int64_t cols, bool gated) {
  if (!use_mm_row(B) || rows <= 0 || cols <= 0) return 0;
  int ks = pi::mm_row16_ks(rows, cols, pi::mm_nbt(B), gated);
  const int kh = pi::mm_row16_ks(rows, cols, pi::mm_nbt(B), false, true);
  ks = kh > ks ? kh : ks;
  for (int dt = 0; dt < 3; ++dt) {
    const int k = pi::mm_row_ks(dt, rows, cols);
    ks = k > ks ? k : ks;
  }
  return (size_t)(gated ? 2 : 1) * ks * (size_t)rows * 16 * pi::mm_nbt(B) * 4;
}
size_t mm_axpy_partial_bytes(int32_t B, int64_t rows, int64_t cols) {
  if (!use_mm_axpy(B) || rows <= 0 || cols <= 0) return 0;
  int rc = 1;
  for (int dt = 0; dt < 2; ++dt) {
    const int r = pi::mm_axpy_row_chunks(dt, pi::mm_nbt(B), rows, cols);
    rc = r > rc ? r : rc;
  }
  return (size_t)rc * B * (size_t)cols * 4;
}
size_t max3(size_t a, size_t b, size_t c) { return a > b ? (a > c ? a : c) : (b > c ? b : c); }

// FC1 -> a, FC2 partials (VALU row chunks or matrix-core row chunks) -> y.
size_t ffn_partial_bytes(int32_t B, int32_t d, int32_t n_g) {
  return max3((size_t)pi::fc2_chunks(B) * B * (size_t)d * 4, mm_row_partial_bytes(B, n_g, d, true),
              mm_axpy_partial_bytes(B, n_g, d));
}

FfnWs ffn_ws_layout(void* ws, int32_t B, int32_t d, int32_t n_g) {
  Carver c{static_cast<char*>(ws)};
  FfnWs w{};
  w.a = c.take<float>(act_bytes(B, n_g));
  w.partials = c.take<float>(ffn_partial_bytes(B, d, n_g));
  w.bytes = c.off;
  return w;
}

// Partial sums of the predictor output layer over its hidden-major rows (the
// separate kernels: batch > 1, or more hidden units than the batch-1 kernel
// compacts).
// (the batch-1 kernel addresses P2 with 32-bit offsets: H * N * 4 bytes bounds any dtype)
bool out_layer_needs_partials(int32_t B, int32_t H, int32_t N) {
  return B > 1 || H > pi::kMaxHiddenB1 || (int64_t)H * N * 4 >= ((int64_t)1 << 31);
}
size_t out_partials_bytes(int32_t B, int32_t H, int32_t N) {
  if (!out_layer_needs_partials(B, H, N)) return 0;
  const size_t v = (size_t)pi::fc2_chunks(B) * B * (size_t)N * 4, m = mm_axpy_partial_bytes(B, H, N);
  return v > m ? v : m;
}
// Predictor scratch: the output layer's partials, or the hidden layer's split-K partials.
size_t pred_partial_bytes(int32_t B, int32_t d, int32_t H, int32_t N) {
  const size_t o = out_partials_bytes(B, H, N), r = mm_row_partial_bytes(B, H, d, false);
  return o > r ? o : r;
}

size_t table_words(int32_t N) { return 2 * (size_t)((N + 63) / 64); }
size_t n_groups64(int32_t N) { return (size_t)((N + 63) / 64); }

// Fused layer workspace: h, logits scratch, activation words, the per-64-id
// group segments of the batch-1 path, a, and the partial sums (FC2 chunks,
// or the output layer's when those are larger).
struct LayerWs {
  float* h;
  float* logits;
  uint32_t* mask;
  int32_t* seg_slot;
  int32_t* seg_cold;
  int32_t* pos_slot;
  float* pos_a;
  uint32_t* cnt;
  float* a;
  float* partials;
  size_t bytes;
};

LayerWs layer_ws_layout(void* ws, int32_t B, int32_t d, int32_t H, int32_t N, int32_t n_g) {
  Carver c{static_cast<char*>(ws)};
  LayerWs w{};
  const size_t ng = n_groups64(N);
  w.h = c.take<float>(h_bytes(B, H));
  w.logits = c.take<float>((size_t)B * N * 4);
  w.mask = c.take<uint32_t>(table_words(N) * 4);
  w.seg_slot = c.take<int32_t>(ng * 64 * 4);
  w.seg_cold = c.take<int32_t>(ng * 64 * 4);
  w.pos_slot = c.take<int32_t>(ng * 64 * 4);
  w.pos_a = c.take<float>(ng * 64 * 4);
  w.cnt = c.take<uint32_t>(ng * 4);
  w.a = c.take<float>(act_bytes(B, n_g));
  const size_t pb = ffn_partial_bytes(B, d, n_g);
  const size_t seg = (size_t)pi::kSegChunks * (size_t)d * 4;
  w.partials = c.take<float>(max3(pb, seg, pred_partial_bytes(B, d, H, N)));
  w.bytes = c.off;
  return w;
}

// pi_ffn_layer_normed's workspace: the layer's, then the normalisation statistics and the
// normalised input (used when the layer does not run the batch-1 kernels).
struct NormedWs {
  void* layer;
  size_t layer_bytes;
  float* stats;
  float* xn;
  size_t bytes;
};

NormedWs normed_ws_layout(void* ws, int32_t B, int32_t d, int32_t H, int32_t N, int32_t n_g) {
  NormedWs n{};
  n.layer = ws;
  n.layer_bytes = layer_ws_layout(nullptr, B, d, H, N, n_g).bytes;
  Carver c{static_cast<char*>(ws)};
  c.off = n.layer_bytes;
  n.stats = c.take<float>(256);
  n.xn = c.take<float>((size_t)(B > 0 ? B : 1) * (size_t)d * 4);
  n.bytes = c.off;
  return n;
}

// The predictor's hidden layer, h[b,m] = max(0, P1[m].x_b + c1[m]): batch 1 on the
// register-x GEMV, batches of kMmRowMinBatch and more on the matrix cores (split-K
// partials in `partials`), others on the LDS-x row-dot kernel.
// Layout of h between the two predictor layers: 0 [B x H]; 1 neuron-major fp32
// ([H x 16 nbt]) between the two matrix-core layers; 2 two fp16 parts in the fp16
// layout when the output layer runs on the fp16 matrix cores (fp16 P2).
int h_layout(int32_t B, int32_t d, int32_t H, int32_t N, const pi_matrix& P1, const pi_matrix& P2) {
  if (!(use_mm_row(B) && use_mm_axpy(B) && pi::mm_rowdot_supported(P1.dtype, H, d) &&
        pi::mm_axpy_supported(P2.dtype, H, N)))
    return 0;
  return pi::mm_axpy16_supported(P2.dtype, N) ? 2 : 1;
}

// The chained-layer input of pi_ffn_layer_normed when the batch-1 kernels normalise it themselves:
// the hidden-layer kernel computes the statistics and leaves them in `stats` for the output-layer +
// FC1 kernel.
struct LnIn {
  float eps;
  float* stats;    // 2 floats in the workspace
  float* x_out;    // optional normalised row
};

int enqueue_hidden(hipStream_t s, int32_t B, int32_t d, int32_t H, const float* x, const pi_matrix& P1,
                   const pi_vector& c1, float* h, float* partials, int h_lay, const LnIn* ln = nullptr) {
  const bool h_tr = h_lay != 0;
  // batch 1: x staged once per workgroup in LDS, normalised there first when ln is given
  if (B == 1 && pi::hidden_lds_supported(P1.dtype, d)) {
    pi::B1Gemv g{};
    g.W = P1.data; g.Ws = P1.scales; g.dt = P1.dtype; g.rows = H; g.cols = d; g.x = x;
    g.bias = c1.data; g.bias_dt = c1.dtype; g.out = h;
    if (ln) { g.ln_stats = ln->stats; g.ln_eps = ln->eps; g.x_out = ln->x_out; }
    return hip_status(pi::launch_hidden_lds(g, s));
  }
  if (ln) return PI_EINVAL;   // only the batch-1 kernel normalises its input
  if (use_mm_row(B) && pi::mm_rowdot_supported(P1.dtype, H, d)) {
    pi::MmRowArgs m{};
    m.W = P1.data; m.Ws = P1.scales; m.dt = P1.dtype; m.gated = 0; m.cols = d; m.n_rows = H; m.list = nullptr;
    m.count_dev = nullptr; m.count_max = H; m.x = x; m.B = B; m.nbt = pi::mm_nbt(B);
    // fp16 P1: the fp16 matrix cores with x in two fp16 parts (the logits keep near-fp32 precision)
    m.x_hilo = P1.dtype == PI_F16;
    m.ks = m.x_hilo ? pi::mm_row16_ks(H, d, m.nbt, false, true) : pi::mm_row_ks(P1.dtype, H, d);
    m.kc = pi::mm_row_kc(P1.dtype, d, m.ks); m.partials = partials;
    m.bias = c1.data; m.bias_dt = c1.dtype; m.relu = 1; m.out = h; m.out_tr = h_tr;
    m.out_h8 = h_lay == 2; m.out_lo = h_lay == 2 ? h_lo_part(h, B, H) : nullptr;
    m.out_stride = h_tr ? 16 * m.nbt : H;
    return hip_status(pi::launch_mm_rowdot(m, s));
  }
  pi::RowdotArgs a{};
  a.W = P1.data; a.Ws = P1.scales; a.dt = P1.dtype; a.cols = d;
  a.count_max = H; a.x = x; a.B = B; a.bias = c1.data; a.bias_dt = c1.dtype;
  a.relu = 1; a.out = h; a.out_stride = H;
  return hip_status(pi::launch_rowdot(a, s));
}

// The predictor's output layer, logits[b,i] = c2[i] + sum_m h[b,m] P2[m,i] with P2
// hidden-major, and the activation words when mask != NULL.  Batch 1 (H within
// the compaction bound): one tile kernel that reads only the rows of positive
// hidden units.  Otherwise: the neuron-major axpy over every row, the ordered
// sum with c2, then the words from the stored logits.
int enqueue_output_layer(hipStream_t s, int32_t B, int32_t H, int32_t N, const float* h, const pi_matrix& P2,
                         const pi_vector& c2, float tau, float* logits, uint32_t* mask, float* partials,
                         int32_t* rows_read = nullptr, int h_lay = 0) {
  if (!out_layer_needs_partials(B, H, N)) {
    pi::PredFc1Args a{};
    a.P2 = P2.data; a.P2s = P2.scales; a.pdt = P2.dtype; a.H = H; a.N = N; a.h = h;
    a.c2 = c2.data; a.c2_dt = c2.dtype; a.tau = tau; a.logits = logits; a.mask = mask; a.rows_read = rows_read;
    return hip_status(pi::launch_pred_out_b1(a, s));
  }
  int st, chunks;
  if (use_mm_axpy(B) && pi::mm_axpy_supported(P2.dtype, H, N)) {
    pi::MmAxpyArgs m{};
    m.W = P2.data; m.Ws = P2.scales; m.dt = P2.dtype; m.cols = N; m.n_rows = H; m.list = nullptr;
    m.count_dev = nullptr; m.count_max = H; m.a = h; m.a_stride = H; m.a_by_row = 1; m.a_tr = h_lay != 0; m.B = B;
    m.a_h8 = h_lay == 2; m.a_lo = h_lay == 2 ? h_lo_part(const_cast<float*>(h), B, H) : nullptr;
    m.nbt = pi::mm_nbt(B);
    m.row_chunks = pi::mm_axpy_row_chunks(P2.dtype, pi::mm_nbt(B), H, N);
    m.partials = partials;
    if (m.a_h8) {
      // every hidden unit in one block per 128 logits: logits, c2 and the words in the same launch
      m.row_chunks = 1; m.rows_per_chunk = pi::mm_axpy_rows_per_chunk(m);
      m.final_out = logits; m.bias = c2.data; m.bias_dt = c2.dtype; m.tau = tau; m.mask = mask;
      return hip_status(pi::launch_mm_axpy(m, s));
    }
    m.rows_per_chunk = pi::mm_axpy_rows_per_chunk(m);
    st = hip_status(pi::launch_mm_axpy(m, s));
    chunks = m.row_chunks;
  } else {
    pi::Fc2Args f{};
    f.W2 = P2.data; f.W2s = P2.scales; f.dt = P2.dtype; f.d = N; f.n_g = H; f.list = nullptr; f.K = nullptr;
    f.a = h; f.a_stride = H; f.a_by_row = 1; f.B = B; f.partials = partials;
    st = hip_status(pi::launch_fc2(f, s));
    chunks = pi::fc2_chunks(B);
  }
  if (st != PI_OK) return st;
  pi::ReduceArgs r{};
  r.partials = partials; r.chunks = chunks; r.B = B; r.d = N; r.y = logits;
  r.y_c = nullptr; r.K_c = nullptr; r.b2 = c2.data; r.b2_dt = c2.dtype;
  return hip_status(mask ? pi::launch_reduce_mask(r, tau, mask, s) : pi::launch_reduce(r, s));
}

}  // namespace

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
  if (B < 1) B = 1;
  switch (op) {
    case PI_OP_PREDICT:
      return H > 0 && N > 0 && d > 0 ? align_up(h_bytes(B, H)) + pred_partial_bytes(B, d, H, N) : 0;
    case PI_OP_PREDICT_OUTPUT: return H > 0 && N > 0 ? out_partials_bytes(B, H, N) : 0;
    case PI_OP_SPARSE_FFN:
      return d > 0 ? ffn_ws_layout(nullptr, B, d, n_g).bytes : 0;
    case PI_OP_FFN_LAYER:
      return (d > 0 && N > 0) ? layer_ws_layout(nullptr, B, d, H > 0 ? H : 1, N, n_g).bytes : 0;
    case PI_OP_FFN_LAYER_NORMED:
      return (d > 0 && N > 0) ? normed_ws_layout(nullptr, B, d, H > 0 ? H : 1, N, n_g).bytes : 0;
    default: return 0;
  }
}

size_t pi_table_bytes(int32_t N) { return N > 0 ? (table_words(N) + n_groups64(N)) * 4 : 0; }

int pi_table_prepare(int32_t N, const int32_t* T_g, int32_t n_g, void* table, size_t table_bytes) {
  if (N <= 0 || n_g < 0 || n_g > N || !table || (n_g > 0 && !T_g)) return PI_EINVAL;
  if (table_bytes < pi_table_bytes(N)) return PI_EWORKSPACE;
  const size_t W = table_words(N);
  uint32_t* bits = static_cast<uint32_t*>(table);
  for (int32_t s = 0; s < n_g; ++s) {
    if (T_g[s] < 0 || T_g[s] >= N || (s > 0 && T_g[s] <= T_g[s - 1])) return PI_EINVAL;
  }
  memset(bits, 0, W * 4);
  for (int32_t s = 0; s < n_g; ++s) bits[T_g[s] / 32] |= 1u << (T_g[s] % 32);
  int32_t* pre = reinterpret_cast<int32_t*>(bits + W);
  int32_t run = 0;
  for (size_t b = 0; b < W / 2; ++b) {  // 64-id groups
    pre[b] = run;
    run += __builtin_popcount(bits[2 * b]) + __builtin_popcount(bits[2 * b + 1]);
  }
  return PI_OK;
}

int pi_predict(void* stream, int32_t B, int32_t d, int32_t H, int32_t N, const float* x, pi_matrix P1,
               pi_vector c1, pi_matrix P2, pi_vector c2, float* logits, void* ws, size_t ws_bytes) {
  if (!valid_batch(B) || d <= 0 || H <= 0 || N <= 0) return PI_EINVAL;
  if (!x || !aligned16(x) || !logits || !valid_matrix(P1, d) || !valid_matrix(P2, N)) return PI_EINVAL;
  if (!valid_vector(c1) || !valid_vector(c2)) return PI_EINVAL;
  if (!ws || !aligned16(ws)) return ws_bytes ? PI_EINVAL : PI_EWORKSPACE;
  if (ws_bytes < pi_workspace_bytes(PI_OP_PREDICT, B, d, H, N, 0)) return PI_EWORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* h = static_cast<float*>(ws);
  float* partials = reinterpret_cast<float*>(static_cast<char*>(ws) + align_up(h_bytes(B, H)));
  const int h_lay = h_layout(B, d, H, N, P1, P2);
  const int st = enqueue_hidden(s, B, d, H, x, P1, c1, h, partials, h_lay);
  if (st != PI_OK) return st;
  return enqueue_output_layer(s, B, H, N, h, P2, c2, 0.f, logits, nullptr, partials, nullptr, h_lay);
}

int pi_predict_output(void* stream, int32_t B, int32_t H, int32_t N, const float* h, pi_matrix P2, pi_vector c2,
                      float tau, float* logits, uint32_t* mask, void* ws, size_t ws_bytes) {
  if (!valid_batch(B) || H <= 0 || N <= 0 || !h || !aligned16(h) || !valid_matrix(P2, N) || !valid_vector(c2))
    return PI_EINVAL;
  if (!logits && (B != 1 || !mask)) return PI_EINVAL;
  const size_t need = pi_workspace_bytes(PI_OP_PREDICT_OUTPUT, B, 0, H, N, 0);
  if (need && (!ws || !aligned16(ws))) return PI_EWORKSPACE;
  if (ws_bytes < need) return PI_EWORKSPACE;
  if (!logits && out_layer_needs_partials(B, H, N)) return PI_EINVAL;
  return enqueue_output_layer(static_cast<hipStream_t>(stream), B, H, N, h, P2, c2, tau, logits, mask,
                              static_cast<float*>(ws));
}

int pi_compact(void* stream, int32_t B, int32_t N, const float* logits, float tau, const int32_t* T_g,
               int32_t n_g, int32_t* A_g, int32_t* K, const int32_t* T_c, int32_t n_c, int32_t* A_c,
               int32_t* K_c, void* ws, size_t ws_bytes) {
  (void)ws; (void)ws_bytes;
  if (!valid_batch(B) || N <= 0 || n_g < 0 || !logits || !K) return PI_EINVAL;
  if (n_g > 0 && (!T_g || !A_g)) return PI_EINVAL;
  if (T_c && (n_c < 0 || !A_c || !K_c)) return PI_EINVAL;
  if (N > PI_MAX_NEURONS) return PI_EUNSUPPORTED;
  if (!T_c) n_c = 0;
  return hip_status(pi::launch_compact(B, N, logits, tau, T_g, n_g, A_g, K, T_c, n_c, A_c, K_c,
                                       static_cast<hipStream_t>(stream)));
}

namespace {

int validate_ffn(int32_t B, int32_t d, int32_t n_g, int32_t kind, const float* x, const pi_matrix& W1,
                 const pi_vector& b1, const pi_matrix& Wup, const pi_matrix& W2) {
  if (!valid_batch(B) || d <= 0 || n_g < 0) return PI_EINVAL;
  if (kind != PI_RELU && kind != PI_GATED_RELU) return PI_EINVAL;
  if (!x || !aligned16(x)) return PI_EINVAL;
  if (!valid_matrix(W1, d) || !valid_matrix(W2, d) || !valid_vector(b1)) return PI_EINVAL;
  if (kind == PI_GATED_RELU) {
    if (!valid_matrix(Wup, d)) return PI_EINVAL;
    if (Wup.dtype != W1.dtype) return PI_EUNSUPPORTED;
  }
  if (W2.dtype != W1.dtype) return PI_EUNSUPPORTED;
  return PI_OK;
}

// FC1 over a given list, then FC2 partials, then the ordered reduction + merge.
// ev (optional, 2 entries) is recorded after FC1 and after FC2.
int enqueue_ffn(hipStream_t s, int32_t B, int32_t d, int32_t n_g, int32_t kind, const float* x, const pi_matrix& W1,
                const pi_vector& b1, const pi_matrix& Wup, const pi_matrix& W2, const int32_t* A_g, const int32_t* K,
                float* a, float* partials, float* y, const float* y_c, const int32_t* K_c, const pi_vector& b2,
                const hipEvent_t* ev, uint32_t stages) {
  const bool gated = kind == PI_GATED_RELU;
  int st = PI_OK;
  const bool mm1 = use_mm_row(B) && pi::mm_rowdot_supported(W1.dtype, n_g, d);
  const bool mm2 = use_mm_axpy(B) && n_g > 0 && pi::mm_axpy_supported(W2.dtype, n_g, d);
  const bool a_tr = mm1 && mm2;      // a kept neuron-major between the two matrix-core GEMMs
  const bool a16 = a_tr && pi::mm_axpy16_supported(W2.dtype, d);   // ... in fp16, for the fp16 FC2
  if (stages & PI_STAGE_FC1) {
    if (mm1) {
      pi::MmRowArgs m{};
      m.W = W1.data; m.Ws = W1.scales; m.dt = W1.dtype; m.gated = gated;
      if (gated) { m.Wup = Wup.data; m.Wups = Wup.scales; }
      m.cols = d; m.n_rows = n_g; m.list = A_g; m.count_dev = K; m.count_max = n_g; m.x = x; m.B = B;
      m.nbt = pi::mm_nbt(B); m.x_f16 = W1.dtype == PI_F16;
      m.ks = m.x_f16 ? pi::mm_row16_ks(n_g, d, m.nbt, gated) : pi::mm_row_ks(W1.dtype, n_g, d);
      m.kc = pi::mm_row_kc(W1.dtype, d, m.ks);
      m.partials = partials; m.bias = b1.data; m.bias_dt = b1.dtype; m.relu = 1; m.out = a; m.out_tr = a_tr;
      m.out_h8 = a16; m.out_stride = a_tr ? 16 * m.nbt : (n_g > 0 ? n_g : 1);
      st = n_g > 0 ? hip_status(pi::launch_mm_rowdot(m, s)) : PI_OK;
    } else if (B == 1 && pi::b1_supported(W1.dtype, d)) {
      pi::B1Gemv g{};
      g.W = W1.data; g.Ws = W1.scales; g.dt = W1.dtype; g.rows = n_g; g.cols = d; g.x = x;
      if (gated) { g.Wu = Wup.data; g.Wus = Wup.scales; }
      g.bias = b1.data; g.bias_dt = b1.dtype; g.out = a; g.list = A_g; g.Kp = K;
      st = n_g > 0 ? hip_status(pi::launch_fc1_b1(g, gated, s)) : PI_OK;
    } else {
      pi::RowdotArgs r{};
      r.W = W1.data; r.Ws = W1.scales; r.dt = W1.dtype; r.cols = d; r.gated = gated;
      if (gated) { r.Wup = Wup.data; r.Wups = Wup.scales; }
      r.list = A_g; r.count_dev = K; r.count_max = n_g;
      r.x = x; r.B = B; r.bias = b1.data; r.bias_dt = b1.dtype; r.relu = 1;
      r.out = a; r.out_stride = n_g > 0 ? n_g : 1;
      st = hip_status(pi::launch_rowdot_ex(r, n_g, nullptr, 0, s));
    }
    if (st != PI_OK) return st;
  }
  if (ev && ev[0] && (st = hip_status(hipEventRecord(ev[0], s))) != PI_OK) return st;
  const int chunks2 = mm2 ? pi::mm_axpy_row_chunks(W2.dtype, pi::mm_nbt(B), n_g, d) : pi::fc2_chunks(B);
  if (stages & PI_STAGE_FC2) {
    if (mm2) {
      pi::MmAxpyArgs m{};
      m.W = W2.data; m.Ws = W2.scales; m.dt = W2.dtype; m.cols = d; m.n_rows = n_g; m.list = A_g; m.count_dev = K;
      m.count_max = n_g; m.a = a; m.a_stride = n_g; m.a_by_row = 0; m.a_tr = a_tr; m.a_h8 = a16; m.B = B;
      m.nbt = pi::mm_nbt(B); m.row_chunks = chunks2; m.rows_per_chunk = pi::mm_axpy_rows_per_chunk(m);
      m.partials = partials;
      if ((st = hip_status(pi::launch_mm_axpy(m, s))) != PI_OK) return st;
    } else {
      pi::Fc2Args f{};
      f.W2 = W2.data; f.W2s = W2.scales; f.dt = W2.dtype; f.d = d; f.n_g = n_g;
      f.list = A_g; f.K = K; f.a = a; f.a_stride = n_g; f.a_by_row = 0; f.B = B; f.partials = partials;
      if ((st = hip_status(pi::launch_fc2(f, s))) != PI_OK) return st;
    }
  }
  if (ev && ev[1] && (st = hip_status(hipEventRecord(ev[1], s))) != PI_OK) return st;
  if (stages & PI_STAGE_SUM) {
    pi::ReduceArgs r{};
    r.partials = partials; r.chunks = chunks2; r.B = B; r.d = d; r.y = y;
    r.y_c = y_c; r.K_c = K_c; r.b2 = b2.data; r.b2_dt = b2.dtype;
    st = hip_status(pi::launch_reduce(r, s));
  }
  return st;
}

}  // namespace

int pi_sparse_ffn(void* stream, int32_t B, int32_t d, int32_t n_g, int32_t kind, const float* x, pi_matrix W1,
                  pi_vector b1, pi_matrix Wup, pi_matrix W2, const int32_t* A_g, const int32_t* K, float* y_g,
                  void* ws, size_t ws_bytes) {
  int st = validate_ffn(B, d, n_g, kind, x, W1, b1, Wup, W2);
  if (st != PI_OK) return st;
  if (!y_g || !aligned16(y_g) || !K || (n_g > 0 && !A_g)) return PI_EINVAL;
  if (!ws || !aligned16(ws)) return PI_EWORKSPACE;
  const FfnWs w = ffn_ws_layout(ws, B, d, n_g);
  if (ws_bytes < w.bytes) return PI_EWORKSPACE;
  return enqueue_ffn(static_cast<hipStream_t>(stream), B, d, n_g, kind, x, W1, b1, Wup, W2, A_g, K, w.a, w.partials,
                     y_g, nullptr, nullptr, pi_vector{nullptr, PI_F32}, nullptr, PI_STAGE_ALL);
}

int pi_merge(void* stream, int32_t B, int32_t d, float* y, const float* y_c, const int32_t* K_c, pi_vector b2) {
  if (!valid_batch(B) || d <= 0 || !y || !valid_vector(b2)) return PI_EINVAL;
  if (!y_c && !b2.data) return PI_OK;  // nothing to add
  return hip_status(pi::launch_merge(B, d, y, y_c, K_c, b2.data, b2.dtype, static_cast<hipStream_t>(stream)));
}

int pi_layer_norm(void* stream, int32_t B, int32_t d, const float* y, float eps, float* x) {
  if (B <= 0 || d <= 0 || d > (1 << 30) || !y || !x || !(eps >= 0.f) || !std::isfinite(eps)) return PI_EINVAL;
  const uintptr_t nb = (uintptr_t)B * (uintptr_t)d * sizeof(float);
  const uintptr_t xa = reinterpret_cast<uintptr_t>(x), ya = reinterpret_cast<uintptr_t>(y);
  if (xa != ya && xa < ya + nb && ya < xa + nb) return PI_EINVAL;   // partial overlap
  return hip_status(pi::launch_layer_norm(B, d, y, eps, x, static_cast<hipStream_t>(stream)));
}

namespace {

// pi_attn_decode's workspace: g, q, the flags, the head logits, the chunk partials and the
// heads' output-projection contributions.
struct AttnWs {
  float* g;
  float* q;
  int32_t* flag;
  float* hlogit;
  float* part;
  float* ypart;
  size_t bytes;
};

AttnWs attn_ws_layout(void* ws, const pi_attn& A) {
  Carver c{static_cast<char*>(ws)};
  AttnWs w{};
  w.g = c.take<float>((size_t)A.Ha * 4);
  w.q = c.take<float>((size_t)A.d * 4);
  w.flag = c.take<int32_t>((size_t)A.n_heads * 4);
  w.hlogit = c.take<float>((size_t)A.n_heads * 4);
  w.part = c.take<float>((size_t)A.n_heads * pi::attn_chunks(A.L_max) * (A.dh + 2) * 4);
  w.ypart = c.take<float>((size_t)A.n_heads * A.d * 4);
  w.bytes = c.off;
  return w;
}

bool f16_matrix(const pi_matrix& m) { return m.data && m.dtype == PI_F16 && aligned16(m.data); }
bool f16_bias(const pi_vector& v) { return !v.data || v.dtype == PI_F16; }

}  // namespace

size_t pi_attn_workspace_bytes(const pi_attn* A) {
  if (!A || A->d <= 0 || A->n_heads <= 0 || A->dh <= 0 || A->Ha <= 0 || A->L_max <= 0) return 0;
  return attn_ws_layout(nullptr, *A).bytes;
}

int pi_attn_decode(void* stream, const pi_attn* A, int32_t t, const float* x, float tau, float* y,
                   float* head_logits, int32_t* heads, int32_t* n_active, void* ws, size_t ws_bytes) {
  if (!A || !x || !y || !heads || !n_active || !aligned16(x) || !aligned16(y)) return PI_EINVAL;
  if (A->d <= 0 || A->n_heads <= 0 || A->dh <= 0 || A->Ha <= 0 || A->L_max <= 0 ||
      (int64_t)A->n_heads * A->dh != A->d || t < 0 || t >= A->L_max)
    return PI_EINVAL;
  if (!pi::attn_supported(A->d, A->n_heads, A->dh, A->Ha)) return PI_EUNSUPPORTED;
  if (!f16_matrix(A->Pa1) || !f16_matrix(A->Pa2) || !f16_matrix(A->Wq) || !f16_matrix(A->Wk) ||
      !f16_matrix(A->Wv) || !f16_matrix(A->WoT) || !f16_bias(A->ca1) || !f16_bias(A->ca2) || !f16_bias(A->bq) ||
      !f16_bias(A->bk) || !f16_bias(A->bv) || !f16_bias(A->bo) || !A->Kc || !A->Vc || !aligned16(A->Kc) ||
      !aligned16(A->Vc))
    return PI_EINVAL;
  // the cache rows of a head are addressed with 32-bit offsets
  if ((int64_t)A->L_max * A->dh * 2 >= ((int64_t)1 << 31)) return PI_EUNSUPPORTED;
  if (ranges_overlap(x, (size_t)A->d * 4, y, (size_t)A->d * 4)) return PI_EINVAL;
  if (!ws || !aligned16(ws)) return PI_EWORKSPACE;
  const AttnWs w = attn_ws_layout(ws, *A);
  if (ws_bytes < w.bytes) return PI_EWORKSPACE;
  pi::AttnArgs a{};
  a.d = A->d; a.n_heads = A->n_heads; a.dh = A->dh; a.Ha = A->Ha; a.L_max = A->L_max; a.t = t;
  a.n_chunks = pi::attn_chunks(A->L_max); a.tau = tau; a.x = x;
  a.Pa1 = A->Pa1.data; a.ca1 = A->ca1.data; a.Pa2 = A->Pa2.data; a.ca2 = A->ca2.data;
  a.Wq = A->Wq.data; a.bq = A->bq.data; a.Wk = A->Wk.data; a.bk = A->bk.data; a.Wv = A->Wv.data; a.bv = A->bv.data;
  a.WoT = A->WoT.data; a.bo = A->bo.data; a.Kc = A->Kc; a.Vc = A->Vc;
  a.g = w.g; a.q = w.q; a.flag = w.flag; a.hlogit = w.hlogit; a.part = w.part; a.ypart = w.ypart;
  a.y = y; a.logits_out = head_logits; a.heads = heads; a.n_active = n_active;
  return hip_status(pi::launch_attn(a, static_cast<hipStream_t>(stream)));
}

int pi_read_probe(void* stream, const void* buf, size_t bytes, int32_t blocks, int32_t depth, uint32_t* out) {
  if (!buf || !out || bytes == 0 || bytes % 16 != 0 || !aligned16(buf) || blocks > 65536) return PI_EINVAL;
  if (depth == 0) depth = PI_READ_PROBE_DEPTH;
  if (depth != 4 && depth != 8 && depth != 16 && depth != 32) return PI_EINVAL;
  if (blocks <= 0) blocks = PI_READ_PROBE_BLOCKS_PER_CU * pi::kNumCU;
  return hip_status(pi::launch_read_probe(buf, (int64_t)bytes, blocks, depth, out, static_cast<hipStream_t>(stream)));
}

namespace {

// The next layer's predictor hidden layer, computed ahead on this layer's input.
struct Ahead {
  const pi_layer* next;
  float* h;              // next's h in its workspace
  float* partials;       // next's predictor partials in its workspace
  int h_lay;
};

// The batch-1 layer runs as the fused tile kernels (output layer + decision + FC1, then the segment
// FC2 and the ordered sum) for these formats and sizes; its hidden layer takes the register-x
// kernel when the predictor's rows fit it and the LDS-x row-dot otherwise.
bool b1_fused(const pi_layer* L, int32_t B) {
  const bool gated = L->kind == PI_GATED_RELU;
  const int bdt = L->b1.data ? L->b1.dtype : (L->c2.data ? L->c2.dtype : PI_F16);
  const int c2dt = L->c2.data ? L->c2.dtype : bdt;
  return B == 1 && n_groups64(L->N) <= (size_t)64 * pi::kSegChunks &&
         pi::pred_fc1_supported(L->P2.dtype, L->W1.dtype, bdt, c2dt, gated, L->H, L->N, L->d);
}

int layer_stages(void* stream, const pi_layer* L, int32_t B, const float* x, float tau, const float* y_c, float* y,
                 float* logits, int32_t* A_g, int32_t* K, int32_t* A_c, int32_t* K_c, void* ws, size_t ws_bytes,
                 void* const* events, uint32_t stages, int32_t* rows_read, const Ahead* ah,
                 const LnIn* ln = nullptr) {
  if (!L) return PI_EINVAL;
  const int32_t d = L->d, N = L->N, H = L->H, n_g = L->n_g;
  if (N <= 0 || H <= 0 || n_g > N) return PI_EINVAL;
  if (N > PI_MAX_NEURONS) return PI_EUNSUPPORTED;
  if (stages == 0 || (stages & ~(uint32_t)PI_STAGE_ALL)) return PI_EINVAL;
  int st = validate_ffn(B, d, n_g, L->kind, x, L->W1, L->b1, L->Wup, L->W2);
  if (st != PI_OK) return st;
  if (!valid_matrix(L->P1, d) || !valid_matrix(L->P2, N) || !valid_vector(L->c1) || !valid_vector(L->c2) ||
      !valid_vector(L->b2))
    return PI_EINVAL;
  if (!L->table || !y || !aligned16(y) || !K || (n_g > 0 && !A_g)) return PI_EINVAL;
  if (L->cold && (!A_c || !K_c)) return PI_EINVAL;
  if (!ws || !aligned16(ws)) return PI_EWORKSPACE;
  const LayerWs w = layer_ws_layout(ws, B, d, H, N, n_g);
  if (ws_bytes < w.bytes) return PI_EWORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipEvent_t ev[6] = {nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};
  if (events)
    for (int i = 0; i < 6; ++i) ev[i] = static_cast<hipEvent_t>(events[i]);
  auto record = [&](int i) { return ev[i] ? hip_status(hipEventRecord(ev[i], s)) : PI_OK; };
  auto want = [&](uint32_t bit) { return (stages & bit) != 0; };

  const bool gated = L->kind == PI_GATED_RELU;
  const int32_t ngroups = (int32_t)n_groups64(N);
  const int bdt = L->b1.data ? L->b1.dtype : (L->c2.data ? L->c2.dtype : PI_F16);
  const bool fused = b1_fused(L, B);
  if (ln && (!fused || !pi::hidden_lds_supported(L->P1.dtype, d) || stages != PI_STAGE_ALL || ah)) return PI_EINVAL;
  float* lg = logits ? logits : w.logits;

  if ((st = record(0)) != PI_OK) return st;
  // predictor hidden layer
  const int h_lay = h_layout(B, d, H, N, L->P1, L->P2);
  if (want(PI_STAGE_HIDDEN) &&
      (st = enqueue_hidden(s, B, d, H, x, L->P1, L->c1, w.h, w.partials, h_lay, ln)) != PI_OK)
    return st;
  if ((st = record(1)) != PI_OK) return st;

  if (fused) {
    // output layer + activation decision + FC1 per tile -> FC2 over the non-zero
    // rows + lists -> ordered sum + merge
    if (want(PI_STAGE_OUTPUT) || want(PI_STAGE_FC1)) {
      pi::PredFc1Args a{};
      a.P2 = L->P2.data; a.P2s = L->P2.scales; a.pdt = L->P2.dtype; a.H = H; a.N = N; a.h = w.h;
      a.c2 = L->c2.data; a.c2_dt = L->c2.dtype; a.tau = tau; a.logits = logits; a.mask = nullptr;
      a.gbits = static_cast<const uint32_t*>(L->table);
      a.gpre = reinterpret_cast<const int32_t*>(a.gbits + table_words(N));
      a.W1 = L->W1.data; a.W1s = L->W1.scales; a.Wu = L->Wup.data; a.Wus = L->Wup.scales; a.dt = L->W1.dtype;
      a.d = d; a.n_g = n_g; a.x = x; a.ln_stats = ln ? ln->stats : nullptr; a.b1 = L->b1.data; a.b1_dt = L->b1.dtype;
      a.seg_slot = w.seg_slot; a.seg_cold = w.seg_cold; a.pos_slot = w.pos_slot; a.pos_a = w.pos_a; a.cnt = w.cnt;
      a.rows_read = rows_read;
      // the next layer's hidden layer rides in this launch when its rows have the FC1 weights' format
      if (ah && ah->h_lay == 0 && ah->next->P1.dtype == L->W1.dtype &&
          (!ah->next->c1.data || ah->next->c1.dtype == bdt)) {
        a.nP1 = ah->next->P1.data; a.nP1s = ah->next->P1.scales; a.nc1 = ah->next->c1.data; a.nH = ah->next->H;
        a.nh = ah->h;
        ah = nullptr;
      }
      if ((st = hip_status(pi::launch_pred_fc1(a, gated, s))) != PI_OK) return st;
    }
    if ((st = record(2)) != PI_OK || (st = record(3)) != PI_OK) return st;
    if (want(PI_STAGE_FC2)) {
      pi::Fc2SegArgs f{};
      f.W2 = L->W2.data; f.W2s = L->W2.scales; f.dt = L->W2.dtype; f.d = d; f.n_g = n_g; f.ngroups = ngroups;
      f.pos_slot = w.pos_slot; f.pos_a = w.pos_a; f.seg_slot = w.seg_slot; f.seg_cold = w.seg_cold; f.cnt = w.cnt;
      f.partials = w.partials; f.A_g = A_g; f.K = K; f.A_c = L->cold ? A_c : nullptr;
      f.K_c = L->cold ? K_c : nullptr; f.n_c = N - n_g; f.rows_read = rows_read ? rows_read + 1 : nullptr;
      if ((st = hip_status(pi::launch_fc2_seg(f, s))) != PI_OK) return st;
    }
    if ((st = record(4)) != PI_OK) return st;
    if (want(PI_STAGE_SUM)) {
      pi::ReduceYArgs r{};
      r.partials = w.partials; r.d = d; r.y = y; r.y_c = y_c; r.K_c = L->cold ? K_c : nullptr;
      r.b2 = L->b2.data; r.b2_dt = L->b2.dtype;
      if ((st = hip_status(pi::launch_reduce_y(r, s))) != PI_OK) return st;
    }
    if ((st = record(5)) != PI_OK) return st;
    return ah ? enqueue_hidden(s, B, d, ah->next->H, x, ah->next->P1, ah->next->c1, ah->h, ah->partials, ah->h_lay)
              : PI_OK;
  }
  // any batch: output layer + activation words, the lists, then FC1 / FC2 / ordered sum over the list
  if (want(PI_STAGE_OUTPUT)) {
    if ((st = enqueue_output_layer(s, B, H, N, w.h, L->P2, L->c2, tau, lg, w.mask, w.partials, rows_read, h_lay)) !=
        PI_OK)
      return st;
    pi::ListCtx lc{};
    lc.mask = w.mask; lc.gbits = static_cast<const uint32_t*>(L->table); lc.W = (int)table_words(N);
    lc.A_g = A_g; lc.K = K; lc.A_c = L->cold ? A_c : nullptr; lc.K_c = L->cold ? K_c : nullptr;
    // these kernels read every hidden-major P2 row (the batch-1 tile kernel reports its own count)
    // and every listed W2 row
    lc.rows_read = rows_read; lc.rows0 = out_layer_needs_partials(B, H, N) ? H : -1;
    if ((st = hip_status(pi::launch_list(lc, n_g, s))) != PI_OK) return st;
  }
  if ((st = record(2)) != PI_OK) return st;
  st = enqueue_ffn(s, B, d, n_g, L->kind, x, L->W1, L->b1, L->Wup, L->W2, A_g, K, w.a, w.partials, y, y_c,
                   L->cold ? K_c : nullptr, L->b2, ev + 3, stages);
  if (st != PI_OK) return st;
  if ((st = record(5)) != PI_OK) return st;
  return ah ? enqueue_hidden(s, B, d, ah->next->H, x, ah->next->P1, ah->next->c1, ah->h, ah->partials, ah->h_lay)
            : PI_OK;
}

}  // namespace

int pi_ffn_layer_stages(void* stream, const pi_layer* L, int32_t B, const float* x, float tau, const float* y_c,
                        float* y, float* logits, int32_t* A_g, int32_t* K, int32_t* A_c, int32_t* K_c, void* ws,
                        size_t ws_bytes, void* const* events, uint32_t stages, int32_t* rows_read) {
  return layer_stages(stream, L, B, x, tau, y_c, y, logits, A_g, K, A_c, K_c, ws, ws_bytes, events, stages, rows_read,
                      nullptr);
}

int pi_ffn_layer_ahead(void* stream, const pi_layer* L, int32_t B, const float* x, float tau, const float* y_c,
                       float* y, float* logits, int32_t* A_g, int32_t* K, int32_t* A_c, int32_t* K_c, void* ws,
                       size_t ws_bytes, uint32_t stages, const pi_layer* next, void* ws_next, size_t ws_next_bytes) {
  if (!L || !next) return PI_EINVAL;
  if (next->d != L->d || next->H <= 0 || next->N <= 0 || next->n_g < 0 || next->n_g > next->N ||
      !valid_matrix(next->P1, next->d) || !valid_vector(next->c1))
    return PI_EINVAL;
  if (!ws_next || !aligned16(ws_next)) return PI_EWORKSPACE;
  const LayerWs wn = layer_ws_layout(ws_next, B, next->d, next->H, next->N, next->n_g);
  if (ws_next_bytes < wn.bytes) return PI_EWORKSPACE;
  // the next layer's h must not overwrite this one's workspace, and the next layer's hidden layer,
  // which may run after this layer's y is written, must still read this layer's input
  if (ranges_overlap(ws, ws_bytes, ws_next, wn.bytes)) return PI_EINVAL;
  if (L->d > 0 && valid_batch(B) && ranges_overlap(x, (size_t)B * L->d * 4, y, (size_t)B * L->d * 4)) return PI_EINVAL;
  Ahead ah{next, wn.h, wn.partials, h_layout(B, next->d, next->H, next->N, next->P1, next->P2)};
  return layer_stages(stream, L, B, x, tau, y_c, y, logits, A_g, K, A_c, K_c, ws, ws_bytes, nullptr, stages, nullptr,
                      &ah);
}

int pi_ffn_layer(void* stream, const pi_layer* L, int32_t B, const float* x, float tau, const float* y_c, float* y,
                 float* logits, int32_t* A_g, int32_t* K, int32_t* A_c, int32_t* K_c, void* ws, size_t ws_bytes,
                 void* const* events) {
  return pi_ffn_layer_stages(stream, L, B, x, tau, y_c, y, logits, A_g, K, A_c, K_c, ws, ws_bytes, events,
                             PI_STAGE_ALL, nullptr);
}

int pi_ffn_layer_normed(void* stream, const pi_layer* L, int32_t B, const float* y_prev, float eps, float tau,
                        const float* y_c, float* y, float* logits, int32_t* A_g, int32_t* K, int32_t* A_c,
                        int32_t* K_c, float* x_out, void* ws, size_t ws_bytes) {
  if (!L || !y_prev || !aligned16(y_prev) || (x_out && !aligned16(x_out))) return PI_EINVAL;
  if (!valid_batch(B) || L->d <= 0 || L->N <= 0 || L->H <= 0 || !(eps >= 0.f) || !std::isfinite(eps))
    return PI_EINVAL;
  const size_t row = (size_t)B * (size_t)L->d * 4;
  // the normalised row is written before y_prev is read again and y is written last
  if (x_out && (ranges_overlap(x_out, row, y_prev, row) || (y && ranges_overlap(x_out, row, y, row))))
    return PI_EINVAL;
  if (!ws || !aligned16(ws)) return PI_EWORKSPACE;
  const NormedWs n = normed_ws_layout(ws, B, L->d, L->H, L->N, L->n_g);
  if (ws_bytes < n.bytes) return PI_EWORKSPACE;
  if (b1_fused(L, B) && pi::hidden_lds_supported(L->P1.dtype, L->d)) {
    LnIn ln{eps, n.stats, x_out};
    return layer_stages(stream, L, B, y_prev, tau, y_c, y, logits, A_g, K, A_c, K_c, n.layer, n.layer_bytes, nullptr,
                        PI_STAGE_ALL, nullptr, nullptr, &ln);
  }
  // other shapes: the normalisation kernel first, then the layer on its output
  float* xn = x_out ? x_out : n.xn;
  const int st = pi_layer_norm(stream, B, L->d, y_prev, eps, xn);
  if (st != PI_OK) return st;
  return layer_stages(stream, L, B, xn, tau, y_c, y, logits, A_g, K, A_c, K_c, n.layer, n.layer_bytes, nullptr,
                      PI_STAGE_ALL, nullptr, nullptr);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// The layer call without a caller workspace (pi_ffn_layer_static).  Its workspace
// is this file-scope device array: each GPU the library runs on holds its own
// copy until the process ends.  In host code `scratch` is a host-side stand-in,
// not a device address, so host code never passes it: it passes the address
// hipGetSymbolAddress gives, looked up once per device (with that device
// current) on the entry point's first call there and kept per device.
static __device__ __align__(256) unsigned char scratch[PI_STATIC_WORKSPACE_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];   // static storage: starts null

// The current device's copy of `scratch` (looked up on the first call per device).
int static_workspace(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) return PI_EUNSUPPORTED;
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (!p) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e);
    if (!p) return PI_EHIP;
    g_scratch_addr[dev].store(p, std::memory_order_release);   // the same address from any thread
  }
  *out = p;
  return PI_OK;
}

}  // namespace

extern "C" {

int pi_ffn_layer_static(void* stream, const pi_layer* L, int32_t B, const float* x, float tau, const float* y_c,
                        float* y, float* logits, int32_t* A_g, int32_t* K, int32_t* A_c, int32_t* K_c) {
  if (!L) return PI_EINVAL;
  if (pi_workspace_bytes(PI_OP_FFN_LAYER, B, L->d, L->H, L->N, L->n_g) > (size_t)PI_STATIC_WORKSPACE_BYTES)
    return PI_EWORKSPACE;
  void* ws = nullptr;
  const int st = static_workspace(&ws);
  if (st != PI_OK) return st;
  return pi_ffn_layer(stream, L, B, x, tau, y_c, y, logits, A_g, K, A_c, K_c, ws, PI_STATIC_WORKSPACE_BYTES,
                      nullptr);
}

}  // extern "C"
