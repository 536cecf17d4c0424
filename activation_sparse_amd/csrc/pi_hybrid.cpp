// pi_hybrid.cpp - the hybrid layer's executor (libpi_host): one thread drives
// the GPU stream through libpi and runs the cold neurons on the host through
// pi_cold_ffn, with the copies and the event waits in between.
#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "../../include/pi_host.h"

namespace {

int hip_ok(hipError_t e) { return e == hipSuccess ? PI_OK : PI_EHIP; }

constexpr int kListHead = 4;  // int32 entries before the CPU list in the cold-list block

}  // namespace

extern "C" int pi_hybrid_layer(void* stream, const pi_layer* L, const int32_t* T_g, const int32_t* T_c,
                               const pi_host_cold* cold, int32_t B, const float* x, float tau, float* y,
                               const pi_hybrid_scratch* s, int32_t threads, int32_t* K_c_out) {
  if (!L || !s || !x || !y || !T_g || B < 1 || B > PI_MAX_BATCH) return PI_EINVAL;
  const int32_t n_c = (T_c && cold) ? cold->n_c : 0;
  if (n_c > 0 && (!s->cold_list || !s->y_c || !s->x_host || !s->cold_list_host || !s->y_c_host || !s->event))
    return PI_EINVAL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int32_t d = L->d, N = L->N, H = L->H, n_g = L->n_g;
  const size_t xb = (size_t)B * d * sizeof(float);
  if (K_c_out) *K_c_out = 0;
  int r = pi_predict(stream, B, d, H, N, x, L->P1, L->c1, L->P2, L->c2, s->logits, s->ws_pred, s->ws_pred_bytes);
  if (r != PI_OK) return r;
  int32_t* K_c = n_c > 0 ? s->cold_list : nullptr;
  r = pi_compact(stream, B, N, s->logits, tau, T_g, n_g, s->A_g, s->K, n_c > 0 ? T_c : nullptr, n_c,
                 n_c > 0 ? s->cold_list + kListHead : nullptr, K_c, nullptr, 0);
  if (r != PI_OK) return r;
  hipEvent_t ev = static_cast<hipEvent_t>(s->event);
  if (n_c > 0) {
    // the two copies back to back: each switch between the copy engine and the kernels costs
    const size_t lb = (size_t)(kListHead + n_c) * sizeof(int32_t);
    if ((r = hip_ok(hipMemcpyAsync(s->x_host, x, xb, hipMemcpyDeviceToHost, st))) != PI_OK) return r;
    if ((r = hip_ok(hipMemcpyAsync(s->cold_list_host, s->cold_list, lb, hipMemcpyDeviceToHost, st))) != PI_OK)
      return r;
    if ((r = hip_ok(hipEventRecord(ev, st))) != PI_OK) return r;
  }
  // the GPU's neurons, queued before this thread waits for the cold list
  r = pi_sparse_ffn(stream, B, d, n_g, L->kind, x, L->W1, L->b1, L->Wup, L->W2, s->A_g, s->K, y, s->ws_ffn,
                    s->ws_ffn_bytes);
  if (r != PI_OK) return r;
  int32_t kc = 0;
  if (n_c > 0) {
    if ((r = hip_ok(hipEventSynchronize(ev))) != PI_OK) return r;
    kc = s->cold_list_host[0];
  }
  if (K_c_out) *K_c_out = kc;
  if (kc > 0) {
    r = pi_cold_ffn(B, d, n_c, L->kind, s->x_host, cold->W1, cold->b1, cold->Wup, cold->W2,
                    s->cold_list_host + kListHead, kc, s->y_c_host, threads);
    if (r != PI_OK) return r;
    if ((r = hip_ok(hipMemcpyAsync(s->y_c, s->y_c_host, xb, hipMemcpyHostToDevice, st))) != PI_OK) return r;
    return pi_merge(stream, B, d, y, s->y_c, K_c, L->b2);
  }
  // nothing from the CPU side: only the output bias, if the layer has one
  return L->b2.data ? pi_merge(stream, B, d, y, nullptr, nullptr, L->b2) : PI_OK;
}

namespace {

bool ahead_buffers_ok(const pi_hybrid_ahead_scratch* s) {
  if (!s || (s->cur != 0 && s->cur != 1) || !s->logits || !s->y_c || !s->x_host || !s->y_c_host || !s->x_event)
    return false;
  for (int i = 0; i < 2; ++i)
    if (!s->A_g[i] || !s->K[i] || !s->cold_list[i] || !s->cold_list_host[i] || !s->list_event[i]) return false;
  return true;
}

// pi_predict + pi_compact of `L` on x into list set `set`, the copy of its CPU list block to the
// host and that set's event.
int predict_into(hipStream_t st, const pi_layer* L, const int32_t* T_g, const int32_t* T_c, int32_t n_c, int32_t B,
                 const float* x, float tau, const pi_hybrid_ahead_scratch* s, int set) {
  int r = pi_predict(st, B, L->d, L->H, L->N, x, L->P1, L->c1, L->P2, L->c2, s->logits, s->ws_pred,
                     s->ws_pred_bytes);
  if (r != PI_OK) return r;
  r = pi_compact(st, B, L->N, s->logits, tau, T_g, L->n_g, s->A_g[set], s->K[set], n_c > 0 ? T_c : nullptr, n_c,
                 n_c > 0 ? s->cold_list[set] + kListHead : nullptr, n_c > 0 ? s->cold_list[set] : nullptr, nullptr, 0);
  if (r != PI_OK) return r;
  if (n_c > 0) {
    const size_t lb = (size_t)(kListHead + n_c) * sizeof(int32_t);
    if ((r = hip_ok(hipMemcpyAsync(s->cold_list_host[set], s->cold_list[set], lb, hipMemcpyDeviceToHost, st))) !=
        PI_OK)
      return r;
  } else {
    s->cold_list_host[set][0] = 0;   // no CPU table: an empty list
  }
  return hip_ok(hipEventRecord(static_cast<hipEvent_t>(s->list_event[set]), st));
}

}  // namespace

extern "C" int pi_hybrid_prime(void* stream, const pi_layer* L, const int32_t* T_g, const int32_t* T_c, int32_t n_c,
                               int32_t B, const float* x, float tau, pi_hybrid_ahead_scratch* s) {
  if (!L || !x || !T_g || B < 1 || B > PI_MAX_BATCH || n_c < 0 || (n_c > 0 && !T_c) || !ahead_buffers_ok(s))
    return PI_EINVAL;
  return predict_into(static_cast<hipStream_t>(stream), L, T_g, T_c, n_c, B, x, tau, s, s->cur);
}

extern "C" int pi_hybrid_layer_ahead(void* stream, const pi_layer* L, const pi_host_cold* cold, const pi_layer* next,
                                     const int32_t* T_g_next, const int32_t* T_c_next, int32_t n_c_next, int32_t B,
                                     const float* x, float tau, float* y, pi_hybrid_ahead_scratch* s,
                                     int32_t threads, int32_t* K_c_out) {
  if (!L || !x || !y || B < 1 || B > PI_MAX_BATCH || !ahead_buffers_ok(s)) return PI_EINVAL;
  if (next && (!T_g_next || n_c_next < 0 || (n_c_next > 0 && !T_c_next))) return PI_EINVAL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int cur = s->cur, nxt = 1 - cur;
  const int32_t d = L->d;
  const size_t xb = (size_t)B * d * sizeof(float);
  // the next layer is predicted from x after this layer's output is written: y must not overlap x
  const uintptr_t xa = reinterpret_cast<uintptr_t>(x), ya = reinterpret_cast<uintptr_t>(y);
  if (d > 0 && xa < ya + xb && ya < xa + xb) return PI_EINVAL;
  if (K_c_out) *K_c_out = 0;
  int r;
  if ((r = hip_ok(hipMemcpyAsync(s->x_host, x, xb, hipMemcpyDeviceToHost, st))) != PI_OK) return r;
  if ((r = hip_ok(hipEventRecord(static_cast<hipEvent_t>(s->x_event), st))) != PI_OK) return r;
  // the GPU's neurons, then the next layer's prediction, both ahead of this thread's wait
  r = pi_sparse_ffn(stream, B, d, L->n_g, L->kind, x, L->W1, L->b1, L->Wup, L->W2, s->A_g[cur], s->K[cur], y,
                    s->ws_ffn, s->ws_ffn_bytes);
  if (r != PI_OK) return r;
  if (next && (r = predict_into(st, next, T_g_next, T_c_next, n_c_next, B, x, tau, s, nxt)) != PI_OK) return r;
  if ((r = hip_ok(hipEventSynchronize(static_cast<hipEvent_t>(s->x_event)))) != PI_OK) return r;
  if ((r = hip_ok(hipEventSynchronize(static_cast<hipEvent_t>(s->list_event[cur])))) != PI_OK) return r;
  const int32_t n_c = cold ? cold->n_c : 0;
  int32_t kc = n_c > 0 ? s->cold_list_host[cur][0] : 0;
  kc = kc < 0 ? 0 : (kc > n_c ? n_c : kc);
  if (K_c_out) *K_c_out = kc;
  s->cur = nxt;
  if (kc > 0) {
    r = pi_cold_ffn(B, d, n_c, L->kind, s->x_host, cold->W1, cold->b1, cold->Wup, cold->W2,
                    s->cold_list_host[cur] + kListHead, kc, s->y_c_host, threads);
    if (r != PI_OK) return r;
    if ((r = hip_ok(hipMemcpyAsync(s->y_c, s->y_c_host, xb, hipMemcpyHostToDevice, st))) != PI_OK) return r;
    return pi_merge(stream, B, d, y, s->y_c, s->cold_list[cur], L->b2);
  }
  return L->b2.data ? pi_merge(stream, B, d, y, nullptr, nullptr, L->b2) : PI_OK;
}

extern "C" int pi_hybrid_stack_ahead(void* stream, int32_t n_layers, const pi_layer* layers,
                                     const pi_host_cold* const* colds, const int32_t* const* T_g,
                                     const int32_t* const* T_c, const int32_t* n_c, int32_t B, const float* const* xs,
                                     float tau, float* const* ys, pi_hybrid_ahead_scratch* s, int32_t threads,
                                     int32_t* K_c_out) {
  if (n_layers < 1 || !layers || !colds || !T_g || !T_c || !n_c || !xs || !ys) return PI_EINVAL;
  int r = pi_hybrid_prime(stream, &layers[0], T_g[0], T_c[0], n_c[0], B, xs[0], tau, s);
  if (r != PI_OK) return r;
  for (int32_t l = 0; l < n_layers; ++l) {
    const bool more = l + 1 < n_layers;
    r = pi_hybrid_layer_ahead(stream, &layers[l], colds[l], more ? &layers[l + 1] : nullptr, more ? T_g[l + 1] : nullptr,
                              more ? T_c[l + 1] : nullptr, more ? n_c[l + 1] : 0, B, xs[l], tau, ys[l], s, threads,
                              K_c_out ? K_c_out + l : nullptr);
    if (r != PI_OK) return r;
  }
  return PI_OK;
}
