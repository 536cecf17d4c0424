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
