// pi_attn.h - arguments and launcher of the self-attention decode kernels (pi_attn.hip).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pi {

constexpr int kMaxAttnHeads = 256;

struct AttnArgs {
  int d, n_heads, dh, Ha, L_max, t, n_chunks;
  float tau;
  const float* x;            // [d]
  const void* Pa1;           // fp16 [Ha x d]
  const void* ca1;           // fp16 [Ha] or NULL
  const void* Pa2;           // fp16 [n_heads x Ha]
  const void* ca2;           // fp16 [n_heads] or NULL
  const void* Wq;            // fp16 [d x d]
  const void* bq;
  const void* Wk;
  const void* bk;
  const void* Wv;
  const void* bv;
  const void* WoT;           // fp16 [d x d], row h*dh + i
  const void* bo;
  uint16_t* Kc;              // fp16 [n_heads x L_max x dh]
  uint16_t* Vc;
  // workspace
  float* g;                  // [Ha] predictor hidden layer
  float* q;                  // [d] queries of the active heads
  int32_t* flag;             // [n_heads] 1 = active
  float* hlogit;             // [n_heads]
  float* part;               // [n_heads x n_chunks x (dh + 2)] per chunk: max, sum, weighted values
  float* ypart;              // [n_heads x d] per head: its output-projection contribution
  // outputs
  float* y;                  // [d]
  float* logits_out;         // [n_heads] or NULL
  int32_t* heads;            // [n_heads] ascending active heads
  int32_t* n_active;         // [1]
};

bool attn_supported(int d, int n_heads, int dh, int Ha);
int attn_chunks(int L_max);
hipError_t launch_attn(const AttnArgs& a, hipStream_t s);

}  // namespace pi
