// pi_internal.h - launchers behind the C ABI (validated arguments only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "../../include/pi.h"

namespace pi {

struct RowdotArgs {
  const void* W;          // [rows x cols]
  const uint16_t* Ws;     // int4 scales
  const void* Wup;        // gated only
  const uint16_t* Wups;
  int dt;
  int64_t cols;
  const int32_t* list;    // gathered rows (NULL = dense rows 0..count)
  const int32_t* count_dev;  // device count for gathered mode
  int64_t count_max;      // dense count, or the bound on *count_dev
  const float* x;         // [B x cols]
  int B;
  const void* bias;       // per row (indexed by row id)
  int bias_dt;
  int relu;               // apply max(0, .)
  int gated;
  float* out;             // [B x out_stride], column = output index
  int64_t out_stride;
};

hipError_t launch_rowdot(const RowdotArgs& a, hipStream_t s);

hipError_t launch_compact(int B, int N, const float* logits, float tau, const int32_t* T_g, int n_g,
                          int32_t* A_g, int32_t* K, const int32_t* T_c, int n_c, int32_t* A_c,
                          int32_t* K_c, hipStream_t s);

struct Fc2Args {
  const void* W2;
  const uint16_t* W2s;
  int dt;
  int64_t d;
  int n_g;
  const int32_t* list;
  const int32_t* K;
  const float* a;         // [B x n_g]
  int B;
  float* partials;        // [chunks x B x d]
  uint32_t* counters;     // [tiles]
  float* y;               // [B x d]
};

int fc2_tiles(int dt, int64_t d);
constexpr int kFc2Chunks = 32;
hipError_t launch_fc2(const Fc2Args& a, hipStream_t s);
hipError_t launch_zero_u32(uint32_t* p, int64_t n, hipStream_t s);

hipError_t launch_merge(int B, int d, float* y, const float* y_c, const int32_t* K_c, const void* b2,
                        int b2_dt, hipStream_t s);

}  // namespace pi
