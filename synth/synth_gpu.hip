// synth_gpu.hip - device side of the seeded synthetic-workload generator.
//
// Input generation only.  Each thread produces whole 128-element groups (or
// plain elements) of a row with the same synth_rng.h functions the host uses,
// so device-generated weights have exactly the host-generated bits.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "synth_rng.h"

namespace {

__global__ void k_fill_dense(void* out, int dtype, uint64_t seed, uint32_t tag, uint32_t layer,
                             const int32_t* row_ids, int64_t row0, int64_t nrows, int64_t cols, double k) {
  int64_t total = nrows * cols;
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < total; e += (int64_t)gridDim.x * blockDim.x) {
    int64_t r = e / cols, c = e - r * cols;
    int64_t id = row_ids ? (int64_t)row_ids[r] : row0 + r;
    uint64_t rk = sx_rowkey(seed, tag, layer, (uint64_t)id);
    double v = (double)sx_ih4(sx_hash(rk, (uint64_t)c)) * k;
    if (dtype == SX_F32) ((float*)out)[e] = (float)v;
    else ((uint16_t*)out)[e] = sx_f64_to_f16(v);
  }
}

__global__ void k_fill_i4(uint8_t* out, uint16_t* scales, uint64_t seed, uint32_t tag, uint32_t layer,
                          const int32_t* row_ids, int64_t row0, int64_t nrows, int64_t cols, double k) {
  int64_t groups = cols / 128, total = nrows * groups;
  for (int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; e < total; e += (int64_t)gridDim.x * blockDim.x) {
    int64_t r = e / groups, g = e - r * groups;
    int64_t id = row_ids ? (int64_t)row_ids[r] : row0 + r;
    uint64_t rk = sx_rowkey(seed, tag, layer, (uint64_t)id);
    double mx = 0.0;
    for (int j = 0; j < 128; ++j) {
      double v = (double)sx_ih4(sx_hash(rk, (uint64_t)(g * 128 + j))) * k;
      double a = v < 0 ? -v : v;
      if (a > mx) mx = a;
    }
    uint16_t s16 = sx_f64_to_f16(mx / 7.0);
    double s = sx_f16_to_f64(s16);
    scales[e] = s16;
    uint8_t* o = out + r * (cols / 2) + g * 64;
    for (int j = 0; j < 128; j += 2) {
      int q[2];
      for (int t = 0; t < 2; ++t) {
        double v = (double)sx_ih4(sx_hash(rk, (uint64_t)(g * 128 + j + t))) * k;
        double rr = s > 0 ? rint(v / s) : 0.0;
        if (rr > 7) rr = 7;
        if (rr < -8) rr = -8;
        q[t] = (int)rr;
      }
      o[j / 2] = (uint8_t)((q[0] & 0xF) | ((q[1] & 0xF) << 4));
    }
  }
}

}  // namespace

extern "C" int sxg_fill_rows(void* out, uint16_t* scales, int dtype, uint64_t seed, uint32_t tag, uint32_t layer,
                             const int32_t* row_ids, int64_t row0, int64_t nrows, int64_t cols, double k, void* stream) {
  if (!out || nrows < 0 || cols <= 0) return 1;
  if (nrows == 0) return 0;
  hipStream_t s = (hipStream_t)stream;
  if (dtype == SX_I4G128) {
    if (!scales || cols % 128) return 1;
    int64_t total = nrows * (cols / 128);
    int grid = (int)((total + 255) / 256 < 65536 ? (total + 255) / 256 : 65536);
    hipLaunchKernelGGL(k_fill_i4, dim3(grid), dim3(256), 0, s, (uint8_t*)out, scales, seed, tag, layer, row_ids, row0, nrows, cols, k);
  } else {
    int64_t total = nrows * cols;
    int grid = (int)((total + 255) / 256 < 65536 ? (total + 255) / 256 : 65536);
    hipLaunchKernelGGL(k_fill_dense, dim3(grid), dim3(256), 0, s, out, dtype, seed, tag, layer, row_ids, row0, nrows, cols, k);
  }
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
