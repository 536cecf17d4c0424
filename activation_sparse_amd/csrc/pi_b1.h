// pi_b1.h - arguments and launchers of the batch-1 layer kernels (pi_fast.hip):
// the register-x GEMVs, the predictor output layer over the active hidden units
// fused with FC1, the segment FC2 with the lists, and the final ordered sum.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pi {

// Batch-1 register-x GEMV kernels (pi_fast.hip).
struct B1Gemv {
  const void* W;
  const uint16_t* Ws;
  const void* Wu;            // gated FC1 only
  const uint16_t* Wus;
  int dt;
  int rows;                  // dense rows, or n_g for FC1
  int cols;
  const float* x;            // [cols]
  const void* bias;
  int bias_dt;
  float* out;
  const int32_t* list;       // FC1
  const int32_t* Kp;         // FC1
  // hidden layer only: x is a raw row to normalise first (layer normalisation, unit gain, zero
  // bias) when ln_stats != NULL; the kernel writes the mean and 1/sqrt(var + ln_eps) it used to
  // ln_stats[0..1] and, when x_out != NULL, the normalised row to x_out [cols]
  float* ln_stats;
  float ln_eps;
  float* x_out;
};
bool b1_supported(int dt, int64_t cols);
// the batch-1 hidden layer with x staged in LDS (rows up to 32 KB); with ln_stats, x is first
// normalised (layer normalisation, unit gain, zero bias) and the statistics and x_out written
bool hidden_lds_supported(int dt, int64_t cols);
hipError_t launch_hidden_lds(const B1Gemv& g, hipStream_t s);
hipError_t launch_fc1_b1(const B1Gemv& g, bool gated, hipStream_t s);

// Batch 1: the predictor output layer over the active hidden units (P2 stored
// hidden-major), with the activation decision, and in the fused layer FC1 of
// the tile's active GPU-resident neurons (pi_fast.hip).  One block per tile of
// 64 or 128 neuron ids; no block waits for another.
constexpr int kMaxHiddenB1 = 4096;   // hidden units the batch-1 output-layer kernel takes
struct PredFc1Args {
  const void* P2;            // [H x N] hidden-major
  const uint16_t* P2s;       // int4 scales [H x N/128]
  int pdt;
  int H;
  int N;
  const float* h;            // [H]
  const void* c2;
  int c2_dt;
  float tau;
  float* logits;             // [N], optional
  uint32_t* mask;            // 2 words per 64 ids, optional (output-layer-only launches)
  // FC1 (fused layer)
  const uint32_t* gbits;     // prepared table: GPU-resident bitmap, 2 words per 64 ids
  const int32_t* gpre;       // prepared table: GPU-resident ids below each 64-id group
  const void* W1;
  const uint16_t* W1s;
  const void* Wu;
  const uint16_t* Wus;
  int dt;
  int d;
  int n_g;
  const float* x;
  const float* ln_stats;     // NULL, or the mean and 1/sqrt(var + eps) to normalise x with
  const void* b1;
  int b1_dt;
  int32_t* seg_slot;         // [groups x 64] ascending slots of each group's active GPU-resident neurons
  int32_t* seg_cold;         // [groups x 64] ascending cold slots of each group's active CPU-resident neurons
  int32_t* pos_slot;         // [groups x 64] the group's slots whose FC1 output is non-zero, ascending
  float* pos_a;              // [groups x 64] their FC1 outputs
  uint32_t* cnt;             // [groups] GPU count | CPU count << 8 | non-zero count << 16
  int32_t* rows_read;        // optional: block 0 writes the number of output-layer rows read
  // look-ahead (FC1 launches only): blocks past the N/T tiles each take T/8 rows of the next
  // layer's predictor hidden layer, nh[m] = max(0, nP1[m].x + nc1[m]), on this layer's x (nP1 in
  // the FC1 weights' format, nc1 in b1's); nh == NULL: none
  const void* nP1;
  const uint16_t* nP1s;
  const void* nc1;
  int nH;
  float* nh;
};
// Group count word fields.
__host__ __device__ constexpr uint32_t cnt_gpu(uint32_t c) { return c & 0xFFu; }
__host__ __device__ constexpr uint32_t cnt_cold(uint32_t c) { return (c >> 8) & 0xFFu; }
__host__ __device__ constexpr uint32_t cnt_nz(uint32_t c) { return (c >> 16) & 0xFFu; }

bool pred_out_b1_supported(int pdt, int H, int N);
hipError_t launch_pred_out_b1(const PredFc1Args& a, hipStream_t s);
// Fused output layer + FC1; false when this combination of dtypes and sizes has no fused kernel.
bool pred_fc1_supported(int pdt, int dt, int bdt, int c2dt, bool gated, int H, int N, int64_t d);
hipError_t launch_pred_fc1(const PredFc1Args& a, bool gated, hipStream_t s);

// Batch-1 FC2 over the group segments, with the list assembly, and the final
// ordered sum.
constexpr int kSegChunks = 32;   // group chunks of the segment FC2 (groups <= 64 * kSegChunks)
struct Fc2SegArgs {
  const void* W2;
  const uint16_t* W2s;
  int dt;
  int64_t d;
  int n_g;
  int ngroups;
  const int32_t* pos_slot;
  const float* pos_a;
  const int32_t* seg_slot;
  const int32_t* seg_cold;
  const uint32_t* cnt;
  float* partials;           // [kSegChunks x d]
  int32_t* A_g;
  int32_t* K;
  int32_t* A_c;              // NULL = no cold list
  int32_t* K_c;
  int n_c;
  int32_t* rows_read;        // optional: list block 0 writes the number of W2 rows read
};
struct ReduceYArgs {
  const float* partials;     // [kSegChunks x d]
  int64_t d;
  float* y;
  const float* y_c;
  const int32_t* K_c;        // the cold count written by the FC2 launch (NULL = always add y_c)
  const void* b2;
  int b2_dt;
};
hipError_t launch_fc2_seg(const Fc2SegArgs& a, hipStream_t s);
hipError_t launch_reduce_y(const ReduceYArgs& r, hipStream_t s);

}  // namespace pi
