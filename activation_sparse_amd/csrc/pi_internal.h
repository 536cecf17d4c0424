// pi_internal.h - launchers behind the C ABI (validated arguments only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "../../include/pi.h"
#include "pi_list.h"

namespace pi {

// Generic row-dot GEMV (any batch, any row length): predictor layers and FC1.
struct RowdotArgs {
  const void* W;             // [rows x cols]
  const uint16_t* Ws;        // int4 scales
  const void* Wup;           // gated only
  const uint16_t* Wups;
  int dt;
  int64_t cols;
  const int32_t* list;       // gathered rows (NULL = dense rows 0..count)
  const int32_t* count_dev;  // device count for gathered mode
  int64_t count_max;         // dense count, or the bound on *count_dev
  const float* x;            // [B x cols]
  int B;
  const void* bias;          // per row (indexed by row id)
  int bias_dt;
  int relu;                  // apply max(0, .)
  int gated;
  float* out;                // [B x out_stride], column = output index
  int64_t out_stride;
};

hipError_t launch_rowdot(const RowdotArgs& a, hipStream_t s);
// n_rows bounds listed row ids; block 0 first clears zero_n u32 words at zero_ptr (or none).
hipError_t launch_rowdot_ex(const RowdotArgs& a, int64_t n_rows, uint32_t* zero_ptr, int zero_n, hipStream_t s);

// Standalone compaction (any table order, single block per table).
hipError_t launch_compact(int B, int N, const float* logits, float tau, const int32_t* T_g, int n_g,
                          int32_t* A_g, int32_t* K, const int32_t* T_c, int n_c, int32_t* A_c,
                          int32_t* K_c, hipStream_t s);

// Batch-1 register-x GEMV kernels.
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
  uint32_t* zero_ptr;        // hidden: words cleared by block 0
  int zero_n;
};
bool b1_supported(int dt, int64_t cols);
hipError_t launch_hidden_b1(const B1Gemv& g, hipStream_t s);
hipError_t launch_fc1_b1(const B1Gemv& g, bool gated, hipStream_t s);

// Output layer; mask8 != NULL also writes the activation bits, 8 rows per byte.
hipError_t launch_logits_b1(const B1Gemv& g, float tau, uint8_t* mask8, hipStream_t s);

// FC1 of the fused batch-1 layer, one 64-id block per 512-thread block (see pi_fast.hip).
struct SegCtx {
  const uint32_t* gbits;     // prepared table: GPU-resident bitmap, 2 words per 64 ids
  const int32_t* gpre;       // prepared table: GPU-resident ids below each 64-id block
  const void* W1;
  const uint16_t* W1s;
  const void* Wu;
  const uint16_t* Wus;
  int d;
  int n_g;
  const float* x;
  const void* b1;
  int b1_dt;
  int32_t* seg_slot;         // [nblk x 64] ascending slots of each block's active GPU neurons
  float* seg_a;              // [nblk x 64] their activations (batch 1)
  int32_t* seg_cold;         // [nblk x 64] ascending cold slots of each block's active CPU neurons
  uint32_t* cnt;             // [nblk] GPU count | CPU count << 16
};
bool fc1_blk_supported(int dt, int64_t d);
hipError_t launch_fc1_blk(const uint32_t* mask, const SegCtx& sg, int dtw, bool gated, int nblk, hipStream_t s);

// Batch-1 FC2 and final reduction over those segments (see pi_fc2.hip).
constexpr int kSegChunks = 64;   // id-block chunks of the segment FC2 (nblk <= 64 * kSegChunks)
struct Fc2SegArgs {
  const void* W2;
  const uint16_t* W2s;
  int dt;
  int64_t d;
  int n_g;
  int nblk;
  const int32_t* seg_slot;
  const float* seg_a;
  const uint32_t* cnt;
  float* partials;           // [kSegChunks x d]
};
struct ReduceListArgs {
  const float* partials;
  int64_t d;
  float* y;
  const float* y_c;
  const void* b2;
  int b2_dt;
  int nblk;
  const uint32_t* cnt;
  const int32_t* seg_slot;
  const int32_t* seg_cold;
  int32_t* A_g;
  int32_t* K;
  int32_t* A_c;              // NULL = no cold list
  int32_t* K_c;
  int n_g;
  int n_c;
  int always_c;              // add y_c even with no active cold neuron (no cold side)
  int chunks;                // set by the launcher
  int reduce_blocks;         // set by the launcher
};
hipError_t launch_fc2_seg(const Fc2SegArgs& a, hipStream_t s);
hipError_t launch_reduce_lists(const ReduceListArgs& r, hipStream_t s);

// Activation words from stored logits (union over the batch), and the lists from them.
hipError_t launch_mask(int B, int N, const float* logits, float tau, uint32_t* mask, hipStream_t s);
hipError_t launch_list(const ListCtx& c, int n_g, hipStream_t s);

struct Fc2Args {
  const void* W2;
  const uint16_t* W2s;
  int dt;
  int64_t d;
  int n_g;
  const int32_t* list;
  const int32_t* K;
  const float* a;            // [B x n_g]
  int B;
  float* partials;           // [chunks x B x d]
};

struct ReduceArgs {
  const float* partials;     // [chunks x B x d]
  int chunks;
  int B;
  int64_t d;
  float* y;                  // [B x d]
  const float* y_c;          // merged when non-NULL and (K_c == NULL or *K_c != 0)
  const int32_t* K_c;
  const void* b2;
  int b2_dt;
};

int fc2_tiles(int dt, int64_t d);
int fc2_chunks(int B);           // row chunks of FC2 for batch B (partials: chunks x B x d floats)
hipError_t launch_fc2(const Fc2Args& a, hipStream_t s);
hipError_t launch_reduce(const ReduceArgs& r, hipStream_t s);
hipError_t launch_zero_u32(uint32_t* p, int64_t n, hipStream_t s);

hipError_t launch_merge(int B, int d, float* y, const float* y_c, const int32_t* K_c, const void* b2,
                        int b2_dt, hipStream_t s);

}  // namespace pi
