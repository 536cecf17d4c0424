// pi_internal.h - launchers behind the C ABI (validated arguments only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "../../include/pi.h"
#include "pi_list.h"

namespace pi {

// Generic row-dot GEMV (any batch, any row length): predictor hidden layer and FC1.
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
};
bool b1_supported(int dt, int64_t cols);
hipError_t launch_hidden_b1(const B1Gemv& g, hipStream_t s);
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
  const void* b1;
  int b1_dt;
  int32_t* seg_slot;         // [groups x 64] ascending slots of each group's active GPU-resident neurons
  int32_t* seg_cold;         // [groups x 64] ascending cold slots of each group's active CPU-resident neurons
  int32_t* pos_slot;         // [groups x 64] the group's slots whose FC1 output is non-zero, ascending
  float* pos_a;              // [groups x 64] their FC1 outputs
  uint32_t* cnt;             // [groups] GPU count | CPU count << 8 | non-zero count << 16
  int32_t* rows_read;        // optional: block 0 writes the number of output-layer rows read
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
// ordered sum (pi_fc2.hip).
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

// The lists from the activation words.
hipError_t launch_list(const ListCtx& c, int n_g, hipStream_t s);

// Neuron-major axpy over listed rows: out[b,:] += a[b, j] * W[list[j], :]
// (FC2, and the predictor output layer over its hidden-major weights).
struct Fc2Args {
  const void* W2;
  const uint16_t* W2s;
  int dt;
  int64_t d;                 // row length
  int n_g;                   // rows in W2 (bound for listed rows)
  const int32_t* list;       // NULL = rows 0 .. n_g in order
  const int32_t* K;          // device count of listed rows (ignored when list == NULL)
  const float* a;            // a[b * a_stride + (a_by_row ? row : j)]
  int64_t a_stride;
  int a_by_row;
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
// The same sum for the logits (no merge), with the activation words (2 per 64 ids) of the union over B.
hipError_t launch_reduce_mask(const ReduceArgs& r, float tau, uint32_t* mask, hipStream_t s);
hipError_t launch_zero_u32(uint32_t* p, int64_t n, hipStream_t s);

hipError_t launch_merge(int B, int d, float* y, const float* y_c, const int32_t* K_c, const void* b2,
                        int b2_dt, hipStream_t s);

// Batched GEMMs on the matrix cores (pi_mfma.hip): the row-dot GEMMs (predictor
// hidden layer, FC1) from kMmRowMinBatch batch rows, the axpy GEMMs (output
// layer, FC2) from kMmAxpyMinBatch (below that the VALU kernels measure faster).
constexpr int kMmRowMinBatch = 2;
constexpr int kMmAxpyMinBatch = 3;
struct MmRowArgs {              // out[b, pos] = finish(sum_k W[row(pos), k] x[b, k])
  const void* W;
  const uint16_t* Ws;
  const void* Wup;              // gated only
  const uint16_t* Wups;
  int dt;
  int gated;
  int64_t cols;
  int64_t n_rows;               // rows in W (bound for listed rows)
  const int32_t* list;          // NULL = rows 0 .. count_max
  const int32_t* count_dev;
  int64_t count_max;
  const float* x;               // [B x cols]
  int B;
  int nbt;                      // batch tiles of 16 (mm_nbt)
  int ks;                       // k chunks (mm_row_ks), kc columns each (mm_row_kc)
  int64_t kc;
  float* partials;              // [(1 + gated) x ks x count_max x 16 nbt]
  const void* bias;             // per row id
  int bias_dt;
  int relu;
  float* out;                   // [B x out_stride], column = position; or, with out_tr,
  int64_t out_stride;           // [count_max x 16 nbt] neuron-major (zeros past B)
  int out_tr;
  int out_h8;                   // with out_tr: fp16 [pos / 8][16 nbt][8] (zeros past B and up to the next
                                // multiple of 32 positions), the activations of the fp16 axpy
  float* out_lo;                // with out_h8, optional: the same layout holding fp16(z - fp16(z))
  int x_f16;                    // fp16 weights: x may be rounded to fp16 (fp16 matrix cores; FC1 only)
};
struct MmAxpyArgs {             // partials[chunk, b, c] = sum over the chunk's rows j of a[b, j] W[row(j), c]
  const void* W;
  const uint16_t* Ws;
  int dt;
  int64_t cols;
  int64_t n_rows;
  const int32_t* list;          // NULL = rows 0 .. count_max
  const int32_t* count_dev;
  int64_t count_max;
  const float* a;               // a[b * a_stride + idx], or with a_tr a[idx * 16 nbt + b];
  int64_t a_stride;             // idx = a_by_row ? row : j
  int a_by_row;
  int a_tr;
  int a_h8;                     // fp16 weights, a in the out_h8 layout: the fp16 matrix cores (FC2)
  const float* a_lo;            // with a_h8, optional: the low fp16 parts (a = hi + lo, ~22 bits)
  int B;
  int nbt;
  int64_t rows_per_chunk;       // a multiple of 16
  int row_chunks;               // mm_axpy_row_chunks
  float* partials;              // [row_chunks x B x cols]
  // the fp16 kernel with one row chunk: out[b, c] = 0 + sum + bias[c] written directly
  // (no partials), and with mask the words of the union over b of out[b, c] > tau (2 per 64 columns)
  float* final_out;             // [B x cols], or NULL
  const void* bias;
  int bias_dt;
  float tau;
  uint32_t* mask;
};
int mm_nbt(int B);
int mm_row_ks(int dt, int64_t count_max, int64_t cols);
int64_t mm_row_kc(int dt, int64_t cols, int ks);
// the fp16 matrix-core row-dot (x rounded to fp16, its k chunk staged in LDS)
bool mm_row16_used(const MmRowArgs& a);
int mm_row16_ks(int64_t count_max, int64_t cols, int nbt, bool gated);
int mm_axpy_col_chunks(int dt, int64_t cols);
int mm_axpy_row_chunks(int dt, int64_t count_max, int64_t cols);
bool mm_rowdot_supported(int dt, int64_t rows, int64_t cols);
bool mm_axpy_supported(int dt, int64_t rows, int64_t cols);
bool mm_axpy16_supported(int dt, int64_t cols);
int64_t mm_axpy_rows_per_chunk(const MmAxpyArgs& a);   // from count_max and row_chunks
hipError_t launch_mm_rowdot(const MmRowArgs& a, hipStream_t s);   // the GEMM, then the finish
hipError_t launch_mm_axpy(const MmAxpyArgs& a, hipStream_t s);

}  // namespace pi
