// pi_internal.h - launchers behind the C ABI (validated arguments only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "../../include/pi.h"
#include "pi_list.h"
#include "pi_b1.h"

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

// The lists from the activation words.
hipError_t launch_layer_norm(int B, int d, const float* y, float eps, float* x, hipStream_t s);
hipError_t launch_read_probe(const void* buf, int64_t bytes, int blocks, int depth, uint32_t* out, hipStream_t s);
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
constexpr int kNumCU = 256;   // compute units of the gfx950 parts (MI350X / MI355X)
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
                                // multiple of 32 positions), the activations of the fp16 axpy; vector q
                                // of each 32-position block holds positions q, q + 4, .., q + 28
  float* out_lo;                // with out_h8, optional: the same layout holding fp16(z - fp16(z))
  int x_f16;                    // fp16 weights: x may be rounded to fp16 (fp16 matrix cores; FC1 only)
  int x_hilo;                   // fp16 weights: x as two fp16 parts, hi = fp16(x) and lo = fp16(x - hi),
                                // both multiplied exactly (fp16 matrix cores at about 22 bits of x)
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
int mm_row16_ks(int64_t count_max, int64_t cols, int nbt, bool gated, bool hilo = false);
int mm_axpy_col_chunks(int dt, int64_t cols);
int mm_axpy_row_chunks(int dt, int nbt, int64_t count_max, int64_t cols);
bool mm_rowdot_supported(int dt, int64_t rows, int64_t cols);
bool mm_axpy_supported(int dt, int64_t rows, int64_t cols);
bool mm_axpy16_supported(int dt, int64_t cols);
int64_t mm_axpy_rows_per_chunk(const MmAxpyArgs& a);   // from count_max and row_chunks
hipError_t launch_mm_rowdot(const MmRowArgs& a, hipStream_t s);   // the GEMM, then the finish
hipError_t launch_mm_axpy(const MmAxpyArgs& a, hipStream_t s);

}  // namespace pi
