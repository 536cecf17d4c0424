/* pi_host.h - C ABI of libpi_host, the CPU side of the hybrid layer.
 *
 * The pages split each FFN layer's neurons between the two devices: the hot
 * neurons live in GPU memory and run on the GPU, the cold ones stay in host
 * memory and run on the CPU; each side computes the same neuron-aware FFN
 * over its own active neurons, and the GPU merges the CPU's partial result
 * (CSDN summary of "PowerInfer: Fast Large Language Model Serving with a
 * Consumer-grade GPU", sections 神经元放置和管理 and GPU-CPU混合执行;
 * unite.ai French article "PowerInfer : Moteur d'inférence ...", section
 * "Placement et gestion des neurones").
 * pi_cold_ffn is the CPU side: pi_sparse_ffn's computation over the neurons of
 * the CPU table, on host memory.  Its result goes to pi_merge (or to the
 * y_c argument of pi_ffn_layer) after a copy to the device.
 *
 * pi_cold_ffn's pointers are HOST pointers owned by the caller (pi_hybrid_layer
 * states which of its own are device pointers).  Matrix formats
 * are those of pi.h (row-major, fp32 / fp16 / int4-g128 with fp16 scales).
 * The work is split over threads in fixed ranges (neurons for FC1, columns for
 * FC2) and every sum runs in one fixed order, so the result bits depend
 * neither on the thread count nor on which vector unit the CPU has. */
#ifndef PI_HOST_H
#define PI_HOST_H

#include <stddef.h>
#include <stdint.h>

#include "pi.h"

#ifdef __cplusplus
extern "C" {
#endif

/* The FFN over the CPU-resident neurons (the pages' CPU side).
 * W1, W2 (and Wup) hold the n_c CPU-resident neurons in CPU-table slot order,
 * [n_c x d] each, W2 neuron-major; b1 [n_c] (optional).  For j < K_c, c = A_c[j]:
 *   a[b,j] = max(0, W1[c].x_b + b1[c])                    (PI_RELU)
 *   a[b,j] = max(0, W1[c].x_b + b1[c]) * (Wup[c].x_b)     (PI_GATED_RELU)
 *   y_c[b,:] = sum_j a[b,j] * W2[c,:]   (a neuron whose a is 0 in every
 *                                        batch row adds nothing and its W2 row
 *                                        is not read; the others are summed in
 *                                        list order within chunks whose size
 *                                        depends on their count only, and the
 *                                        chunk sums in chunk order)
 * x [B x d] fp32; A_c [K_c] int32 (the CPU-table slots pi_compact lists);
 * y_c [B x d] fp32, fully written (zero when K_c = 0).  threads: the number
 * of threads (<= 0: the OpenMP default).  Host scratch of B * K_c floats is
 * allocated for the FC1 outputs; the FC2 chunks' partial sums (at most
 * 64 * B * d floats) live in a buffer the calling thread keeps between calls.
 * Errors: PI_EINVAL for a NULL required pointer, B outside 1..PI_MAX_BATCH,
 * d <= 0 or not a multiple of 8 (128 for int4), K_c < 0, n_c < K_c, a slot
 * outside [0, n_c), a kind outside PI_RELU / PI_GATED_RELU or a gated call
 * without Wup; PI_EUNSUPPORTED when W1, Wup and W2 do not share one dtype. */
int pi_cold_ffn(int32_t B, int32_t d, int32_t n_c, int32_t kind, const float* x, pi_matrix W1, pi_vector b1,
                pi_matrix Wup, pi_matrix W2, const int32_t* A_c, int32_t K_c, float* y_c, int32_t threads);

/* pi_cold_ffn with the code path chosen: path = 1 the AVX2 + FMA + F16C loops
 * (PI_EUNSUPPORTED when this CPU lacks them), 0 the scalar loops, -1 the best
 * this CPU has (what pi_cold_ffn does).  Both paths give the same bits. */
int pi_cold_ffn_ex(int32_t B, int32_t d, int32_t n_c, int32_t kind, const float* x, pi_matrix W1, pi_vector b1,
                   pi_matrix Wup, pi_matrix W2, const int32_t* A_c, int32_t K_c, float* y_c, int32_t threads,
                   int32_t path);

/* The path pi_cold_ffn takes on this CPU: 1 = AVX2 + FMA + F16C, 0 = scalar. */
int pi_host_vector_path(void);

/* The host streaming-read reference that the CPU side's bandwidth is read
 * against: `threads` threads (<= 0: the OpenMP default) read `bytes` bytes of
 * `buf` once, each a contiguous share of whole 64-byte lines, with 32-byte
 * loads when the CPU has AVX2 (8-byte loads otherwise), and *out receives the
 * XOR of every 8-byte word (so that no load can be dropped; the same for any
 * thread count).  buf: host memory, 64-byte aligned; bytes a multiple of 64.
 * Errors: PI_EINVAL for a NULL pointer, bytes == 0 or not a multiple of 64,
 * or an unaligned buf. */
int pi_host_read_probe(const void* buf, size_t bytes, int32_t threads, uint64_t* out);

/* The CPU-resident neurons of one layer in HOST memory, rows in CPU-table slot
 * order (the arguments pi_cold_ffn takes). */
typedef struct pi_host_cold {
  int32_t n_c;
  pi_matrix W1;
  pi_vector b1;  /* optional */
  pi_matrix Wup; /* gated only */
  pi_matrix W2;
} pi_host_cold;

/* Buffers of one pi_hybrid_layer call, owned by the caller: device buffers for the
 * predictor, the lists and the cold partial, the two device workspaces, pinned
 * host buffers for the copies, and a hipEvent_t.
 * The CPU list travels as one block, cold_list = [K_c, 0, 0, 0, A_c...]: K_c in
 * entry 0 and the list from entry 4 (16-byte aligned), so that one copy moves
 * the count and the list. */
typedef struct pi_hybrid_scratch {
  float* logits;           /* device [B x N] */
  int32_t* A_g;            /* device [n_g] */
  int32_t* K;              /* device [1] */
  int32_t* cold_list;      /* device [4 + n_c] */
  float* y_c;              /* device [B x d] */
  void* ws_pred;           /* device, pi_workspace_bytes(PI_OP_PREDICT, B, d, H, N, 0) bytes */
  size_t ws_pred_bytes;
  void* ws_ffn;            /* device, pi_workspace_bytes(PI_OP_SPARSE_FFN, B, d, 0, 0, n_g) bytes */
  size_t ws_ffn_bytes;
  float* x_host;           /* pinned host [B x d] */
  int32_t* cold_list_host; /* pinned host [4 + n_c] */
  float* y_c_host;         /* pinned host [B x d] */
  void* event;             /* hipEvent_t: x and the cold list are on the host */
} pi_hybrid_scratch;

/* One layer of the pages' GPU-CPU hybrid execution (CSDN summary, section
 * GPU-CPU混合执行: each unit computes its own active neurons, the GPU merges,
 * and the synchronisation is skipped when the CPU side has no active neuron).
 * The calling thread is the CPU executor and `stream` the GPU's:
 *  1. enqueues pi_predict and pi_compact (the layer's predictor; T_g / T_c
 *     the raw device neuron tables), then the copies of x and of the CPU list
 *     block to the pinned host buffers, back to back, and records the event;
 *  2. enqueues pi_sparse_ffn over the GPU-resident neurons (y = y_g);
 *  3. waits for the copies and runs pi_cold_ffn on the host rows;
 *  4. when K_c > 0, enqueues the copy of y_c to the device and pi_merge (which also
 *     adds b2); with K_c = 0 only b2, if any, is added.
 * Returns with step 4 enqueued (not finished); *K_c_out (optional) gets K_c.
 * x, y: device [B x d] fp32.  A layer with no CPU table (T_c NULL or n_c = 0)
 * runs steps 1-2 (without copies) and the b2 merge only.
 * Errors: those of the calls it makes; PI_EINVAL for a missing buffer or event;
 * PI_EHIP when a copy, an event record or a wait fails (pi_last_hip_error() in
 * libpi does not see these). */
int pi_hybrid_layer(void* stream, const pi_layer* layer, const int32_t* T_g, const int32_t* T_c,
                    const pi_host_cold* cold, int32_t B, const float* x, float tau, float* y,
                    const pi_hybrid_scratch* scratch, int32_t threads, int32_t* K_c_out);

/* Buffers of the look-ahead hybrid executor, owned by the caller.  Two list
 * sets: the one `cur` names holds the lists of the layer the next
 * pi_hybrid_layer_ahead call runs; that call predicts the layer after it into
 * the other set and flips `cur`.  Sizes are the largest over the layers the
 * scratch serves. */
typedef struct pi_hybrid_ahead_scratch {
  float* logits;               /* device [B x N] */
  void* ws_pred;               /* device, pi_workspace_bytes(PI_OP_PREDICT, ...) bytes */
  size_t ws_pred_bytes;
  void* ws_ffn;                /* device, pi_workspace_bytes(PI_OP_SPARSE_FFN, ...) bytes */
  size_t ws_ffn_bytes;
  int32_t* A_g[2];             /* device [n_g] each */
  int32_t* K[2];               /* device [1] each */
  int32_t* cold_list[2];       /* device [4 + n_c] each, as in pi_hybrid_scratch */
  int32_t* cold_list_host[2];  /* pinned host [4 + n_c] each */
  void* list_event[2];         /* hipEvent_t each: that set's cold list is on the host */
  float* y_c;                  /* device [B x d] */
  float* x_host;               /* pinned host [B x d] */
  float* y_c_host;             /* pinned host [B x d] */
  void* x_event;               /* hipEvent_t: x is on the host */
  int32_t cur;                 /* 0 or 1, updated by the calls */
} pi_hybrid_ahead_scratch;

/* Look-ahead prediction in the hybrid layer (a variant of the method; the
 * pages note that activations can be predicted some layers ahead while the
 * model runs).  pi_hybrid_prime predicts `layer`'s neurons from x (pi_predict,
 * pi_compact with the raw device tables T_g / T_c of n_c entries) into list
 * set scratch->cur and copies its CPU list to the host (no wait).
 * pi_hybrid_layer_ahead runs `layer` on its input x with the lists in set cur,
 * which an earlier prime or look-ahead call produced:
 *  1. copies x to the host and enqueues pi_sparse_ffn over the GPU's list;
 *  2. when `next` is given, enqueues next's prediction from this x into the
 *     other set (pi_predict, pi_compact with T_g_next / T_c_next of
 *     n_c_next entries, the copy of its CPU list), so that it runs on the GPU
 *     while this thread computes the cold neurons;
 *  3. waits for x and set cur's CPU list, runs pi_cold_ffn, and when K_c > 0
 *     enqueues the copy of y_c and pi_merge (else the b2 merge only);
 *  4. flips scratch->cur.
 * The GPU's predictor work thus leaves the path between two layers: the
 * thread waits only for the copy of x.  cold: the CPU rows of `layer` (NULL:
 * none).  Returns with the merge enqueued; *K_c_out (optional) gets K_c.
 * y may not overlap x (the next layer is predicted from x after y is
 * written).
 * Errors: PI_EINVAL for a NULL required pointer or buffer, B outside
 * 1..PI_MAX_BATCH, cur outside 0..1, or y overlapping x; those of the calls it
 * makes; PI_EHIP when a copy, an event record or a wait fails.  After an error
 * the list sets may be partly written: call pi_hybrid_prime again before the
 * next layer. */
int pi_hybrid_prime(void* stream, const pi_layer* layer, const int32_t* T_g, const int32_t* T_c, int32_t n_c,
                    int32_t B, const float* x, float tau, pi_hybrid_ahead_scratch* scratch);
int pi_hybrid_layer_ahead(void* stream, const pi_layer* layer, const pi_host_cold* cold, const pi_layer* next,
                          const int32_t* T_g_next, const int32_t* T_c_next, int32_t n_c_next, int32_t B,
                          const float* x, float tau, float* y, pi_hybrid_ahead_scratch* scratch, int32_t threads,
                          int32_t* K_c_out);

/* A stack of n_layers look-ahead hybrid layers in one call: pi_hybrid_prime on
 * layer 0 and xs[0], then pi_hybrid_layer_ahead on each layer l with its input
 * xs[l] and output ys[l] (device [B x d] each), next = layer l + 1.  The
 * executor loop of one decode step over the FFN layers, for callers whose
 * layers' inputs are ready (layers[l], colds[l], T_g[l], T_c[l], n_c[l] per
 * layer; colds[l] NULL for a layer without CPU rows).  K_c_out (optional,
 * n_layers entries) gets each layer's K_c.
 * Errors: PI_EINVAL for n_layers < 1 or a NULL array; those of the calls. */
int pi_hybrid_stack_ahead(void* stream, int32_t n_layers, const pi_layer* layers, const pi_host_cold* const* colds,
                          const int32_t* const* T_g, const int32_t* const* T_c, const int32_t* n_c, int32_t B,
                          const float* const* xs, float tau, float* const* ys, pi_hybrid_ahead_scratch* scratch,
                          int32_t threads, int32_t* K_c_out);

#ifdef __cplusplus
}
#endif

#endif /* PI_HOST_H */
