/* pi.h - C ABI of libpi, the MI355X (gfx950) neuron-aware sparse FFN.
 *
 * The operation, per decoded token and FFN layer, follows PowerInfer as the
 * pages describe it:
 *   1. a small per-layer MLP predictor marks the neurons that will fire
 *      (CSDN summary of "PowerInfer: Fast Large Language Model Serving with a
 *      Consumer-grade GPU", section 自适应稀疏预测器; unite.ai French article
 *      "PowerInfer : Moteur d'inférence ...", section "Prévisionnistes de
 *      rareté adaptatifs");
 *   2. the active neurons are looked up through the GPU neuron table, which
 *      maps each GPU-resident neuron to its original position in the weight
 *      matrices (CSDN summary, section 神经元放置和管理; French article,
 *      section "Placement et gestion des neurones");
 *   3. only those neurons' FC1 rows are multiplied, ReLU keeps the positive
 *      ones, and only the matching FC2 rows (a neuron's FC2 column, stored
 *      neuron-major) are accumulated (CSDN summary, background part on the MLP
 *      block and section 神经元-觉察算子; French article, section "Opérateur
 *      sensible aux neurones");
 *   4. the partial result computed elsewhere for the cold neurons is merged
 *      on the GPU, and the merge is skipped when there is none (CSDN summary,
 *      section GPU-CPU混合执行).
 *
 * Conventions shared by every entry point
 *  - Every array argument is a DEVICE pointer owned by the caller, 16-byte
 *    aligned.  The library never allocates, frees or synchronises, and never
 *    reads device memory from the host.  Work is enqueued on `stream` (a
 *    hipStream_t; NULL = the null stream) in the order of the calls.
 *  - Matrices are row-major.  Row r of a [rows x cols] matrix starts at
 *    r * row_bytes, row_bytes = cols * 4 (PI_F32), cols * 2 (PI_F16) or
 *    cols / 2 (PI_I4G128).  cols must be a multiple of 8 (PI_F32, PI_F16) or
 *    of 128 (PI_I4G128).
 *  - PI_I4G128: symmetric int4, two elements per byte, even element in the
 *    low nibble, two's-complement value q in [-8, 7]; element value is
 *    q * scale, one fp16 scale per 128 consecutive elements of a row,
 *    scales[rows x cols/128].
 *  - Counts (K, K_c) stay on the device, so a decode step needs no host
 *    synchronisation.  Grids are bounded by the table sizes.
 *  - Return value: PI_OK, or an error status with nothing enqueued
 *    (PI_EINVAL, PI_EWORKSPACE, PI_EUNSUPPORTED), or PI_EHIP when the HIP
 *    launch itself failed (pi_last_hip_error() then gives the hipError_t of
 *    this thread's last failure).  Device faults surface at the caller's next
 *    synchronisation.  No entry point prints, aborts or throws.
 *  - Results are bitwise repeatable: the same inputs give the same bits.
 *  - The library holds no mutable global state other than each thread's
 *    last HIP error (pi_last_hip_error) and the static workspace of
 *    pi_ffn_layer_static (one per GPU, with its address kept per device);
 *    calls on different streams with disjoint outputs and workspaces may run
 *    concurrently.
 */
#ifndef PI_H
#define PI_H
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PI_ABI_VERSION 3
#define PI_MAX_BATCH 32
/* Largest neuron count N of pi_compact and the layer entry points: each
 * workgroup that builds the active lists holds the activation decision of
 * every neuron id in its LDS. */
#define PI_MAX_NEURONS 65536

enum pi_dtype { PI_F32 = 0, PI_F16 = 1, PI_I4G128 = 2 };
enum pi_ffn_kind { PI_RELU = 0, PI_GATED_RELU = 1 };
enum pi_status { PI_OK = 0, PI_EINVAL = 1, PI_EWORKSPACE = 2, PI_EUNSUPPORTED = 3, PI_EHIP = 4 };
enum pi_op { PI_OP_PREDICT = 0, PI_OP_COMPACT = 1, PI_OP_SPARSE_FFN = 2, PI_OP_MERGE = 3, PI_OP_FFN_LAYER = 4,
             PI_OP_PREDICT_OUTPUT = 5, PI_OP_FFN_LAYER_NORMED = 6 };

/* A weight matrix on the device.  `scales` is used by PI_I4G128 only. */
typedef struct pi_matrix {
  const void* data;
  const uint16_t* scales;
  int32_t dtype; /* enum pi_dtype */
} pi_matrix;

/* A bias vector on the device, PI_F32 or PI_F16.  data == NULL means zero. */
typedef struct pi_vector {
  const void* data;
  int32_t dtype;
} pi_vector;

/* Predictor (step 1).  For each batch row b < B:
 *   h[b,m]      = max(0, sum_k P1[m,k] * x[b,k] + c1[m])      m < H
 *   logits[b,i] = sum_m P2[m,i] * h[b,m] + c2[i]               i < N
 * x      [B x d] fp32.   P1 [H x d] (row m = hidden unit m's input weights).
 * P2 [H x N] HIDDEN-MAJOR: row m holds hidden unit m's weights to the N
 * outputs, the same neuron-major convention as W2 below, so that a hidden
 * unit whose ReLU output is zero is one row that need not be read.  Both
 * PI_F32/PI_F16/PI_I4G128 (int4 groups run along the row, i.e. along N).
 * logits [B x N] fp32, written.   h lives in the workspace.
 * Precision: fp32 accumulation.  With fp16 weights and B >= 2 the matrix
 * cores take x and h each as two fp16 parts, hi = fp16(v) and lo =
 * fp16(v - hi) (about 22 bits; every product exact), so |x| and |h| must
 * stay below 65504, fp16's largest value: a larger value becomes infinite,
 * and so do the logits it reaches.
 * ws: at least pi_workspace_bytes(PI_OP_PREDICT, B, d, H, N, 0) bytes.
 * Errors: PI_EINVAL for a NULL required pointer, B outside 1..PI_MAX_BATCH,
 * a non-positive size, a column count the dtype forbids (d for P1, N for P2)
 * or an unknown dtype; PI_EWORKSPACE for a short workspace. */
int pi_predict(void* stream, int32_t B, int32_t d, int32_t H, int32_t N, const float* x,
               pi_matrix P1, pi_vector c1, pi_matrix P2, pi_vector c2,
               float* logits, void* ws, size_t ws_bytes);

/* The predictor's output layer alone, with the activation decision:
 *   logits[b,i] = sum_m P2[m,i] * h[b,m] + c2[i]                i < N
 *   mask bit i  = (logits[b,i] > tau for some b < B)
 * h [B x H] fp32 (the hidden layer, e.g. from a previous pi_predict); P2
 * hidden-major as for pi_predict.  logits [B x N] fp32 (may be NULL when
 * B == 1 and H <= 4096: not stored).  mask (optional, NULL = not stored):
 * 2*ceil(N/64) uint32 words, bit i%32 of word i/32; bits of ids >= N are
 * zero.  ws: pi_workspace_bytes(PI_OP_PREDICT_OUTPUT, B, 0, H, N, 0) bytes
 * (zero at batch 1 with H <= 4096; ws may then be NULL).
 * Errors: as pi_predict. */
int pi_predict_output(void* stream, int32_t B, int32_t H, int32_t N, const float* h, pi_matrix P2, pi_vector c2,
                      float tau, float* logits, uint32_t* mask, void* ws, size_t ws_bytes);

/* Activation decision and compaction (step 2).
 * Neuron i is active when logits[b,i] > tau (fp32 compare) for SOME b < B
 * (the union over the batch).
 *   A_g[0..K)   = the slots s < n_g with T_g[s] active, ascending; *K = count
 *   A_c[0..K_c) = the slots c < n_c with T_c[c] active, ascending; *K_c = count
 * T_g [n_g] int32: slot -> original neuron id (the GPU neuron table); the
 * ids must lie in [0, N).  T_c [n_c] (optional, NULL = no cold side): the
 * CPU neuron table.  A_g needs n_g entries, A_c n_c.  K, K_c: one device
 * int32 each.  ws may be NULL (pi_workspace_bytes returns 0).
 * Errors: PI_EINVAL for a NULL required pointer, B outside 1..PI_MAX_BATCH,
 * n_g < 0, N <= 0, or T_c given without A_c/K_c; PI_EUNSUPPORTED for
 * N > PI_MAX_NEURONS. */
int pi_compact(void* stream, int32_t B, int32_t N, const float* logits, float tau,
               const int32_t* T_g, int32_t n_g, int32_t* A_g, int32_t* K,
               const int32_t* T_c, int32_t n_c, int32_t* A_c, int32_t* K_c,
               void* ws, size_t ws_bytes);

/* Neuron-aware FFN over the GPU-resident neurons (step 3).
 * W1, W2 (and Wup) hold the n_g GPU-resident neurons in slot order,
 * [n_g x d] each; W2 is stored neuron-major (row s = the FC2 column of the
 * neuron in slot s).  For j < *K, s = A_g[j]:
 *   a[b,j] = max(0, W1[s].x_b + b1[s])                    (PI_RELU)
 *   a[b,j] = max(0, W1[s].x_b + b1[s]) * (Wup[s].x_b)     (PI_GATED_RELU)
 *   y_g[b,:] = sum_j a[b,j] * W2[s,:]                      (fixed-order sum)
 * x [B x d] fp32; b1 [n_g]; y_g [B x d] fp32, fully written (zero if K = 0).
 * A_g entries must be < n_g; *K <= n_g.
 * Precision: accumulation is fp32.  With fp16 weights and B >= 2 the matrix
 * cores take x rounded to fp16 for FC1, and from B >= 3 the FC1 outputs a
 * (after the gate's product) rounded to fp16 for FC2 (each product of two
 * fp16 values is exact), so |x| and |a| must stay below 65504, fp16's
 * largest value: a larger value becomes infinite, and so does y.  The
 * predictor's logits keep near-fp32 precision (x and h enter it as two fp16
 * parts each).  Other cases use fp32 products.
 * ws: at least pi_workspace_bytes(PI_OP_SPARSE_FFN, B, d, 0, 0, n_g) bytes.
 * Errors: as pi_predict, plus PI_EINVAL for a kind outside PI_RELU /
 * PI_GATED_RELU or a gated call without Wup, and PI_EUNSUPPORTED when W1,
 * Wup and W2 do not share one dtype. */
int pi_sparse_ffn(void* stream, int32_t B, int32_t d, int32_t n_g, int32_t kind, const float* x,
                  pi_matrix W1, pi_vector b1, pi_matrix Wup, pi_matrix W2,
                  const int32_t* A_g, const int32_t* K, float* y_g, void* ws, size_t ws_bytes);

/* Merge (step 4):  y[b,:] = y[b,:] + y_c[b,:] + b2   (in place, [B x d] fp32).
 * y_c (device [B x d] fp32, the cold-neuron partial) is added only when it
 * is non-NULL and, if K_c is non-NULL, *K_c != 0: with no active cold neuron
 * the cold partial is skipped.  b2.data == NULL adds no bias.
 * Errors: PI_EINVAL for a NULL y, B outside 1..PI_MAX_BATCH or d <= 0. */
int pi_merge(void* stream, int32_t B, int32_t d, float* y, const float* y_c, const int32_t* K_c,
             pi_vector b2);

/* ---------------------------------------------------------------------------
 * Prepared neuron table and the fused layer call.
 *
 * The GPU neuron table T_g (slot -> original neuron id) in the form the fused
 * kernels read: a bitmap of the GPU-resident original ids (one bit per id,
 * 32 per word), then, for each group of 64 ids, the number of GPU-resident
 * ids below the group.  The
 * slot of a GPU-resident id is then its rank among the GPU-resident ids,
 * which is what T_g gives when T_g is ascending; the CPU table is the
 * ascending complement (CSDN summary, section 神经元放置和管理: one table per
 * processing unit, both mapping neurons to their original positions).
 * ------------------------------------------------------------------------- */

/* Bytes of a prepared table for N neurons. */
size_t pi_table_bytes(int32_t N);

/* Host-only (no HIP call): build the prepared table of T_g into the HOST
 * buffer `table` (pi_table_bytes(N) bytes); the caller copies it to the
 * device.  T_g [n_g] host int32 must be strictly ascending with ids in
 * [0, N).  Errors: PI_EINVAL (NULL pointers, N <= 0, n_g outside 0..N, an id
 * out of range or out of order), PI_EWORKSPACE (buffer too small). */
int pi_table_prepare(int32_t N, const int32_t* T_g, int32_t n_g, void* table, size_t table_bytes);

/* One FFN layer, all four steps: predictor, activation decision and
 * compaction, neuron-aware FFN over the GPU-resident neurons, merge.
 * Weights as for the separate calls (P2 hidden-major); `table` is a device copy of the
 * prepared table of the layer's T_g (W1, b1, Wup, W2 in that T_g's slot
 * order).  With `cold` non-zero the neurons outside T_g are CPU-resident and
 * their active ascending slots in the CPU table are listed in A_c / K_c. */
typedef struct pi_layer {
  int32_t d, N, H, n_g;
  int32_t kind; /* PI_RELU | PI_GATED_RELU */
  int32_t cold; /* non-zero: produce the CPU-side list A_c, K_c */
  pi_matrix P1;
  pi_vector c1;
  pi_matrix P2;
  pi_vector c2;
  const void* table;
  pi_matrix W1;
  pi_vector b1;
  pi_matrix Wup;
  pi_matrix W2;
  pi_vector b2;
} pi_layer;

/* y[b,:] = sum over active GPU-resident neurons (as pi_sparse_ffn)
 *          + y_c[b,:] when y_c != NULL and (cold == 0 or *K_c != 0)
 *          + b2.
 * x [B x d] fp32, y [B x d] fp32 written.  logits [B x N] (optional, NULL =
 * not stored).  A_g [n_g] and K (device) receive the GPU list and its count;
 * A_c [N - n_g] and K_c the CPU list when cold != 0 (else they may be NULL).
 * ws: pi_workspace_bytes(PI_OP_FFN_LAYER, B, d, H, N, n_g) bytes.
 * events: NULL, or 6 hipEvent_t (any may be NULL) recorded on `stream`
 * before the first kernel and after each stage: the predictor hidden layer,
 * the output layer with the activation decision, FC1, FC2, and the final
 * ordered sum with the merge (per-stage timing).  At batch 1 the output
 * layer, the decision and FC1 run as one kernel per tile of neuron ids
 * (events 2 and 3 are then recorded together) and FC2 also writes the lists.
 * Errors: as the separate calls (PI_EUNSUPPORTED for N > PI_MAX_NEURONS). */
int pi_ffn_layer(void* stream, const pi_layer* layer, int32_t B, const float* x, float tau,
                 const float* y_c, float* y, float* logits, int32_t* A_g, int32_t* K,
                 int32_t* A_c, int32_t* K_c, void* ws, size_t ws_bytes, void* const* events);

/* pi_ffn_layer for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The same call without ws / ws_bytes / events: the workspace is a static
 * device array of PI_STATIC_WORKSPACE_BYTES inside the library, one per GPU,
 * held until the process ends; the entry point allocates nothing and frees
 * nothing (its first call on a device looks up that device's array address).
 * 16 MiB holds batch 1 at every shape this library is measured on (up to
 * d = 12288, N = 49152, H = 4096) and batch 4 at d = 7168, N = 28672.
 * Every call on one GPU shares that GPU's array and the array keeps the last
 * call's contents: calls that overlap on one GPU (other streams or threads)
 * race and give undefined results.  No part of the array needs to start at
 * zero (each call writes what it reads).
 * Errors: PI_EWORKSPACE when pi_workspace_bytes(PI_OP_FFN_LAYER, B, d, H, N,
 * n_g) exceeds PI_STATIC_WORKSPACE_BYTES (nothing enqueued; use pi_ffn_layer
 * with a caller workspace); PI_EUNSUPPORTED for a device index of 64 or more;
 * PI_EHIP when the device or the array's address cannot be read; otherwise as
 * pi_ffn_layer. */
#define PI_STATIC_WORKSPACE_BYTES (16u << 20)
int pi_ffn_layer_static(void* stream, const pi_layer* layer, int32_t B, const float* x, float tau,
                        const float* y_c, float* y, float* logits, int32_t* A_g, int32_t* K, int32_t* A_c,
                        int32_t* K_c);

/* Stages of pi_ffn_layer, as bits. */
enum pi_stage {
  PI_STAGE_HIDDEN = 1, /* predictor hidden layer -> h in the workspace */
  PI_STAGE_OUTPUT = 2, /* output layer + activation decision (+ lists / FC1 segments) */
  PI_STAGE_FC1 = 4,    /* FC1 over the active GPU-resident neurons */
  PI_STAGE_FC2 = 8,    /* FC2 partial sums (+ lists at batch 1) */
  PI_STAGE_SUM = 16,   /* ordered sum of the partials + merge -> y */
  PI_STAGE_ALL = 31
};

/* pi_ffn_layer restricted to the stages in `stages` (a non-zero subset of
 * PI_STAGE_ALL), for timing and profiling one kernel in isolation, with an
 * optional report of the weight rows read.  A stage enqueued without the
 * stages before it reads what an earlier call with the same layer, inputs and
 * workspace left in the workspace; with PI_STAGE_ALL and rows_read == NULL it
 * is pi_ffn_layer.  At batch 1 PI_STAGE_OUTPUT and PI_STAGE_FC1 name the same
 * kernel.
 * rows_read (optional device int32[2], written when the whole layer runs):
 * [0] the rows of P2 read (at batch 1 only the hidden units with h > 0;
 * else H), [1] the rows of W2 read (at batch 1 only the listed neurons whose
 * FC1 output is non-zero, the only ones that add to y; else K).
 * Errors: as pi_ffn_layer, plus PI_EINVAL for an empty or unknown stage
 * set. */
int pi_ffn_layer_stages(void* stream, const pi_layer* layer, int32_t B, const float* x, float tau,
                        const float* y_c, float* y, float* logits, int32_t* A_g, int32_t* K,
                        int32_t* A_c, int32_t* K_c, void* ws, size_t ws_bytes, void* const* events,
                        uint32_t stages, int32_t* rows_read);

/* Look-ahead prediction (a variant of the method; the pages note that
 * activations can be predicted some layers ahead while the model runs):
 * pi_ffn_layer_stages on `layer` (events and rows_read not taken), and the
 * predictor hidden layer of `next` computed from this call's x, the input of
 * `layer`, into the workspace ws_next.  A later call on `next` with its own
 * input and without PI_STAGE_HIDDEN then predicts `next`'s neurons from
 * `layer`'s input.  At batch 1, when next->P1 has the format of layer->W1,
 * the hidden rows are computed by extra workgroups of the launch that runs
 * `layer`'s output layer and FC1, on the x it stages; otherwise by the
 * separate hidden-layer kernels after `layer`'s stages.
 * next: d equal to layer->d; its P1, c1, H, N and n_g are used.  ws_next:
 * pi_workspace_bytes(PI_OP_FFN_LAYER, B, d, next->H, next->N, next->n_g)
 * bytes, not ws.
 * x and y may not overlap (the next layer's hidden layer can run after y is
 * written), and neither may ws and ws_next (compared as byte ranges).
 * Errors: as pi_ffn_layer_stages; PI_EINVAL for a NULL next, another d, a bad
 * P1 / c1 of next, x overlapping y, or ws overlapping ws_next; PI_EWORKSPACE
 * for a short ws_next. */
int pi_ffn_layer_ahead(void* stream, const pi_layer* layer, int32_t B, const float* x, float tau,
                       const float* y_c, float* y, float* logits, int32_t* A_g, int32_t* K,
                       int32_t* A_c, int32_t* K_c, void* ws, size_t ws_bytes, uint32_t stages,
                       const pi_layer* next, void* ws_next, size_t ws_next_bytes);

/* Chained layers: the next layer's input from this layer's output (CSDN
 * summary, background part on the MLP block: the block's output goes on to
 * the next layer).  The pages name no normalisation between layers; the
 * reading here is layer normalisation with unit gain and zero bias, as in
 * front of each FFN of the OPT models they serve:
 *   x[b,k] = (y[b,k] - mean_b) / sqrt(var_b + eps),
 * mean_b and the population variance var_b (divided by d) over row b.
 * y, x: device [B x d] fp32 row-major; x may be y itself (in place) but may
 * not overlap it otherwise.  One workgroup per row; fp32 sums in a fixed
 * order, so the result is bitwise repeatable.  A constant row gives zeros
 * (eps > 0).  Rows whose squares overflow fp32 give inf/NaN, as the formula
 * in fp32 does.  No workspace.
 * Errors: PI_EINVAL for a NULL pointer, B <= 0, d outside 1..2^30, eps
 * negative or not finite, or x overlapping y without being equal to it. */
int pi_layer_norm(void* stream, int32_t B, int32_t d, const float* y, float eps, float* x);

/* Chained layers without the separate normalisation launch: pi_ffn_layer on
 * x = the layer normalisation of y_prev (as pi_layer_norm: unit gain, zero
 * bias, population variance, eps), with y_prev being the previous layer's
 * output.  At batch 1, where the layer runs its fused kernels, the predictor's
 * hidden-layer kernel normalises the row it holds and leaves the mean and
 * 1/sqrt(var + eps) in the workspace, and the output-layer + FC1 kernel
 * normalises x with those same two values, so the predictor and FC1 see the
 * same x bit for bit; no other launch is added.  Other batches and formats run
 * pi_layer_norm into the workspace (or x_out) first, then the layer.  The
 * statistics are fp32 sums in a fixed order, so results are bitwise
 * repeatable; the batch-1 sums run in another order than pi_layer_norm's, so
 * they may differ from pi_layer_norm + pi_ffn_layer in the last bits.
 * y_prev: device [B x d] fp32, 16-byte aligned; it may be y itself (or overlap
 * it): every read of y_prev comes before y is written.  x_out: NULL, or device
 * [B x d] fp32, 16-byte aligned, receiving the normalised input (e.g. for a
 * host-side cold FFN); it may overlap neither y_prev nor y.  Other arguments as
 * pi_ffn_layer.  ws: pi_workspace_bytes(PI_OP_FFN_LAYER_NORMED, B, d, H, N,
 * n_g) bytes.
 * Errors: as pi_ffn_layer and pi_layer_norm; PI_EINVAL for a NULL or
 * unaligned y_prev, an unaligned x_out, x_out overlapping y_prev or y, or eps
 * negative or not finite; PI_EWORKSPACE for a short or unaligned ws. */
int pi_ffn_layer_normed(void* stream, const pi_layer* layer, int32_t B, const float* y_prev, float eps,
                        float tau, const float* y_c, float* y, float* logits, int32_t* A_g, int32_t* K,
                        int32_t* A_c, int32_t* K_c, float* x_out, void* ws, size_t ws_bytes);

/* ---- Self-attention block with head sparsity at decode (batch 1) ----
 * The pages note that in the self-attention block nearly half of the heads
 * contribute little, a sparsity of its own beside the MLP block's (CSDN
 * summary, background part on activation sparsity), and that a predictor per
 * block (self-attention and MLP) limits the computation to what it predicts
 * active (same page, section 自适应稀疏预测器).  One new token at position t:
 *   head predictor  s_h = ca2[h] + Pa2[h] . max(0, Pa1 x + ca1) (the MLP of
 *                   pi_predict with one output per head); head h is active iff
 *                   s_h > tau (in fp32);
 *   cache entry     K and V rows of every head: Kc[h][t] = fp16(Wk x + bk)
 *                   (head h's part), Vc likewise (later tokens attend to this
 *                   position whatever this token's prediction);
 *   attention       active h only: q_h = (Wq x + bq)[h*dh ..]; over positions
 *                   j = 0..t of the cache, softmax(q_h . Kc[h][j] / sqrt(dh))
 *                   weights the rows Vc[h][j] into o_h;
 *   output          y = bo + sum over active h of WoT[h*dh + i, :] o_h[i].
 * A predicted-inactive head reads none of its query or output-projection
 * rows and none of its cached positions. */
typedef struct {
  int32_t d;       /* model width, n_heads * dh */
  int32_t n_heads; /* 1 .. 256 */
  int32_t dh;      /* 64 or 128 */
  int32_t Ha;      /* head predictor hidden size: a multiple of 4, at most 1024 */
  int32_t L_max;   /* cache capacity in positions */
  pi_matrix Pa1;   /* [Ha x d] */
  pi_vector ca1;   /* [Ha] or NULL */
  pi_matrix Pa2;   /* [n_heads x Ha], row per head */
  pi_vector ca2;   /* [n_heads] or NULL */
  pi_matrix Wq;    /* [d x d], row r = query element r (head r / dh) */
  pi_vector bq;
  pi_matrix Wk;    /* [d x d] */
  pi_vector bk;
  pi_matrix Wv;    /* [d x d] */
  pi_vector bv;
  pi_matrix WoT;   /* [d x d], row h*dh + i = output-projection weights of head h's element i */
  pi_vector bo;
  uint16_t* Kc;    /* device fp16 [n_heads x L_max x dh]: a head's positions are contiguous */
  uint16_t* Vc;    /* device fp16 [n_heads x L_max x dh] */
} pi_attn;

/* One decode step of the attention block above.  Every matrix is fp16
 * (PI_F16) and every bias fp16 or NULL; d at most 8192.  x [d] fp32, y [d]
 * fp32 written; head_logits [n_heads] fp32 (optional, NULL = not stored);
 * heads [n_heads] and *n_active (device int32) receive the ascending active
 * heads and their count.  Positions 0..t-1 of the caches are read, position t
 * is written for every head, and no other position is touched.
 * ws: pi_attn_workspace_bytes(A) bytes, 16-byte aligned.  All pointers are
 * device pointers except A.  Results are bitwise repeatable.
 * Errors: PI_EINVAL for a NULL or unaligned pointer, t outside 0..L_max-1,
 * inconsistent sizes, a matrix or bias of another dtype, or y overlapping x;
 * PI_EUNSUPPORTED for dh other than 64 / 128, d above 8192, more than 256
 * heads or Ha outside the bounds; PI_EWORKSPACE for a short workspace. */
int pi_attn_decode(void* stream, const pi_attn* A, int32_t t, const float* x, float tau, float* y,
                   float* head_logits, int32_t* heads, int32_t* n_active, void* ws, size_t ws_bytes);

/* Workspace bytes of pi_attn_decode for this block (0 for NULL). */
size_t pi_attn_workspace_bytes(const pi_attn* A);

/* The streaming-read reference that the kernels' bandwidths are read against:
 * reads `bytes` bytes of `buf` once, in 16-byte vectors, grid-stride, with
 * `blocks` workgroups of 256 threads (blocks <= 0: PI_READ_PROBE_BLOCKS_PER_CU
 * per compute unit) each keeping `depth` loads per lane in flight (4, 8, 16
 * or 32; 0: PI_READ_PROBE_DEPTH), and writes the XOR of the words each wave
 * read to out[4 * block + wave] (so that no load can be dropped).  The
 * defaults are the fastest setting of a sweep over depth and grid size on
 * MI355X.
 * buf: device, 16-byte aligned; bytes a multiple of 16; out: device uint32
 * [4 * blocks].  Errors: PI_EINVAL for a NULL pointer, bytes == 0 or not a
 * multiple of 16, blocks > 65536, or another depth. */
#define PI_READ_PROBE_DEPTH 16
#define PI_READ_PROBE_BLOCKS_PER_CU 8
int pi_read_probe(void* stream, const void* buf, size_t bytes, int32_t blocks, int32_t depth, uint32_t* out);

/* Environment: PI_MATRIX_CORE_MIN_BATCH, read once at the first call, raises
 * the smallest batch that takes the matrix-core GEMMs (by default batch 2 for
 * the row-dot GEMMs, the predictor's hidden layer and FC1, and batch 3 for the
 * axpy GEMMs, the output layer and FC2); a value above 32 keeps every batch on
 * the VALU kernels.  It exists for comparisons; pi_workspace_bytes follows it. */

/* Workspace bytes an entry point needs for these sizes (0 when none).
 * Arguments an op does not use are ignored. */
size_t pi_workspace_bytes(int32_t op, int32_t B, int32_t d, int32_t H, int32_t N, int32_t n_g);

/* Static description of a status code. */
const char* pi_status_string(int32_t status);

/* hipError_t of the calling thread's last PI_EHIP (0 if none). */
int32_t pi_last_hip_error(void);

/* PI_ABI_VERSION the library was built with. */
int32_t pi_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif
