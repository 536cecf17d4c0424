/* oracle.h - plain, slow CPU oracle for the neuron-aware sparse FFN.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library; the product path never
 * calls it.  It shares no code with the HIP library.
 *
 * Every stored element (fp32, fp16, or int4 times its fp16 group scale) is
 * widened to double exactly and all arithmetic is done in double, in the
 * plain order of the definitions, one output element per thread.
 *
 * Sources (PowerInfer, as summarised by the pages):
 *  - CSDN summary "PowerInfer: Fast Large Language Model Serving with a
 *    Consumer-grade GPU", background part on the MLP block (FC1, ReLU, FC2;
 *    each output element is the dot product of the input with a neuron, and
 *    ReLU keeps only the positive FC1 neurons).
 *  - same page, section "自适应稀疏预测器" (adaptive sparsity predictor: an MLP
 *    with an input, a hidden and an output layer).
 *  - same page, section "神经元放置和管理" (two neuron tables mapping each
 *    neuron to its original position in the matrix).
 *  - same page, section "GPU-CPU混合执行" (each unit computes its own active
 *    neurons; results merged on the GPU; merge skipped when the CPU side has no
 *    active neuron).
 *  - same page, section "神经元-觉察算子" (first decide whether a neuron is
 *    active, then process its row or column of the weight matrix).
 *  - same page, background part on the MLP block (its output goes on to the
 *    next layer): or_layer_norm, the normalisation that turns one layer's
 *    output into the next layer's input in a chained stack, is not on the
 *    pages; it is a reading (layer normalisation with unit gain and zero
 *    bias, as in front of each FFN of the OPT models the pages serve).
 */
#ifndef PI_ORACLE_H
#define PI_ORACLE_H
#include <stdint.h>

enum { OR_F32 = 0, OR_F16 = 1, OR_I4G128 = 2 };
enum { OR_RELU = 0, OR_GATED_RELU = 1 };

typedef struct {
  const void* data;        /* host, rows x cols row-major in `dtype` */
  const uint16_t* scales;  /* fp16 bits [rows x cols/128], int4 only */
  int32_t dtype;
  int64_t cols;
} or_mat;

typedef struct {
  const void* data;        /* host, NULL = all zeros */
  int32_t dtype;           /* OR_F32 or OR_F16 */
} or_vec;

double or_f16_to_double(uint16_t h);
double or_mat_at(or_mat m, int64_t row, int64_t col);
double or_vec_at(or_vec v, int64_t i);

/* h[b,m] = max(0, sum_k P1[m,k] x[b,k] + c1[m]);  l[b,i] = sum_m P2[i,m] h[b,m] + c2[i].
 * h_out [B x H] may be NULL. */
void or_predict(int B, int d, int H, int N, const float* x, or_mat P1, or_vec c1,
                or_mat P2, or_vec c2, double* h_out, double* logits);

/* M_i = OR over b of (float)logit[b,i] > tau (the comparison is made in fp32).
 * A_g = ascending slots s < n_g with M[T_g[s]]; *K = |A_g|.
 * If T_c != NULL: A_c = ascending slots c < n_c with M[T_c[c]]; *K_c = |A_c|. */
void or_compact(int B, int N, const double* logits, float tau, const int32_t* T_g, int n_g,
                int32_t* A_g, int32_t* K, const int32_t* T_c, int n_c, int32_t* A_c, int32_t* K_c);

/* Neuron-aware FFN over the rows listed in `rows` (K of them, indices into the
 * given matrices):  a[b,j] = max(0, W1[r_j].x_b + b1[r_j])  (ReLU), or
 * max(0, W1[r_j].x_b + b1[r_j]) * (Wup[r_j].x_b)  (gated);
 * y[b,:] = sum_j a[b,j] W2[r_j,:].   a_out [B x K] may be NULL. */
void or_sparse_ffn(int B, int d, int kind, const float* x, or_mat W1, or_vec b1, or_mat Wup,
                   or_mat W2, const int32_t* rows, int K, double* a_out, double* y);

/* Dense FFN over all n rows (the same sum with rows = 0..n-1). */
void or_dense_ffn(int B, int d, int n, int kind, const float* x, or_mat W1, or_vec b1, or_mat Wup,
                  or_mat W2, or_vec b2, double* y);

/* y = y_g + y_c (+ b2): y_c is added only when y_c != NULL and K_c != 0. */
void or_merge(int B, int d, const double* y_g, const double* y_c, int K_c, or_vec b2, double* y);

/* Chained layers:  x[b,k] = (y[b,k] - mu_b) / sqrt(var_b + eps), with mu_b the
 * mean and var_b the population variance (divided by d) of row b of y [B x d].
 * In-place use (x aliasing y) is not supported: y is fp32, x is double. */
void or_layer_norm(int B, int d, const float* y, double eps, double* x);

/* Threads the oracle's OpenMP loops may use (0 = library default). */
void or_set_threads(int n);
int or_get_threads(void);

#endif
