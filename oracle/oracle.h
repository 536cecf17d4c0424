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
 *  - same page, background part on activation sparsity and section
 *    "自适应稀疏预测器": or_attn_decode, the self-attention block with head
 *    sparsity (see its declaration).
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

/* fp16 bits of v, rounded to nearest with ties to even (IEEE binary16: overflow to
 * infinity, gradual underflow to subnormals). */
uint16_t or_double_to_f16(double v);

/* Self-attention block with head sparsity at decode, one new token at position t
 * (CSDN summary, background part on activation sparsity: in the self-attention
 * block nearly half of the heads contribute little, a sparsity of its own; section
 * "自适应稀疏预测器": each layer has a predictor for the self-attention block beside
 * the one for the MLP block, and computation is limited to what is predicted active).
 *   head predictor  s_h = ca2[h] + sum_m Pa2[h,m] max(0, Pa1[m].x + ca1[m])  (or_predict
 *                   with N = n_heads); head h active iff (float)s_h > tau; heads[] the
 *                   active heads ascending, *n_active their count;
 *   cache entry     k_new = fp16(Wk.x + bk), v_new = fp16(Wv.x + bv) for every head (the
 *                   entry at position t, which later tokens attend to whatever this
 *                   token's prediction);
 *   attention       for active h with q = (Wq.x + bq)[h d_h .. h d_h + d_h - 1]:
 *                   e_j = q . K_h[j] / sqrt(d_h) for j = 0..t, where K_h[j] is the cache's
 *                   entry for j < t and k_new's head-h part for j = t (likewise V);
 *                   o_h = sum_j softmax(e)_j V_h[j];
 *   output          y = bo + sum over active h and i < d_h of o_h[i] WoT[h d_h + i, :].
 * Weights: Wq, Wk, Wv [d x d] with row r the output element r (head r / d_h); WoT [d x d]
 * with row h d_h + i the output-projection weights of head h's element i; Pa1 [Ha x d],
 * Pa2 [n_heads x Ha].  Kc, Vc: fp16 bits [n_heads x L_max x d_h] (positions 0..t-1 read).
 * head_logits [n_heads], heads [n_heads], k_new, v_new [d] (fp16 bits), y [d]. */
void or_attn_decode(int d, int n_heads, int d_h, int Ha, int t, const float* x, or_mat Pa1, or_vec ca1,
                    or_mat Pa2, or_vec ca2, float tau, or_mat Wq, or_vec bq, or_mat Wk, or_vec bk, or_mat Wv,
                    or_vec bv, or_mat WoT, or_vec bo, const uint16_t* Kc, const uint16_t* Vc, int L_max,
                    double* head_logits, int32_t* heads, int32_t* n_active, uint16_t* k_new, uint16_t* v_new,
                    double* y);

/* Threads the oracle's OpenMP loops may use (0 = library default). */
void or_set_threads(int n);
int or_get_threads(void);

#endif
