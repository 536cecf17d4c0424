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
 * Every pointer here is a HOST pointer owned by the caller.  Matrix formats
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
 *   y_c[b,:] = sum_j a[b,j] * W2[c,:]   (list order; a neuron whose a is 0 in
 *                                        every batch row adds nothing and its
 *                                        W2 row is not read)
 * x [B x d] fp32; A_c [K_c] int32 (the CPU-table slots pi_compact lists);
 * y_c [B x d] fp32, fully written (zero when K_c = 0).  threads: the number
 * of threads (<= 0: the OpenMP default).  Host scratch of B * K_c floats is
 * allocated for the FC1 outputs.
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

#ifdef __cplusplus
}
#endif

#endif /* PI_HOST_H */
