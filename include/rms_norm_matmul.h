/*
 * RMSNorm-fused matrix product on AMD CDNA4 (gfx950, MI355X): C ABI.
 *
 * Computes, as the fused kernel of the docs.rs source page of meganeura
 * 0.2.0, src/shaders/matmul_rms_norm.wgsl (its header comment, the per-row
 * rsqrt prologue and the normalise-on-load A staging) does:
 *
 *   r[i]    = 1 / sqrt(sum_k x[i, k]^2 / k + eps)
 *   C[i, j] = sum_k (x[i, k] * r[i] * norm_weight[k]) * proj[k, j]
 *
 * Layouts (dense, row-major, fp32 in device memory):
 *   x            [m, k]   the raw activations (read)
 *   norm_weight  [k]      the RMSNorm scale (read)
 *   proj         [k, n]   the projection weight (read)
 *   out          [m, n]   C (fully overwritten)
 *
 * fp32 operands on the fp32 matrix cores (v_mfma_f32_16x16x4_f32), fp32
 * accumulation; the row sums of squares are taken from the same staged
 * tiles in fp32 and the factor r[i] is applied to the finished row, so the
 * rounding order differs from the page's (normalise, then multiply) by fp32
 * rounding only.  Asynchronous on `stream` (a hipStream_t; NULL: the null
 * stream).
 *
 * Status codes are the CONV2D_* codes of conv2d_bwd.h:
 *   CONV2D_ERR_NULL_PTR   p, or a pointer of a non-empty tensor, is NULL;
 *   CONV2D_ERR_BAD_SHAPE  k == 0 (the mean needs one column) or eps is
 *                         negative or not finite;
 *   CONV2D_ERR_ALIAS      out overlaps an input;
 *   CONV2D_ERR_OVERFLOW   a tensor reaches 2^31 bytes;
 *   CONV2D_ERR_HIP        the launch failed.
 * m == 0 or n == 0 is a valid empty call.
 */
#ifndef RMS_NORM_MATMUL_H_
#define RMS_NORM_MATMUL_H_

#include <stddef.h>
#include <stdint.h>

#include "conv2d_bwd.h"

#ifdef __cplusplus
extern "C" {
#endif

/* The page's Params (m, n, k, eps_bits), with eps as a float. */
typedef struct rms_matmul_params {
  uint32_t m;
  uint32_t n;
  uint32_t k;
  float eps;
} rms_matmul_params;

int rms_norm_matmul(const float* x, const float* norm_weight, const float* proj,
                    float* out, const rms_matmul_params* p, void* stream);

/* Host replay of rms_norm_matmul's kernel (no device needed): every staged
 * element is the x / proj element of the definition or 0 past k, every LDS
 * cell of a stage is written once, each row's sum of squares gathers every
 * column of that row once, and every output element is stored once.
 * Returns CONV2D_OK, 1 with a message in msg[0 .. msg_len-1], or the
 * shape's error code. */
int rms_norm_matmul_check_indexing(const rms_matmul_params* p, char* msg,
                                   size_t msg_len);

#ifdef __cplusplus
}
#endif

#endif /* RMS_NORM_MATMUL_H_ */
