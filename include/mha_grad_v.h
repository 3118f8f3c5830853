/*
 * Gradient of multi-head attention with respect to V on AMD CDNA4 (gfx950,
 * MI355X): C ABI.
 *
 * Computes what the docs.rs source page of meganeura 0.2.0,
 * src/shaders/mha_grad_v.wgsl, computes (its Params, the bounds of its
 * position loop, the score recomputation and the P * dO sum): for key t of
 * kv head g,
 *
 *   dv[t, g, :] = sum over pos in [causal ? t : 0,
 *                                  window > 0 ? min(q_seq, t + window) : q_seq)
 *                 and heads h = g * heads / kv_heads + r (r < heads / kv_heads)
 *                 of  P * dout[pos, h, :],
 *   P = exp(min(s - lse[pos, h, 0], 0) - lse[pos, h, 1]),
 *   s = q[pos, h, :] . k[t, g, :] / sqrt(head_dim).
 *
 * lse holds the forward pass's row statistics: the row maximum of the scaled
 * scores and the log of the sum of exp(score - maximum).
 *
 * Layouts (dense, row-major, fp32 in device memory):
 *   dout, q   [q_seq, heads, head_dim]      (read)
 *   k         [kv_seq, kv_heads, head_dim]  (read)
 *   lse       [q_seq, heads, 2]             (read)
 *   dv        [kv_seq, kv_heads, head_dim]  (fully overwritten)
 *
 * fp32 operands on the fp32 matrix cores (v_mfma_f32_16x16x4_f32), fp32
 * accumulation.  Asynchronous on `stream` (a hipStream_t; NULL: the null
 * stream).  Causal launches with too few units of work to give every
 * compute unit two workgroups (and an even number of heads per kv head)
 * split each unit's heads over two workgroups: dv is first zeroed by a fill
 * kernel on `stream`, then each workgroup adds its partial sum with an fp32
 * atomic add.  Exactly two terms meet on zero, so the result is the same on
 * every run (0 + a + b = 0 + b + a in IEEE arithmetic).  dv must then be
 * ordinary (coarse-grained) device memory, as hipMalloc and torch return:
 * the adds use the device's fp32 atomic instruction, which fine-grained or
 * host-coherent memory does not support.  Status codes are the CONV2D_* codes of conv2d_bwd.h:
 *   CONV2D_ERR_NULL_PTR   p, or a pointer of a non-empty tensor, is NULL;
 *   CONV2D_ERR_BAD_SHAPE  head_dim != 64 (the page's 64-lane workgroup),
 *                         kv_heads == 0, heads not a multiple of kv_heads,
 *                         causal with q_seq != kv_seq, or q, k or dv not
 *                         16-byte aligned (they are read and written in
 *                         16-byte pieces);
 *   CONV2D_ERR_ALIAS      dv overlaps an input;
 *   CONV2D_ERR_OVERFLOW   a tensor reaches 2^31 bytes;
 *   CONV2D_ERR_HIP        the launch failed.
 * kv_seq == 0 is a valid empty call; heads == 0 writes zeros.
 */
#ifndef MHA_GRAD_V_H_
#define MHA_GRAD_V_H_

#include <stddef.h>
#include <stdint.h>

#include "conv2d_bwd.h"

#ifdef __cplusplus
extern "C" {
#endif

/* The page's Params, with its packed head counts split and its causal
 * convention (kv_seq == 0) made an explicit flag. */
typedef struct mha_grad_v_params {
  uint32_t q_seq;
  uint32_t kv_seq;
  uint32_t heads;
  uint32_t kv_heads;
  uint32_t head_dim;
  uint32_t window;   /* 0: no window */
  uint32_t causal;   /* 0 or 1 */
} mha_grad_v_params;

int mha_grad_v(const float* dout, const float* q, const float* k, const float* lse,
               float* dv, const mha_grad_v_params* p, void* stream);

/* Host replay of mha_grad_v's launch (no device needed): the workgroups
 * cover every (key block, kv head) once, each key block's query blocks cover
 * every position of every one of its keys' ranges, and every staged element
 * is the definition's (0 past the sequence).  Returns CONV2D_OK, 1 with a
 * message, or the shape's error code. */
int mha_grad_v_check_indexing(const mha_grad_v_params* p, char* msg, size_t msg_len);

#ifdef __cplusplus
}
#endif

#endif /* MHA_GRAD_V_H_ */
