/*
 * CPU oracle for the convolution backward pass with respect to the input (and
 * the operators beside it: the forward convolution, the weight gradient, and
 * the RMSNorm-fused matrix product of a second page).
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this code.  The product path (the HIP
 * library under conv2d_backward_implicit_amd/csrc) never calls it, links it or
 * shares a line with it.
 *
 * Source cited throughout as [p3]: the docs.rs source page of meganeura 0.2.0,
 * "src/shaders/conv2d_grad_input_gemm_coop.wgsl".  The sections referred to
 * are that shader's header comment, its `Params` struct, the two branches of
 * its im2col (B-tile) staging (stride 1 and stride > 1), its weight_T (A-tile)
 * staging and its final store to grad_input.  [p2] is the docs.rs source page
 * of the same crate, "src/shaders/matmul_rms_norm.wgsl" (header comment,
 * per-row rsqrt prologue, normalise-on-load A staging); only
 * oracle_rms_norm_matmul follows it.  [p1] is the page
 * "src/shaders/mha_grad_v.wgsl" of the same crate (its Params, the causal
 * and window bounds of the position loop, the score recomputation and the
 * P * dO sum); oracle_attention_lse and oracle_mha_grad_v follow it.
 *
 * Every routine here is a plain loop nest over the definition, accumulated in
 * double precision, with no blocking, no reordering beyond the definition and
 * no shared helpers with the GPU path.  Arrays are dense, row-major:
 *   grad_out   [N, Co, OH, OW]
 *   weight     [Co, Ci, KH, KW]
 *   grad_input [N, Ci, H, W]
 *   x (forward input) [N, Ci, H, W],  y (forward output) [N, Co, OH, OW]
 * All extents are passed explicitly; OH and OW are taken as given (they bound
 * the gather, as in [p3] `Params`), the caller decides whether they are the
 * forward-conv extents.
 *
 * Parallelism: OpenMP over independent output elements only (each element is
 * still one serial sum in the definition's loop order), so results do not
 * depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef int64_t i64;

/*
 * Direct gather (the definition).
 *
 * [p3] header comment: per batch item the result is the product
 *   grad_input[ci, (ih, iw)] = sum over k = (co, kh, kw) of
 *       weight^T[ci, k] * im2col(grad_out)[k, (ih, iw)].
 * [p3] weight_T staging: weight^T[ci, (co, kh, kw)] = weight[co, ci, kh, kw]
 *   (no spatial flip of the kernel).
 * [p3] stride > 1 im2col branch: the im2col entry for pixel (ih, iw) and tap
 *   (kh, kw) is grad_out[n, co, oh, ow] with oh = (ih + padding_h - kh) / s and
 *   ow = (iw + padding_w - kw) / s when both numerators are non-negative and
 *   divisible by s and oh < OH, ow < OW; otherwise the entry is zero.  This
 *   rule is applied here for every stride, s = 1 included.  (The shader's
 *   stride-1 branch instead offsets by kH-1-padding_h / kW-1-padding_w; the
 *   two branches give the same entry only when padding = (k-1)/2, and only
 *   the rule used here is the adjoint of the forward convolution below.)
 * [p3] final store: grad_input is overwritten, every element is written.
 */
void oracle_grad_input_gather(const double* go, const double* w, double* gi,
                              i64 N, i64 Ci, i64 H, i64 W, i64 Co, i64 KH,
                              i64 KW, i64 s, i64 ph, i64 pw, i64 OH, i64 OW) {
  i64 total = N * Ci * H * W;
#pragma omp parallel for schedule(static)
  for (i64 e = 0; e < total; ++e) {
    i64 iw = e % W;
    i64 ih = (e / W) % H;
    i64 ci = (e / (W * H)) % Ci;
    i64 n = e / (W * H * Ci);
    double acc = 0.0;
    for (i64 co = 0; co < Co; ++co) {
      for (i64 kh = 0; kh < KH; ++kh) {
        for (i64 kw = 0; kw < KW; ++kw) {
          i64 th = ih + ph - kh;
          i64 tw = iw + pw - kw;
          if (th < 0 || tw < 0) continue;
          if (th % s != 0 || tw % s != 0) continue;
          i64 oh = th / s;
          i64 ow = tw / s;
          if (oh >= OH || ow >= OW) continue;
          acc += go[((n * Co + co) * OH + oh) * OW + ow] *
                 w[((co * Ci + ci) * KH + kh) * KW + kw];
        }
      }
    }
    gi[e] = acc;
  }
}

/*
 * The same gather, evaluated only at the listed flat grad_input indices
 * (idx[j] in [0, N*Ci*H*W)).  Used to check outputs of full-size problems
 * one element at a time.  Identical arithmetic to oracle_grad_input_gather.
 */
void oracle_grad_input_gather_at(const double* go, const double* w,
                                 const i64* idx, i64 count, double* out,
                                 i64 N, i64 Ci, i64 H, i64 W, i64 Co, i64 KH,
                                 i64 KW, i64 s, i64 ph, i64 pw, i64 OH,
                                 i64 OW) {
  (void)N;
#pragma omp parallel for schedule(static)
  for (i64 j = 0; j < count; ++j) {
    i64 e = idx[j];
    i64 iw = e % W;
    i64 ih = (e / W) % H;
    i64 ci = (e / (W * H)) % Ci;
    i64 n = e / (W * H * Ci);
    double acc = 0.0;
    for (i64 co = 0; co < Co; ++co) {
      for (i64 kh = 0; kh < KH; ++kh) {
        for (i64 kw = 0; kw < KW; ++kw) {
          i64 th = ih + ph - kh;
          i64 tw = iw + pw - kw;
          if (th < 0 || tw < 0) continue;
          if (th % s != 0 || tw % s != 0) continue;
          i64 oh = th / s;
          i64 ow = tw / s;
          if (oh >= OH || ow >= OW) continue;
          acc += go[((n * Co + co) * OH + oh) * OW + ow] *
                 w[((co * Ci + ci) * KH + kh) * KW + kw];
        }
      }
    }
    out[j] = acc;
  }
}

/*
 * Scatter formulation, an independent code path for the same quantity: every
 * grad_out element (n, co, oh, ow) is pushed back through every tap (kh, kw)
 * to the input pixel it was computed from in the forward pass,
 *   ih = oh*s - padding_h + kh,  iw = ow*s - padding_w + kw,
 * and added there if that pixel lies inside the input.  This is the transpose
 * of the forward map; it needs no divisibility test at all.
 * Parallel over (n, ci) planes, each plane owned by one thread.
 */
void oracle_grad_input_scatter(const double* go, const double* w, double* gi,
                               i64 N, i64 Ci, i64 H, i64 W, i64 Co, i64 KH,
                               i64 KW, i64 s, i64 ph, i64 pw, i64 OH, i64 OW) {
  i64 planes = N * Ci;
#pragma omp parallel for schedule(static)
  for (i64 pl = 0; pl < planes; ++pl) {
    i64 n = pl / Ci;
    i64 ci = pl % Ci;
    double* dst = gi + pl * H * W;
    for (i64 q = 0; q < H * W; ++q) dst[q] = 0.0;
    for (i64 co = 0; co < Co; ++co) {
      for (i64 oh = 0; oh < OH; ++oh) {
        for (i64 ow = 0; ow < OW; ++ow) {
          double g = go[((n * Co + co) * OH + oh) * OW + ow];
          for (i64 kh = 0; kh < KH; ++kh) {
            i64 ih = oh * s - ph + kh;
            if (ih < 0 || ih >= H) continue;
            for (i64 kw = 0; kw < KW; ++kw) {
              i64 iw = ow * s - pw + kw;
              if (iw < 0 || iw >= W) continue;
              dst[ih * W + iw] += g * w[((co * Ci + ci) * KH + kh) * KW + kw];
            }
          }
        }
      }
    }
  }
}

/*
 * Forward 2-D cross-correlation (the operator whose input-gradient is the
 * quantity above):
 *   y[n, co, oh, ow] = sum_{ci, kh, kw} x[n, ci, oh*s - ph + kh, ow*s - pw + kw]
 *                                        * weight[co, ci, kh, kw],
 * with x taken as zero outside [0,H) x [0,W).  Serves the adjoint identity
 * <grad_input(go), x> = <go, conv2d_fwd(x)>.
 */
void oracle_conv2d_forward(const double* x, const double* w, double* y, i64 N,
                           i64 Ci, i64 H, i64 W, i64 Co, i64 KH, i64 KW, i64 s,
                           i64 ph, i64 pw, i64 OH, i64 OW) {
  i64 total = N * Co * OH * OW;
#pragma omp parallel for schedule(static)
  for (i64 e = 0; e < total; ++e) {
    i64 ow = e % OW;
    i64 oh = (e / OW) % OH;
    i64 co = (e / (OW * OH)) % Co;
    i64 n = e / (OW * OH * Co);
    double acc = 0.0;
    for (i64 ci = 0; ci < Ci; ++ci) {
      for (i64 kh = 0; kh < KH; ++kh) {
        i64 ih = oh * s - ph + kh;
        if (ih < 0 || ih >= H) continue;
        for (i64 kw = 0; kw < KW; ++kw) {
          i64 iw = ow * s - pw + kw;
          if (iw < 0 || iw >= W) continue;
          acc += x[((n * Ci + ci) * H + ih) * W + iw] *
                 w[((co * Ci + ci) * KH + kh) * KW + kw];
        }
      }
    }
    y[e] = acc;
  }
}

/*
 * Gradient with respect to the weight of the same forward cross-correlation
 * (not on the pages; it is the other half of that convolution's backward
 * pass, and its index map is the forward one above, which is the map of the
 * [p3] stride > 1 im2col branch read forwards):
 *   grad_weight[co, ci, kh, kw] = sum over n, oh, ow of
 *       grad_out[n, co, oh, ow] * x[n, ci, oh*s - ph + kh, ow*s - pw + kw],
 * with x taken as zero outside [0,H) x [0,W).  It is the adjoint of the
 * forward map in its weight argument: <grad_weight(go, x), V> =
 * <go, conv2d_fwd(x, V)> for every V.  Parallel over (co, ci) pairs, each
 * element one serial sum in the definition's loop order.
 */
void oracle_grad_weight(const double* go, const double* x, double* gw, i64 N,
                        i64 Ci, i64 H, i64 W, i64 Co, i64 KH, i64 KW, i64 s,
                        i64 ph, i64 pw, i64 OH, i64 OW) {
  i64 total = Co * Ci * KH * KW;
#pragma omp parallel for schedule(static)
  for (i64 e = 0; e < total; ++e) {
    i64 kw = e % KW;
    i64 kh = (e / KW) % KH;
    i64 ci = (e / (KW * KH)) % Ci;
    i64 co = e / (KW * KH * Ci);
    double acc = 0.0;
    for (i64 n = 0; n < N; ++n) {
      for (i64 oh = 0; oh < OH; ++oh) {
        i64 ih = oh * s - ph + kh;
        if (ih < 0 || ih >= H) continue;
        for (i64 ow = 0; ow < OW; ++ow) {
          i64 iw = ow * s - pw + kw;
          if (iw < 0 || iw >= W) continue;
          acc += go[((n * Co + co) * OH + oh) * OW + ow] *
                 x[((n * Ci + ci) * H + ih) * W + iw];
        }
      }
    }
    gw[e] = acc;
  }
}

/* RMSNorm-fused matrix product (meganeura 0.2.0, matmul_rms_norm.wgsl: the
 * header comment's C = RmsNorm(X, W_norm) x W_proj, the per-row prologue and
 * the normalise-on-load step), in the page's order and in double precision:
 *   r[i]    = 1 / sqrt(sum_k x[i, k]^2 / K + eps)
 *   a[i, k] = x[i, k] * r[i] * g[k]
 *   c[i, j] = sum_k a[i, k] * w[k, j]
 * x [M, K], g [K] (the norm scale), w [K, N], c [M, N], all row-major.  Only
 * the rows listed in rows[0 .. nrows-1] are computed (c keeps M rows).  K >=
 * 1 is the caller's to ensure. */
void oracle_rms_norm_matmul(const double* x, const double* g, const double* w, double* c,
                            i64 M, i64 K, i64 N, double eps, const i64* rows, i64 nrows) {
  (void)M;
#pragma omp parallel for schedule(dynamic, 1)
  for (i64 t = 0; t < nrows; ++t) {
    const i64 i = rows[t];
    const double* xi = x + i * K;
    double ss = 0.0;
    for (i64 k = 0; k < K; ++k) ss += xi[k] * xi[k];
    const double r = 1.0 / sqrt(ss / (double)K + eps);
    double* ci = c + i * N;
    for (i64 j = 0; j < N; ++j) ci[j] = 0.0;
    for (i64 k = 0; k < K; ++k) {
      const double a = xi[k] * r * g[k];
      const double* wk = w + k * N;
      for (i64 j = 0; j < N; ++j) ci[j] += a * wk[j];
    }
  }
}

/* Attention rows for the dV routine below ([p1] = meganeura 0.2.0,
 * src/shaders/mha_grad_v.wgsl, its kv_seq == 0 causal convention and its
 * window bound): query pos sees key t when t <= pos (causal) and
 * pos < t + window (window > 0).  Fills lse[(pos * H + h) * 2 + {0, 1}] =
 * (max_t s, log sum_t exp(s - max)) over the keys pos sees, s = q . k /
 * sqrt(D), the forward-pass statistics the dV routine takes.  A row that
 * sees no key gets (0, 0). */
void oracle_attention_lse(const double* q, const double* k, double* lse, i64 q_seq,
                          i64 kv_seq, i64 H, i64 HKV, i64 D, i64 window, i64 causal) {
  const double scale = 1.0 / sqrt((double)D);
  const i64 group = H / HKV;
#pragma omp parallel for collapse(2) schedule(static)
  for (i64 pos = 0; pos < q_seq; ++pos)
    for (i64 h = 0; h < H; ++h) {
      const double* qp = q + (pos * H + h) * D;
      const i64 kvh = h / group;
      double mx = -INFINITY;
      for (i64 t = 0; t < kv_seq; ++t) {
        if ((causal && t > pos) || (window > 0 && pos >= t + window)) continue;
        double s = 0.0;
        for (i64 d = 0; d < D; ++d) s += qp[d] * k[(t * HKV + kvh) * D + d];
        s *= scale;
        if (s > mx) mx = s;
      }
      double sum = 0.0;
      for (i64 t = 0; t < kv_seq; ++t) {
        if ((causal && t > pos) || (window > 0 && pos >= t + window)) continue;
        double s = 0.0;
        for (i64 d = 0; d < D; ++d) s += qp[d] * k[(t * HKV + kvh) * D + d];
        sum += exp(s * scale - mx);
      }
      lse[(pos * H + h) * 2] = sum > 0.0 ? mx : 0.0;
      lse[(pos * H + h) * 2 + 1] = sum > 0.0 ? log(sum) : 0.0;
    }
}

/* Gradient of multi-head attention with respect to V ([p1]): for key t of
 * kv head kvh,
 *   dv[t, kvh, :] = sum over pos in [causal ? t : 0, window > 0 ?
 *                   min(q_seq, t + window) : q_seq) and heads h of the group
 *                   of kvh (h = kvh * H / HKV + r) of P * dout[pos, h, :],
 *   P = exp(min(s - lse[pos, h, 0], 0) - lse[pos, h, 1]),  s = q . k / sqrt(D).
 * q, dout [q_seq, H, D]; k, dv [kv_seq, HKV, D]; lse [q_seq, H, 2]. */
void oracle_mha_grad_v(const double* dout, const double* q, const double* k, const double* lse,
                       double* dv, i64 q_seq, i64 kv_seq, i64 H, i64 HKV, i64 D, i64 window,
                       i64 causal) {
  const double scale = 1.0 / sqrt((double)D);
  const i64 group = H / HKV;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
  for (i64 t = 0; t < kv_seq; ++t)
    for (i64 kvh = 0; kvh < HKV; ++kvh) {
      const double* kt = k + (t * HKV + kvh) * D;
      double* out = dv + (t * HKV + kvh) * D;
      for (i64 d = 0; d < D; ++d) out[d] = 0.0;
      const i64 start = causal ? t : 0;
      const i64 end = window > 0 ? (q_seq < t + window ? q_seq : t + window) : q_seq;
      for (i64 pos = start; pos < end; ++pos)
        for (i64 r = 0; r < group; ++r) {
          const i64 h = kvh * group + r;
          const double* qp = q + (pos * H + h) * D;
          double s = 0.0;
          for (i64 d = 0; d < D; ++d) s += qp[d] * kt[d];
          s *= scale;
          const double* l = lse + (pos * H + h) * 2;
          double e = s - l[0];
          if (e > 0.0) e = 0.0;
          const double pr = exp(e - l[1]);
          const double* g = dout + (pos * H + h) * D;
          for (i64 d = 0; d < D; ++d) out[d] += pr * g[d];
        }
    }
}

/* Number of OpenMP threads the routines above will use. */
int oracle_num_threads(void) {
  int t = 1;
#ifdef _OPENMP
#pragma omp parallel
  {
#pragma omp single
    t = omp_get_num_threads();
  }
#endif
  return t;
}
