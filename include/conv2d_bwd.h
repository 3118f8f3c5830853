/*
 * conv2d_bwd.h -- C ABI of the MI355X (gfx950) convolution input-gradient
 * library (libconv2d_bwd.so).
 *
 * Operation.  For a 2-D cross-correlation y = conv2d(x, weight) with one
 * stride s for both axes and separate paddings padding_h / padding_w, the
 * library computes the gradient with respect to the input:
 *
 *   grad_input[n, ci, ih, iw] =
 *       sum over co, kh, kw with  th = ih + padding_h - kh >= 0,
 *                                 tw = iw + padding_w - kw >= 0,
 *                                 th % s == 0, tw % s == 0,
 *                                 th / s < out_h,  tw / s < out_w
 *       of grad_out[n, co, th / s, tw / s] * weight[co, ci, kh, kw].
 *
 * Source: the docs.rs source page of meganeura 0.2.0,
 * src/shaders/conv2d_grad_input_gemm_coop.wgsl.  Its header comment defines
 * the per-item product C[Ci, H*W] = A[Ci, Co*kH*kW] x B[Co*kH*kW, H*W] with
 * A = weight transposed and B = im2col(grad_out) transposed; its weight_T
 * staging fixes the weight index (no kernel flip); its stride > 1 im2col
 * branch fixes the divisibility rule above, used here for every stride; its
 * `Params` struct fixes the twelve shape fields (reordered below) and its
 * final store overwrites grad_input.
 *
 * Layouts (all dense, row-major, fp32 in device memory):
 *   grad_out   [batch, out_channels, out_h, out_w]
 *   weight     [out_channels, in_channels, kernel_h, kernel_w]
 *   grad_input [batch, in_channels, in_h, in_w]
 *
 * Ownership.  The caller owns all three device buffers and keeps them alive
 * until the work enqueued on `stream` has completed.  `p` is read during the
 * call only.  The library allocates no device memory and keeps no per-call
 * state; it keeps a host-side memo of recent launch plans (at most 64,
 * least recently used evicted; a memo changes no result) and a table of the
 * variants chosen per shape by conv2d_tune / conv2d_select_variant (never
 * evicted), both guarded by a mutex, so calls are reentrant and
 * thread-safe.  Calls on different streams that write the same grad_input
 * race like any other kernels would.
 *
 * Reproducibility.  A call's result is a deterministic function of its
 * inputs and of the kernel variant that runs it: repeated calls with one
 * variant are bitwise identical, on any stream.  Variants differ in
 * summation order only, so their results differ in rounding (within the
 * fp32 / f16 tolerances), and the variant of the default entry points is
 * the planner's model choice for the shape and the device's compute-unit
 * count until conv2d_tune or conv2d_select_variant chooses another for the
 * rest of the process.  For bitwise-identical results across processes,
 * pass the variant conv2d_tune chose in one process to
 * conv2d_select_variant in the other (or call conv2d_grad_input_variant).
 *
 * Semantics.  grad_input is fully overwritten (elements no tap reaches are
 * set to 0).  grad_out and weight are only read.  grad_input must not overlap
 * either input.  The call is asynchronous on `stream` (a hipStream_t; NULL
 * means the null stream); execution faults surface at the caller's next
 * synchronisation.  A call enqueues kernel launches only (no memset, no
 * allocation, no host synchronisation; conv2d_tune excepted), so once a shape
 * has been planned by one call, later calls on a stream under HIP graph
 * capture are recorded and replay to the same bits.
 *
 * Errors.  Every entry point returns an int status: CONV2D_OK (0) or a
 * negative CONV2D_ERR_* code.  On any validation error nothing is enqueued and
 * nothing is written.  Nothing is printed and no exception crosses the ABI.
 */
#ifndef CONV2D_BWD_H_
#define CONV2D_BWD_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The twelve shape fields of the shader's `Params` uniform, in the order
 * batch, in_channels, in_h, in_w, out_channels, kernel_h, kernel_w, stride,
 * padding_h, padding_w, out_h, out_w (the shader itself stores padding_w
 * last).  48 bytes. */
typedef struct conv2d_params {
  uint32_t batch;
  uint32_t in_channels;
  uint32_t in_h;
  uint32_t in_w;
  uint32_t out_channels;
  uint32_t kernel_h;
  uint32_t kernel_w;
  uint32_t stride;
  uint32_t padding_h;
  uint32_t padding_w;
  uint32_t out_h;
  uint32_t out_w;
} conv2d_params;

enum {
  CONV2D_OK = 0,
  CONV2D_ERR_NULL_PTR = -1,    /* a required pointer is NULL                 */
  CONV2D_ERR_BAD_SHAPE = -2,   /* stride/kernel 0, input smaller than kernel
                                  after padding, or out_h/out_w differ from
                                  floor((in + 2*pad - k) / stride) + 1       */
  CONV2D_ERR_ALIAS = -3,       /* grad_input overlaps grad_out or weight     */
  CONV2D_ERR_OVERFLOW = -4,    /* a per-image plane or the weight has
                                  >= 2^31 elements, or the tile count does   */
  CONV2D_ERR_UNSUPPORTED = -5, /* one kernel tap window of one stride phase
                                  does not fit the on-chip staging tile
                                  (kernel_h*kernel_w / stride^2 too large),
                                  or a forced kernel variant is out of range
                                  or cannot tile the shape                  */
  CONV2D_ERR_HIP = -6,         /* the HIP runtime reported an error at
                                  launch (hipGetLastError)                   */
  CONV2D_ERR_WORKSPACE = -7,   /* conv2d_grad_weight: the workspace is
                                  smaller than its workspace size or not
                                  16-byte aligned                            */
  CONV2D_ERR_SCRATCH = -8      /* conv2d_grad_weight_noalloc: the shape needs
                                  more than the library's scratch array
                                  (CONV2D_GRAD_WEIGHT_NOALLOC_MAX_BYTES)     */
};

/*
 * fp32 path: operands staged in fp32, products on the fp32 matrix cores
 * (v_mfma_f32_16x16x4_f32), fp32 accumulation.
 *   grad_out, weight: device pointers to the inputs (layouts above).
 *   grad_input:       device pointer to the output, fully overwritten.
 *   p:                host pointer to the shape.
 *   stream:           hipStream_t to enqueue on (NULL: null stream).
 * Returns CONV2D_OK or a CONV2D_ERR_* code.
 */
int conv2d_grad_input(const float* grad_out, const float* weight,
                      float* grad_input, const conv2d_params* p, void* stream);

/*
 * f16-staged path: the same operation and contract.  Storage stays fp32;
 * every operand element is rounded to f16 (round to nearest even) exactly
 * once, on its way from on-chip staging into the matrix cores
 * (v_mfma_f32_16x16x32_f16, v_mfma_f32_16x16x16_f16), with fp32
 * accumulation and an fp32 store.  This is the shader's $ENABLE_F16
 * specialisation: f16 tiles, fp32 buffers and store.
 */
int conv2d_grad_input_f16(const float* grad_out, const float* weight,
                          float* grad_input, const conv2d_params* p,
                          void* stream);

/*
 * Route of 1x1, stride-1, unpadded shapes (both paths above, and
 * conv2d_forward / conv2d_forward_f16 below): with in_channels and
 * in_h*in_w multiples of 4, each tensor below 2^31 bytes and all three
 * pointers 16-byte aligned, the call is one GEMM over the pixels of all
 * images (grad_input[n, :, p] = weight^T grad_out[n, :, p]; forward:
 * y[n, :, p] = weight x[n, :, p]), with the same rounding contract.  Such
 * a shape has no kernel variant (conv2d_tune runs it once and reports -1;
 * conv2d_select_variant refuses a variant for it).  Other pointers take
 * the variant kernels.
 */

/*
 * Validate a shape without touching any device or pointer (pure host code).
 * Returns CONV2D_OK, CONV2D_ERR_NULL_PTR (p == NULL), CONV2D_ERR_BAD_SHAPE,
 * CONV2D_ERR_OVERFLOW or CONV2D_ERR_UNSUPPORTED, exactly as the compute entry
 * points would for this shape.
 */
int conv2d_check_params(const conv2d_params* p);

/* Static English description of a status code (never NULL). */
const char* conv2d_status_string(int status);

/*
 * Measured choice of the kernel variant for a shape, once, before the
 * steady-state calls (like a framework's first-call tuning).  The variants
 * of the path (f16 != 0: the f16-staged path) whose modelled run time is
 * within 1.3x of the best (at most 8) each run once as a warm-up, then
 * three rounds time two runs of each in turn on the caller's buffers and
 * `stream` with HIP events; the one whose fastest round is fastest
 * becomes the plan conv2d_grad_input (or conv2d_grad_input_f16) uses for
 * this shape on devices with this many compute units, for the rest of the
 * process (as conv2d_select_variant would make it; at most 4096 shapes hold
 * a chosen variant, after which CONV2D_ERR_UNSUPPORTED is returned and the
 * model's choice stays in force).
 *   grad_out, weight, grad_input, p, stream: as for conv2d_grad_input;
 *     grad_input is overwritten, and on success holds the input gradient
 *     (computed by the chosen variant).
 *   variant_out: receives the chosen variant index (may be NULL; -1 if the
 *     shape launches nothing).
 * Blocking: waits for `stream` (HIP events are created and destroyed here;
 * no device memory is allocated).  Returns CONV2D_OK or a CONV2D_ERR_* code
 * (validation errors as for conv2d_grad_input, with nothing enqueued).
 * Thread-safe; concurrent tuning of one shape keeps the last result.
 */
int conv2d_tune(const float* grad_out, const float* weight, float* grad_input,
                const conv2d_params* p, int f16, void* stream, int* variant_out);

/*
 * The variant index conv2d_grad_input (f16 == 0) or conv2d_grad_input_f16
 * (f16 != 0) uses for this shape now, on the current device: the tuned one
 * after conv2d_tune, else the planner's model choice.  *variant_out gets the
 * index, or -1 if the shape launches nothing.  Returns CONV2D_OK or the
 * CONV2D_ERR_* code of an invalid shape (CONV2D_ERR_NULL_PTR for a NULL
 * argument).  Host code (reads the device's compute-unit count once).
 */
int conv2d_planned_variant(const conv2d_params* p, int f16, int* variant_out);

/*
 * Choose the variant conv2d_grad_input (f16 == 0) or conv2d_grad_input_f16
 * (f16 != 0) uses for this shape on the current device from now on, without
 * running anything: `variant` is a variant of that path that tiles the shape
 * (for instance the one conv2d_tune chose in another process, which makes
 * the two processes' results bitwise identical), or -1 to return to the
 * planner's model choice.  Returns CONV2D_OK, the shape's CONV2D_ERR_* code,
 * CONV2D_ERR_NULL_PTR, or CONV2D_ERR_UNSUPPORTED (variant out of range, of
 * the other path, unable to tile the shape, 4096 shapes already chosen, or
 * a variant for a shape on the 1x1 GEMM, which has none).
 * Host code (reads the device's compute-unit count once).
 */
int conv2d_select_variant(const conv2d_params* p, int f16, int variant);

/*
 * Launch plan of a shape, for inspection and host-side tests (pure host
 * code).  `f16` selects the plan of conv2d_grad_input_f16.  Fills `out`:
 *   out->launches      kernel launches the call would make
 *   out->tiles         workgroups over all launches
 *   out->phases        stride-residue phases with at least one pixel
 *   out->zero_phases   of those, phases no kernel tap reaches (written as 0)
 *   out->macs          multiply-adds issued, counting padded tile lanes
 *   out->useful_macs   N*Co*out_h*out_w*Ci*kH*kW
 * Returns the status conv2d_check_params returns.
 */
typedef struct conv2d_plan_info {
  int64_t launches;
  int64_t tiles;
  int64_t phases;
  int64_t zero_phases;
  int64_t macs;
  int64_t useful_macs;
} conv2d_plan_info;

int conv2d_describe_plan(const conv2d_params* p, int f16,
                         conv2d_plan_info* out);

/*
 * conv2d_describe_plan for the plan conv2d_grad_input_variant would make
 * with kernel variant `variant` (pure host code).  Returns as
 * conv2d_describe_plan, or CONV2D_ERR_UNSUPPORTED if the index is out of
 * range or the variant cannot tile the shape.
 */
int conv2d_describe_plan_variant(const conv2d_params* p, int variant,
                                 conv2d_plan_info* out);

/*
 * Host-side replay of the kernels' addressing for a shape (pure host code,
 * no device needed).  Walks every workgroup and thread of every launch that
 * conv2d_grad_input (f16 == 0) or conv2d_grad_input_f16 (f16 != 0) would
 * make and checks that every global and LDS access is in bounds, that every
 * tap reads the grad_out and weight elements of the gather rule above, and
 * that each grad_input element is written exactly once.  Returns CONV2D_OK,
 * a CONV2D_ERR_* code of conv2d_check_params, or 1 on a failed check, with a
 * description in `msg` (NUL-terminated, at most msg_len bytes; may be NULL).
 * Cost is proportional to the problem's multiply-adds / 64.
 */
int conv2d_check_indexing(const conv2d_params* p, int f16, char* msg,
                          size_t msg_len);

/*
 * Kernel variants.  Both paths run one kernel family; a variant fixes its
 * wave layout (waves along channels and pixels, 16-channel and 16-pixel
 * blocks per wave) and whether it is an fp32 or an f16-staged instance.
 * The compute entry points let the planner pick the variant; the calls
 * below force one, so that tests and tuning can reach every variant.
 */

/* Number of kernel variants the library carries (indices 0 .. n-1). */
int conv2d_num_variants(void);

/* 1 if `variant` is an f16-staged instance, 0 if fp32,
 * CONV2D_ERR_UNSUPPORTED if the index is out of range. */
int conv2d_variant_is_f16(int variant);

/* 1 if `variant` puts the kernel's column taps into its matrix rows next to
 * the input channels (the few-input-channel variants: one matrix block of
 * 16 rows holds 16 / ceil(kernel_w / stride) input channels, each with its
 * column taps, and the column taps of a pixel are added in the epilogue),
 * 0 if its matrix rows are input channels only, CONV2D_ERR_UNSUPPORTED if
 * the index is out of range.  Results are the same up to summation order. */
int conv2d_variant_uses_column_taps(int variant);

/* 1 if `variant` is a multi-class instance (stride 2 only: one workgroup
 * covers the same grid points of all four stride-residue classes, which
 * share one staged grad_out window, and the epilogue stores each class's
 * pixels), 0 if each workgroup covers one class, CONV2D_ERR_UNSUPPORTED if
 * the index is out of range.  Multi-class variants tile only shapes with
 * stride 2 whose four classes all have pixels and taps and whose kernel has
 * at most 9 taps (else CONV2D_ERR_UNSUPPORTED from the calls that force a
 * variant); they have no forward or f16-staged instance.  Results are the
 * same up to summation order. */
int conv2d_variant_is_multi_class(int variant);

/*
 * conv2d_grad_input (or conv2d_grad_input_f16, as the variant's path
 * dictates) with the kernel variant forced to `variant`.  Same contract and
 * results (up to summation order); returns CONV2D_ERR_UNSUPPORTED, with
 * nothing enqueued, if the index is out of range or the variant cannot tile
 * the shape.
 */
int conv2d_grad_input_variant(const float* grad_out, const float* weight,
                              float* grad_input, const conv2d_params* p,
                              int variant, void* stream);

/*
 * conv2d_check_indexing for the launches conv2d_grad_input_variant would
 * make.  Returns as conv2d_check_indexing, or CONV2D_ERR_UNSUPPORTED as
 * conv2d_grad_input_variant does.
 */
int conv2d_check_indexing_variant(const conv2d_params* p, int variant,
                                  char* msg, size_t msg_len);

/*
 * Forward convolution (the adjoint operator of the input gradient above):
 *
 *   y[n, co, oh, ow] = sum over ci, kh, kw with
 *                          ih = oh * s - padding_h + kh in [0, in_h),
 *                          iw = ow * s - padding_w + kw in [0, in_w)
 *                      of x[n, ci, ih, iw] * weight[co, ci, kh, kw]
 *
 * (no bias, no kernel flip).  Source: the same shader page; its stride > 1
 * im2col branch relates grad_out[n, co, oh, ow] to input pixel
 * (oh * s - padding_h + kh, ow * s - padding_w + kw) through tap (kh, kw),
 * which is the index map of this convolution, so that
 * <grad_input(grad_out), x> = <grad_out, y(x)> for every x and grad_out.
 *
 * Layouts (dense, row-major, fp32 in device memory), with the same
 * conv2d_params as above (out_h / out_w must be the forward extents):
 *   x      [batch, in_channels, in_h, in_w]           (read)
 *   weight [out_channels, in_channels, kernel_h, kernel_w]   (read)
 *   y      [batch, out_channels, out_h, out_w]        (fully overwritten)
 * Ownership, asynchrony and errors as for conv2d_grad_input; y must not
 * overlap x or weight (CONV2D_ERR_ALIAS); an empty contraction
 * (in_channels = 0) writes zeros.  The weight tensor must be below 2^31
 * bytes (else CONV2D_ERR_OVERFLOW).  Runs on the kernels of the input
 * gradient with the operand roles exchanged (the kernel variants without
 * column taps); conv2d_forward_f16 rounds x and weight to f16 (round to
 * nearest even) and accumulates in fp32, as conv2d_grad_input_f16 does.
 * conv2d_forward with 1 to 15 input channels runs an im2col GEMM over
 * (ci, kh, kw) instead, when x and y each stay below 2^31 bytes and
 * batch*out_h*out_w below 2^31; larger such shapes take the variant
 * kernels, like every other shape.  Other 1x1, stride-1, unpadded shapes
 * take the 1x1 GEMM (described after conv2d_grad_input_f16).
 */
int conv2d_forward(const float* x, const float* weight, float* y,
                   const conv2d_params* p, void* stream);
int conv2d_forward_f16(const float* x, const float* weight, float* y,
                       const conv2d_params* p, void* stream);

/* conv2d_forward (or _f16, as the variant's path dictates) with the kernel
 * variant forced; CONV2D_ERR_UNSUPPORTED, nothing enqueued, if the index is
 * out of range, the variant has column taps or cannot tile the shape. */
int conv2d_forward_variant(const float* x, const float* weight, float* y,
                           const conv2d_params* p, int variant, void* stream);

/* conv2d_tune for the forward convolution: times the best-modelled variants
 * on the caller's buffers (x and weight read, y written, with the result of
 * the chosen variant left in y), makes the fastest the shape's default
 * forward plan, blocks until done, and stores it in *variant_out if that is
 * not NULL.  A shape conv2d_forward runs on the im2col GEMM or the 1x1
 * GEMM (above) has no variant: it is run once and *variant_out gets -1.
 * Errors as
 * conv2d_forward, or CONV2D_ERR_HIP. */
int conv2d_tune_forward(const float* x, const float* weight, float* y,
                        const conv2d_params* p, int f16, void* stream,
                        int* variant_out);

/* The variant conv2d_forward (f16 == 0) or conv2d_forward_f16 uses for the
 * shape now, in *variant_out (-1 if nothing is launched or the shape runs
 * on the im2col GEMM or the 1x1 GEMM).  CONV2D_OK, or the error of conv2d_check_params, or
 * CONV2D_ERR_NULL_PTR. */
int conv2d_planned_forward_variant(const conv2d_params* p, int f16, int* variant_out);

/* conv2d_select_variant for conv2d_forward / conv2d_forward_f16;
 * CONV2D_ERR_UNSUPPORTED also for a variant of a shape on the im2col GEMM
 * or the 1x1 GEMM. */
int conv2d_select_forward_variant(const conv2d_params* p, int f16, int variant);

/* conv2d_describe_plan / _variant for the forward launches (host only). */
int conv2d_describe_forward_plan(const conv2d_params* p, int f16,
                                 conv2d_plan_info* out);
int conv2d_describe_forward_plan_variant(const conv2d_params* p, int variant,
                                         conv2d_plan_info* out);

/* conv2d_check_indexing / _variant for the forward launches: every access
 * in bounds, every tap of every output pixel reading the x and weight
 * elements of the definition above (checked against p's stride and
 * paddings), every y element written exactly once.  Host only. */
int conv2d_check_indexing_forward(const conv2d_params* p, int f16, char* msg,
                                  size_t msg_len);
int conv2d_check_indexing_forward_variant(const conv2d_params* p, int variant,
                                          char* msg, size_t msg_len);

/*
 * Weight gradient of the same forward convolution (the other half of its
 * backward pass):
 *
 *   grad_weight[co, ci, kh, kw] = sum over n, oh, ow with
 *                                     ih = oh * s - padding_h + kh in [0, in_h),
 *                                     iw = ow * s - padding_w + kw in [0, in_w)
 *                                 of grad_out[n, co, oh, ow] * x[n, ci, ih, iw]
 *
 * Not on the source page; its index map is the forward convolution's above
 * (the page's stride > 1 im2col branch read forwards), and it is the
 * weight-adjoint of that map: <grad_weight(go, x), V> = <go, y(x, V)>.
 *
 * Layouts (dense, row-major, fp32 in device memory), same conv2d_params:
 *   grad_out    [batch, out_channels, out_h, out_w]            (read)
 *   x           [batch, in_channels, in_h, in_w]               (read)
 *   grad_weight [out_channels, in_channels, kernel_h, kernel_w] (overwritten)
 *   workspace   conv2d_grad_weight_workspace_size bytes of device memory,
 *               16-byte aligned (hipMalloc gives 256), owned by the caller,
 *               overwritten (partial sums of pixel chunks; it holds nothing
 *               between calls)
 * The contraction over all batch x out_h x out_w pixels is split into
 * chunks; the chunks' partial sums are added in a fixed order by a second
 * kernel, so results do not depend on scheduling.  fp32 matrix cores, fp32
 * accumulation.  Asynchronous on `stream` like conv2d_grad_input; calls that
 * share a workspace must not overlap.
 *
 * Errors: as conv2d_grad_input (CONV2D_ERR_ALIAS if grad_weight or the
 * workspace overlaps an input or each other), CONV2D_ERR_WORKSPACE if the
 * workspace is NULL, not 16-byte aligned or smaller than the size below
 * while that size is not 0, CONV2D_ERR_OVERFLOW if grad_out or x reaches 2^31 bytes.  batch = 0 (no
 * pixel) writes zeros.
 */
int conv2d_grad_weight(const float* grad_out, const float* x, float* grad_weight,
                       const conv2d_params* p, void* workspace, size_t workspace_bytes,
                       void* stream);

/* Bytes of workspace conv2d_grad_weight needs for the shape on the current
 * device, in *bytes (may be 0).  CONV2D_OK or the shape's error code. */
int conv2d_grad_weight_workspace_size(const conv2d_params* p, size_t* bytes);

/* Host replay of conv2d_grad_weight's kernels (no device needed), through
 * the kernels' own index functions and pixel walk: for every stored weight
 * row and column each pixel contributes the grad_out x x product of the
 * definition above (or 0 where it has no term), every LDS cell of a stage
 * is written once, the products pair A and B cells of one pixel, every
 * partial-tile element is stored once, and the reduction takes every weight
 * element from exactly one partial element.  Returns as
 * conv2d_check_indexing. */
int conv2d_check_indexing_grad_weight(const conv2d_params* p, char* msg,
                                      size_t msg_len);

/*
 * Weight-gradient column layouts.  The kernel tiles the (out_channels) x
 * (in_channels * kernel_h * kernel_w) product in 64 x 64 tiles; a variant
 * fixes how the 64 column slots of a tile map to weight columns:
 *   0  flat: 64 consecutive columns of the weight layout;
 *   1, 2, 3  tap tiles: 64, 32 or 16 input channels x 1, 2 or 4 kernel taps.
 * conv2d_grad_weight takes the planner's choice; the calls below force one
 * (tests and measurement).  Every variant computes the same result (up to
 * fp32 summation order); variant < -1 or > 3 gives CONV2D_ERR_UNSUPPORTED,
 * -1 the planner's choice.
 */
int conv2d_grad_weight_variant(const float* grad_out, const float* x,
                               float* grad_weight, const conv2d_params* p,
                               void* workspace, size_t workspace_bytes,
                               void* stream, int variant);

/*
 * conv2d_grad_weight for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same operation, plan and result (bit for bit), with the
 * partial sums in a scratch array the library holds in device memory
 * (CONV2D_GRAD_WEIGHT_NOALLOC_MAX_BYTES per device, from the first load of
 * the library until the process ends) instead of a caller's workspace.  The
 * call allocates nothing.
 *   grad_out, x, grad_weight, p, stream: as for conv2d_grad_weight.
 * Returns what conv2d_grad_weight returns (no workspace error), or
 * CONV2D_ERR_SCRATCH, with nothing enqueued, if
 * conv2d_grad_weight_workspace_size reports more than
 * CONV2D_GRAD_WEIGHT_NOALLOC_MAX_BYTES for the shape (on a 256-CU device
 * that takes a weight of more than 2048 tiles of 64 x 64, about 8.4M
 * elements), or CONV2D_ERR_HIP if the scratch's address cannot be taken.
 * Every call on one device shares that device's scratch: calls that may
 * overlap on one device (other streams, other host threads) race and must
 * be ordered by the caller.
 */
#define CONV2D_GRAD_WEIGHT_NOALLOC_MAX_BYTES (32u << 20)
int conv2d_grad_weight_noalloc(const float* grad_out, const float* x,
                               float* grad_weight, const conv2d_params* p,
                               void* stream);

/* Workspace bytes of conv2d_grad_weight_variant, as
 * conv2d_grad_weight_workspace_size. */
int conv2d_grad_weight_variant_workspace_size(const conv2d_params* p,
                                              int variant, size_t* bytes);

/* The weight-gradient plan of a shape and variant (pure host code; -1: the
 * planner's), in info[0 .. n-1] (at most 7 values written): variant, input
 * channels and taps of a tap tile (0, 0 for flat tiles), tiles along
 * out_channels, column tiles, pixel chunks, pixels per chunk.  CONV2D_OK
 * or the shape's error code. */
int conv2d_describe_grad_weight_plan(const conv2d_params* p, int variant,
                                     int32_t* info, int n);

/* conv2d_check_indexing_grad_weight for a forced variant. */
int conv2d_check_indexing_grad_weight_variant(const conv2d_params* p,
                                              int variant, char* msg,
                                              size_t msg_len);

#ifdef __cplusplus
}
#endif

#endif /* CONV2D_BWD_H_ */
