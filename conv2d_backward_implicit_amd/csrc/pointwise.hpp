// Geometry and index arithmetic of the 1x1 GEMM (pointwise_gemm.hip) that
// serves the input gradient and the forward convolution of 1x1, stride-1,
// unpadded layers, shared by its kernel, its host replay and the planner's
// description of a shape's launch.
#pragma once

#include <stdint.h>
#include <string.h>

#include "plan.hpp"

#if defined(__HIP__) || defined(__HIPCC__)
#include <hip/hip_runtime.h>
#define PW_HD __host__ __device__ __forceinline__
#else
#define PW_HD inline
#endif

namespace c2b {
namespace fg {   // forward_gemm.hip
bool fg_applies(const conv2d_params* p, int f16);
}  // namespace fg
namespace pw {

constexpr int kBM = 128, kBN = 128;   // channels x pixels per tile
constexpr int kBK = 32;               // output channels (k) per stage
constexpr int kBufs = 4;              // stage buffers: loads run 3 stages ahead
constexpr int kBufsShared = 2;        // ... or 1 ahead, two workgroups per CU
constexpr int kThreads = 256;
constexpr int kWave = 64;             // each wave 64 x 64
constexpr int kLoads = 4;             // 16-byte loads per wave, operand and stage
constexpr int kStageBytes = (kBK * kBM + kBK * kBN) * 4;   // A then B
constexpr uint32_t kPad = 0x80000000u;   // byte offset past every buffer range
constexpr int64_t kI31 = int64_t(1) << 31;
static_assert(kLoads * 4 * 2 == kBK, "a wave's loads cover its share of both operands");

// Operands of one launch.  Input gradient (fwd = 0): rows m are input
// channels, k output channels, A[k][m] = weight[k, m], B = grad_out, C =
// grad_input.  Forward convolution (fwd = 1, the same GEMM with the
// weight's other index first): rows m are output channels, k input
// channels, A[m][k] = weight[m, k], B = x, C = y.
struct PWArgs {
  const float* go;   // B: grad_out, or x
  const float* w;
  float* gi;         // C: grad_input, or y
  int32_t M;    // rows of the product
  int32_t K;    // contraction
  int32_t P;    // pixels per image, H * W
  int32_t Q;    // pixels of all images, N * H * W
  int32_t TM, TN;
  int32_t fwd;  // 1: A is [m][k] (forward)
};

PW_HD int imin(int a, int b) { return a < b ? a : b; }

// Tile (channel tile tm, pixel tile tn) of workgroup bid: the workgroups of
// one XCD (bid mod 8) take one contiguous run of tiles, channel tiles
// fastest.
PW_HD void tile_of(const PWArgs& a, int bid, int* tm, int* tn) {
  const int T = a.TM * a.TN;
  const int q = T >> 3, r = T & 7, x = bid & 7, k = bid >> 3;
  const int t = x * q + imin(x, r) + k;
  *tm = t % a.TM;
  *tn = t / a.TM;
}

// Load j (0 .. 15) of an operand's stage, lane l: k row 2j + l / 32 and
// quad l % 32 of the row's 128 elements.  It lands at byte 1024 j + 16 l of
// the operand's region, i.e. [k row][4 * quad .. +3].
PW_HD int load_krow(int j, int l) { return 2 * j + l / 32; }
PW_HD int load_quad(int l) { return l % 32; }

// Byte offset in weight of the A quad (k row krow of stage st, channels
// m0 + 4 quad ..), or kPad past Co or Ci.
PW_HD uint32_t a_offset(const PWArgs& a, int st, int m0, int krow, int quad) {
  const int k = st * kBK + krow, m = m0 + 4 * quad;
  if (k >= a.K || m >= a.M) return kPad;
  return (uint32_t(k) * uint32_t(a.M) + uint32_t(m)) * 4u;
}

// Forward (A = [m][k]): load j of the A stage, lane l: tile row 8j + l / 8
// and LDS slot l % 8 of the row's eight k quads; the slot holds k quad
// slot ^ a_swizzle(row), so that 16 lanes reading 16 consecutive rows at
// one k quad hit 16 distinct 4-bank groups (rows 128 bytes apart).  The
// swizzle is its own inverse.
PW_HD int a_swizzle(int row) { return (row >> 1) & 7; }
PW_HD int arow_row(int j, int l) { return 8 * j + l / 8; }
PW_HD int arow_kq(int j, int l) { return (l % 8) ^ a_swizzle(arow_row(j, l)); }

// Byte offset in weight of forward A row `row` (tile row), k quad kq of
// stage st, or kPad past the rows or K.
PW_HD uint32_t arow_offset(const PWArgs& a, int st, int m0, int row, int kq) {
  const int m = m0 + row, k = st * kBK + 4 * kq;
  if (m >= a.M || k >= a.K) return kPad;
  return (uint32_t(m) * uint32_t(a.K) + uint32_t(k)) * 4u;
}

// Element offset n * K * P + p of grad_out pixel q (k = 0), or -1 past Q.
PW_HD int64_t b_base(const PWArgs& a, int q) {
  if (q >= a.Q) return -1;
  const int n = q / a.P, p = q - n * a.P;
  return int64_t(n) * a.K * a.P + p;
}

// Byte offset in grad_out of the B quad (k row krow of stage st, pixels
// q0 + 4 quad ..) whose first pixel has element offset `base` (b_base).
PW_HD uint32_t b_offset(const PWArgs& a, int st, int64_t base, int krow) {
  const int k = st * kBK + krow;
  if (base < 0 || k >= a.K) return kPad;
  return uint32_t((base + int64_t(k) * a.P) * 4);
}

// Matrix instruction q of a wave's 64 rows (or columns) covers elements
// 4 c + q of lane c = c16: the element of lane c16 in block q.
PW_HD int strided(int c16, int q) { return 4 * c16 + q; }

// The shapes this path takes: kernel 1x1, stride 1, no padding, input
// channels and pixels per image in multiples of 4, something to write, and
// grad_out, grad_input and weight below 2^31 bytes (32-bit buffer offsets).
// The tensors must also be 16-byte aligned (pw_applies).
inline bool pw_shape(const conv2d_params* p) {
  if (p == nullptr || validate_shape(p) != CONV2D_OK) return false;
  if (p->kernel_h != 1 || p->kernel_w != 1 || p->stride != 1 || p->padding_h != 0 ||
      p->padding_w != 0)
    return false;
  const int64_t P = int64_t(p->in_h) * p->in_w, N = p->batch;
  if (p->in_channels % 4 != 0 || P % 4 != 0) return false;
  if (N * p->out_channels * P * 4 >= kI31 || N * p->in_channels * P * 4 >= kI31) return false;
  if (int64_t(p->out_channels) * p->in_channels * 4 >= kI31) return false;
  return N * P * p->in_channels > 0;
}

inline void pw_plan(const conv2d_params* p, PWArgs* a, int fwd = 0) {
  memset(a, 0, sizeof(*a));
  a->fwd = fwd;
  a->M = int32_t(fwd ? p->out_channels : p->in_channels);
  a->K = int32_t(fwd ? p->in_channels : p->out_channels);
  a->P = int32_t(int64_t(p->in_h) * p->in_w);
  a->Q = int32_t(int64_t(p->batch) * a->P);
  a->TM = (a->M + kBM - 1) / kBM;
  a->TN = (a->Q + kBN - 1) / kBN;
}

// Whether a shape's default path (input gradient, or forward with fwd = 1)
// is this GEMM: forward shapes that the few-input-channel im2col GEMM takes
// stay there.
inline bool pw_route(const conv2d_params* p, int fwd, int f16) {
  return pw_shape(p) && (!fwd || !fg::fg_applies(p, f16));
}

// Tiles and multiply-adds issued for a shape (pw_shape must hold).
inline void pw_describe(const conv2d_params* p, int64_t* tiles, int64_t* macs, int fwd = 0) {
  PWArgs a;
  pw_plan(p, &a, fwd);
  *tiles = int64_t(a.TM) * a.TN;
  *macs = *tiles * kBM * kBN * int64_t((a.K + kBK - 1) / kBK) * kBK;
}

// Launch and host replay (pointwise_gemm.hip); fwd = 1: the forward
// convolution, with x in the place of grad_out and y in that of grad_input.
bool pw_applies(const conv2d_params* p, const float* go, const float* w, const float* gi);
// `cus`: compute units of the device; with more tiles than that, the
// launch uses two-buffer workgroups that share a CU two at a time.
int pw_launch(const float* go, const float* w, float* gi, const conv2d_params* p, int f16,
              void* stream, int fwd, int cus);
int pw_check(const conv2d_params* p, char* msg, size_t len, int fwd = 0);

}  // namespace pw
}  // namespace c2b
