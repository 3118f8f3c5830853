// Weight gradient of the forward cross-correlation as an implicit GEMM on
// CDNA4 (gfx950) matrix cores, its host replay, and its C-ABI entry points.
//
// What is computed (the other half of the backward pass of the convolution
// whose input gradient the rest of this library computes; its index map is
// the forward one, which is the map of the stride > 1 im2col branch of
// meganeura 0.2.0, conv2d_grad_input_gemm_coop.wgsl, read forwards):
//   grad_weight[co, ci, kh, kw] = sum over pixels p = (n, oh, ow) of
//       grad_out[n, co, oh, ow] * x[n, ci, s*oh - padding_h + kh, s*ow - padding_w + kw]
// with x zero outside the image.  As a GEMM: M = Co rows, N = Ci*kH*kW
// columns (ci, t = kh*kW + kw), contracted over all N*OH*OW pixels.
//
// How (fp32):
//  * The contraction is split: every workgroup takes a 64 x 64 tile of
//    (co, column) and one chunk of consecutive pixels, and writes its partial
//    tile to a caller-provided workspace; a second kernel adds the chunks'
//    partial tiles in a fixed order (deterministic) into grad_weight.
//    Workgroups are dealt to the 8 XCDs in contiguous runs, so the tiles of
//    one chunk share an L2.
//  * Column tiles come in two layouts.  Tap tiles: CB channels x TB taps
//    (CB * TB = 64, TB = 1, 2 or 4), slot s holding channel s / TB and tap
//    s % TB; every copy thread's columns then share one tap, so whether a
//    pixel reads inside the image is decided once per thread and stage, and
//    each element costs one add.  Flat tiles: 64 consecutive columns of the
//    weight layout, each element checked on its own; the planner takes them
//    only where tap tiles would be mostly empty (few channels, big kernel).
//  * A stage is 32 pixels.  Its operands go to LDS through registers:
//    A[co][px] = grad_out, B[slot][px] = the im2col of x, rows 32 + 4 floats
//    apart (each 16-lane group's 16-byte reads then hit distinct banks).
//    Each thread owns one pixel of the stage and 8 rows of each operand (rows
//    r0 + 8j, r0 = thread / 32); the pixel's (n, oh, ow) is decomposed once
//    per tile and advanced by 32 pixels per stage.  Loads whose element the
//    definition lacks read 0 (offset past the buffer range).  Rows past Co
//    and slots that are no column load real elements of a clamped row or
//    column: a product's row or column depends only on its own operand row
//    or column, and those are never stored.  Two stage buffers: stage s+1 is
//    written after the products of stage s, stage s+2 is loaded then; one
//    barrier per stage.  37 KB of LDS per workgroup: four workgroups share a
//    CU, so that one's copies can run beside the others' products (measured:
//    64-pixel stages with two workgroups per CU were up to 16% slower).
//  * Products: v_mfma_f32_16x16x4_f32, the k index being the pixel; lane
//    group g reads pixels 4g .. 4g+3 of each 16-pixel unit from A and B with
//    one 16-byte read each.  Four waves, each 2 x 2 blocks of 16 x 16.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "plan.hpp"
#include "tile_index.hpp"

namespace c2b {
namespace gw {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kTile = 64;                 // rows and columns (slots) of a tile
constexpr int kTileElems = kTile * kTile;
constexpr int kStagePx = 32;              // pixels of a stage
constexpr int kPitch = kStagePx + 4;      // floats between operand rows in LDS
constexpr int kThreads = 256;             // four waves
constexpr int kRowStep = kThreads / kStagePx;                 // copy: rows r0 + kRowStep * j
static_assert(kRowStep % 4 == 0, "a copy thread's slots must share their tap in tap tiles");
constexpr int kRowsPerThread = kTile * kStagePx / kThreads;   // 8 per operand
constexpr int kWaveRows = 32;             // each wave: 2 x 2 blocks of 16 x 16
constexpr int kTargetGroupsPerCU = 4;     // workgroups the split aims at, per CU
constexpr uint32_t kPad = 0x80000000u;    // byte offset past every buffer range

enum ColumnMode { kColsFlat = 0, kColsTap = 1 };

// By-value kernel arguments.
struct GWArgs {
  const float* go;
  const float* x;
  float* part;   // workspace: [nchunks][TM * TN][64 rows][64 slots]
  float* dw;     // [Co][Ci][KH][KW]
  int32_t N, Ci, H, W, Co, KH, KW, S, PH, PW, OH, OW;
  int32_t KHW;        // KH * KW
  int32_t NC;         // Ci * KHW
  int32_t OHOW;
  int32_t P;          // N * OH * OW pixels
  int32_t chunk_px;   // pixels per chunk (a multiple of kStagePx)
  int32_t nchunks;
  int32_t TM, TN;     // tiles along co and along columns
  int32_t mode;       // ColumnMode
  int32_t CB, TB;     // tap tiles: channels and taps of a tile
  int32_t TNT;        // tap tiles: tap blocks (column tile tn = cb * TNT + tb)
  uint32_t m_OW, m_OH;   // fast_div reciprocals of the pixel walk
};

// Tile of a workgroup: (chunk, co tile, column tile), the index dealt so that
// each XCD (workgroups x, x + 8, ...) takes one contiguous run.
struct GWTile {
  int chunk, tm, tn, co0, p_begin, p_end, nst;
};

C2B_HD GWTile gw_tile(const GWArgs& a, int bid) {
  const int T = a.TM * a.TN * a.nchunks;
  const int q = T >> 3, r = T & 7, x = bid & 7, k = bid >> 3;
  int t = x * q + imin(x, r) + k;
  GWTile g;
  g.tn = t % a.TN;
  t /= a.TN;
  g.tm = t % a.TM;
  g.chunk = t / a.TM;
  g.co0 = g.tm * kTile;
  g.p_begin = g.chunk * a.chunk_px;
  g.p_end = imin(g.p_begin + a.chunk_px, a.P);
  g.nst = (g.p_end - g.p_begin + kStagePx - 1) / kStagePx;
  return g;
}

// Slot s of column tile tn -> weight column (ci, t); false if the slot holds
// no column (then (ci, t) may lie outside the weight).
C2B_HD bool gw_slot_column(const GWArgs& a, int tn, int s, int* ci, int* t) {
  if (a.mode == kColsTap) {
    const int cb = tn / a.TNT, tb = tn - cb * a.TNT;
    *ci = cb * a.CB + s / a.TB;
    *t = tb * a.TB + s % a.TB;
    return *ci < a.Ci && *t < a.KHW;
  }
  const int c = tn * kTile + s;
  *ci = c / a.KHW;
  *t = c - *ci * a.KHW;
  return c < a.NC;
}

// The column a copy thread loads for slot s: the slot's own, or, for a slot
// that holds none, a real one (its values are never stored).
C2B_HD void gw_load_column(const GWArgs& a, int tn, int s, int* ci, int* kh, int* kw) {
  int c, t;
  gw_slot_column(a, tn, s, &c, &t);
  c = imin(c, a.Ci - 1);
  t = imin(t, a.KHW - 1);
  *ci = c;
  *kh = t / a.KW;
  *kw = t - *kh * a.KW;
}

// Byte offset of grad_out row co within an image, co clamped to a real row.
C2B_HD uint32_t gw_a_row(const GWArgs& a, int co) {
  return uint32_t(imin(co, a.Co - 1)) * uint32_t(a.OHOW) * 4u;
}

// A copy thread's pixel: index p and (n, oh, ow), decomposed once per tile
// and advanced by one stage at a time.
struct GWPixel {
  int p, n, oh, ow;
};

C2B_HD GWPixel gw_pixel_start(const GWArgs& a, int p) {
  GWPixel x;
  x.p = p;
  x.n = p / a.OHOW;
  const int q = p - x.n * a.OHOW;
  x.oh = q / a.OW;
  x.ow = q - x.oh * a.OW;
  return x;
}

// ow < OW + kStagePx and oh < OH + kStagePx here; the planner bounds
// (OW + kStagePx) * OW and (OH + kStagePx) * OH below 2^31, which makes
// fast_div exact.
C2B_HD void gw_pixel_next(const GWArgs& a, GWPixel* x) {
  x->p += kStagePx;
  x->ow += kStagePx;
  const int c1 = fast_div(x->ow, a.m_OW);
  x->ow -= c1 * a.OW;
  x->oh += c1;
  const int c2 = fast_div(x->oh, a.m_OH);
  x->oh -= c2 * a.OH;
  x->n += c2;
}

// Byte offset of the pixel's grad_out element in row 0; kPad past the chunk.
// Adding gw_a_row (< 2^31) keeps either case exact in 32 bits.
C2B_HD uint32_t gw_a_base(const GWArgs& a, bool pin, const GWPixel& x) {
  const uint32_t off = ((uint32_t(x.n) * uint32_t(a.Co) * uint32_t(a.OHOW)) +
                        uint32_t(x.oh * a.OW + x.ow)) * 4u;
  return pin ? off : kPad;
}

// Tap tiles: byte offset of the pixel's x element for tap (dkh, dkw) = (kh -
// PH, kw - PW) in channel 0, or kPad where the definition has no term; the
// channel's ci * H * W * 4 is added per element.
C2B_HD uint32_t gw_b_base(const GWArgs& a, bool pin, const GWPixel& x, int dkh, int dkw) {
  const int ih = x.oh * a.S + dkh, iw = x.ow * a.S + dkw;
  const bool term = pin & ((unsigned)ih < (unsigned)a.H) & ((unsigned)iw < (unsigned)a.W);
  const uint32_t off = (uint32_t(x.n) * uint32_t(a.Ci) * uint32_t(a.H * a.W) +
                        uint32_t(ih * a.W + iw)) * 4u;
  return term ? off : kPad;
}

// Flat tiles: the same per element, column (ci, kh, kw) given as xcol = ci*H*W
// + (kh - PH)*W + (kw - PW) and (dkh, dkw).  No branch: a branch per element
// would put a wait for the loads in flight at every join.
C2B_HD uint32_t gw_b_flat(const GWArgs& a, bool pin, const GWPixel& x, int xcol, int dkh,
                          int dkw) {
  const int ih = x.oh * a.S + dkh, iw = x.ow * a.S + dkw;
  const bool term = pin & ((unsigned)ih < (unsigned)a.H) & ((unsigned)iw < (unsigned)a.W);
  const uint32_t off = (uint32_t(x.n) * uint32_t(a.Ci) * uint32_t(a.H * a.W) +
                        uint32_t(xcol + x.oh * a.S * a.W + x.ow * a.S)) * 4u;
  return term ? off : kPad;
}

__device__ __forceinline__ float load_f32(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
}

template <bool TAP>
__global__ __launch_bounds__(kThreads, 4) void grad_weight_mm_kernel(const GWArgs a) {
  // [stage buffer][A, B][row * kPitch + px], 16-byte aligned (f32x4 storage)
  __shared__ f32x4 lds4[2 * 2 * kTile * kPitch / 4];
  auto lds = [&](int buf, int op) __attribute__((always_inline)) {
    return reinterpret_cast<float*>(lds4) + (buf * 2 + op) * kTile * kPitch;
  };
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int g = lane >> 4, c16 = lane & 15;
  const GWTile T = gw_tile(a, blockIdx.x);
  // copy: pixel cpx, rows r0 + kRowStep * j (wave-uniform for 64-pixel stages)
  const int cpx = tid & (kStagePx - 1);
  const int r0 = kStagePx == 64 ? wave : tid / kStagePx;

  const __amdgpu_buffer_rsrc_t rsA = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(a.go), 0, a.N * a.Co * a.OHOW * 4, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsB = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(a.x), 0, a.N * a.Ci * a.H * a.W * 4, 0x00020000);
  // per tile: the pixel-independent parts of the thread's offsets
  uint32_t arow[kRowsPerThread];
  int bcol[kRowsPerThread], bdkh[kRowsPerThread], bdkw[kRowsPerThread];
#pragma unroll
  for (int j = 0; j < kRowsPerThread; ++j) {
    arow[j] = gw_a_row(a, T.co0 + r0 + kRowStep * j);
    int ci, kh, kw;
    gw_load_column(a, T.tn, r0 + kRowStep * j, &ci, &kh, &kw);
    bdkh[j] = kh - a.PH;
    bdkw[j] = kw - a.PW;
    bcol[j] = TAP ? int(uint32_t(ci) * uint32_t(a.H * a.W) * 4u)
                  : ci * a.H * a.W + bdkh[j] * a.W + bdkw[j];
  }
  GWPixel px = gw_pixel_start(a, T.p_begin + cpx);

  float sa[kRowsPerThread], sb[kRowsPerThread];
  // the next stage's elements, then one stage on: all offsets first, then
  // all loads back to back
  auto load_stage = [&]() __attribute__((always_inline)) {
    const bool pin = px.p < T.p_end;
    const uint32_t abase = gw_a_base(a, pin, px);
    uint32_t oa[kRowsPerThread], ob[kRowsPerThread];
    if constexpr (TAP) {
      // tap tiles: all of the thread's columns share the tap of slot r0
      // (kRowStep is a multiple of the taps per tile)
      const uint32_t bbase = gw_b_base(a, pin, px, bdkh[0], bdkw[0]);
#pragma unroll
      for (int j = 0; j < kRowsPerThread; ++j) {
        oa[j] = abase + arow[j];
        ob[j] = bbase + uint32_t(bcol[j]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < kRowsPerThread; ++j) {
        oa[j] = abase + arow[j];
        ob[j] = gw_b_flat(a, pin, px, bcol[j], bdkh[j], bdkw[j]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < kRowsPerThread; ++j) {
      sa[j] = load_f32(rsA, oa[j]);
      sb[j] = load_f32(rsB, ob[j]);
    }
    gw_pixel_next(a, &px);
  };
  auto write_stage = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < kRowsPerThread; ++j) {
      lds(buf, 0)[(r0 + kRowStep * j) * kPitch + cpx] = sa[j];
      lds(buf, 1)[(r0 + kRowStep * j) * kPitch + cpx] = sb[j];
    }
  };

  f32x4 acc[2][2];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[m][b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  // 16-pixel unit u: lane group g supplies pixels 16u + 4g .. +3 of its A row
  // (co) and its B slot; MFMA q takes pixel 16u + 4g + q from every group
  auto compute = [&](int st) __attribute__((always_inline)) {
    const float* As = lds(st & 1, 0);
    const float* Bs = lds(st & 1, 1);
#pragma unroll
    for (int u = 0; u < kStagePx / 16; ++u) {
      f32x4 av[2], bv[2];
#pragma unroll
      for (int m = 0; m < 2; ++m)
        av[m] = *reinterpret_cast<const f32x4*>(
            As + (wm * kWaveRows + m * 16 + c16) * kPitch + 16 * u + 4 * g);
#pragma unroll
      for (int b = 0; b < 2; ++b)
        bv[b] = *reinterpret_cast<const f32x4*>(
            Bs + (wn * kWaveRows + b * 16 + c16) * kPitch + 16 * u + 4 * g);
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int b = 0; b < 2; ++b)
            acc[m][b] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[m][q], bv[b][q], acc[m][b], 0,
                                                             0, 0);
    }
  };

  load_stage();
  write_stage(0);
  if (T.nst > 1) load_stage();
  __syncthreads();
  for (int st = 0; st < T.nst; ++st) {
    compute(st);
    if (st + 1 < T.nst) write_stage((st + 1) & 1);
    if (st + 2 < T.nst) load_stage();
    __syncthreads();
  }

  // partial tile, whole: register r of block (m, b) holds row wm*32 + m*16 +
  // 4g + r, slot wn*32 + b*16 + c16
  float* part = a.part + (size_t(T.chunk) * a.TM * a.TN + size_t(T.tm) * a.TN + T.tn) * kTileElems;
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        part[(wm * kWaveRows + m * 16 + 4 * g + r) * kTile + wn * kWaveRows + b * 16 + c16] =
            acc[m][b][r];
}

// grad_weight[co, ci, t] = the sum over chunks of the partial tiles, in a
// fixed order.  A workgroup takes 256 / L groups of four consecutive
// partial-tile elements (row, slots s .. s+3) and L chunk lanes (L = 1, 2,
// .., 16, about nchunks / 8): thread (group q, lane l) adds chunks l, l + L,
// ... with 16-byte loads, four in flight, then lane 0 adds the L lane sums in
// lane order.  Rows past Co and slots with no column store nothing.
constexpr int kReduceMaxLanes = 16;

int reduce_lanes(int nchunks) {
  int lanes = 1;
  while (lanes < kReduceMaxLanes && lanes * 8 < nchunks) lanes *= 2;
  return lanes;
}

__global__ __launch_bounds__(256) void grad_weight_reduce_kernel(const GWArgs a, int lanes) {
  __shared__ f32x4 sums[256];
  const int quads = 256 / lanes;
  const int q = threadIdx.x % quads, l = threadIdx.x / quads;
  const int total = a.TM * a.TN * kTileElems;   // a multiple of 4 * 256
  const int e = (blockIdx.x * quads + q) * 4;
  const f32x4* src = reinterpret_cast<const f32x4*>(a.part + e);
  const size_t stride = size_t(total) / 4;
  f32x4 s[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) s[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  int k = l;
  for (; k + 3 * lanes < a.nchunks; k += 4 * lanes) {
    f32x4 v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = src[size_t(k + i * lanes) * stride];
#pragma unroll
    for (int i = 0; i < 4; ++i) s[i] += v[i];
  }
  for (int i = 0; k < a.nchunks; k += lanes, ++i) s[i] += src[size_t(k) * stride];
  f32x4 t = (s[0] + s[1]) + (s[2] + s[3]);
  if (lanes > 1) {
    sums[threadIdx.x] = t;
    __syncthreads();
    if (l != 0) return;
    for (int i = 1; i < lanes; ++i) t += sums[i * quads + q];
  }
  const int tile = e / kTileElems, rs = e - tile * kTileElems;
  const int tm = tile / a.TN, tn = tile - tm * a.TN;
  const int co = tm * kTile + rs / kTile;
  if (co >= a.Co) return;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    int ci, c;
    if (gw_slot_column(a, tn, rs % kTile + r, &ci, &c))
      a.dw[(co * a.Ci + ci) * a.KHW + c] = t[r];
  }
}

// ---------------------------------------------------------------------------
// Host side: plan, workspace size, replay.

constexpr int64_t kI31 = int64_t(1) << 31;
constexpr int kVariants = 4;   // 0: flat tiles; 1, 2, 3: tap tiles of 1, 2, 4 taps

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Column slots of a variant (tiles x 64).
int64_t variant_slots(int64_t Ci, int64_t KHW, int v) {
  if (v == 0) return cdiv(Ci * KHW, kTile) * kTile;
  const int64_t TB = int64_t(1) << (v - 1), CB = kTile / TB;
  return cdiv(Ci, CB) * cdiv(KHW, TB) * kTile;
}

// The planner's variant: the tap layout with the fewest slots (the fewer
// taps per tile on a tie), unless it has over 1.5 times the flat layout's
// slots; a flat slot costs about that much more to copy.
int choose_variant(int64_t Ci, int64_t KHW) {
  int best = 1;
  for (int v = 2; v < kVariants; ++v)
    if (variant_slots(Ci, KHW, v) < variant_slots(Ci, KHW, best)) best = v;
  return 2 * variant_slots(Ci, KHW, best) <= 3 * variant_slots(Ci, KHW, 0) ? best : 0;
}

// Plan of a shape for `cus` compute units and a variant (-1: the planner's);
// CONV2D_OK or an error code.
int gw_plan(const conv2d_params* p, int cus, int variant, GWArgs* a) {
  int rc = validate_shape(p);
  if (rc != CONV2D_OK) return rc;
  if (variant < -1 || variant >= kVariants) return CONV2D_ERR_UNSUPPORTED;
  std::memset(a, 0, sizeof(*a));
  a->N = int32_t(p->batch);
  a->Ci = int32_t(p->in_channels);
  a->H = int32_t(p->in_h);
  a->W = int32_t(p->in_w);
  a->Co = int32_t(p->out_channels);
  a->KH = int32_t(p->kernel_h);
  a->KW = int32_t(p->kernel_w);
  a->S = int32_t(p->stride);
  a->PH = int32_t(p->padding_h);
  a->PW = int32_t(p->padding_w);
  a->OH = int32_t(p->out_h);
  a->OW = int32_t(p->out_w);
  const int64_t KHW = int64_t(p->kernel_h) * p->kernel_w;
  const int64_t NC = int64_t(p->in_channels) * KHW;
  const int64_t OHOW = int64_t(p->out_h) * p->out_w;
  const int64_t P = int64_t(p->batch) * OHOW;
  // whole-tensor byte offsets (chunks cross images), and the pixel walk's
  // fast_div bounds
  if (P >= kI31 || int64_t(p->batch) * p->out_channels * OHOW * 4 >= kI31 ||
      int64_t(p->batch) * p->in_channels * p->in_h * p->in_w * 4 >= kI31 ||
      (int64_t(p->out_w) + kStagePx) * p->out_w >= kI31 ||
      (int64_t(p->out_h) + kStagePx) * p->out_h >= kI31)
    return CONV2D_ERR_OVERFLOW;
  a->KHW = int32_t(KHW);
  a->NC = int32_t(NC);
  a->OHOW = int32_t(OHOW);
  a->P = int32_t(P);
  a->m_OW = fast_div_magic(uint32_t(std::max<int32_t>(a->OW, 1)));
  a->m_OH = fast_div_magic(uint32_t(std::max<int32_t>(a->OH, 1)));
  const int v = variant >= 0 ? variant : choose_variant(p->in_channels, KHW);
  if (v == 0) {
    a->mode = kColsFlat;
    a->CB = a->TB = a->TNT = 0;
    a->TN = int32_t(cdiv(NC, kTile));
  } else {
    a->mode = kColsTap;
    a->TB = 1 << (v - 1);
    a->CB = kTile / a->TB;
    a->TNT = int32_t(cdiv(KHW, a->TB));
    a->TN = int32_t(cdiv(p->in_channels, a->CB) * a->TNT);
  }
  a->TM = int32_t(cdiv(a->Co, kTile));
  if (cus < 1) cus = kDefaultCUs;
  if (P == 0 || a->TM == 0 || a->TN == 0) {
    a->chunk_px = kStagePx;
    a->nchunks = 0;   // no pixel: grad_weight is zeros (no tile, or no output)
    return CONV2D_OK;
  }
  const int64_t target = int64_t(kTargetGroupsPerCU) * cus;
  const int64_t tiles = int64_t(a->TM) * a->TN;
  int64_t chunk = cdiv(P * tiles, target);
  chunk = std::max<int64_t>(kStagePx, cdiv(chunk, kStagePx) * kStagePx);
  a->chunk_px = int32_t(std::min<int64_t>(chunk, cdiv(P, kStagePx) * kStagePx));
  a->nchunks = int32_t(cdiv(P, a->chunk_px));
  // pixel indices up to nchunks * chunk_px + 64, grid, workspace
  if (int64_t(a->nchunks) * a->chunk_px + kStagePx >= kI31 || tiles * a->nchunks >= kI31 ||
      tiles * kTileElems >= kI31 ||
      int64_t(a->nchunks) * tiles * kTileElems * 4 >= (int64_t(1) << 40))
    return CONV2D_ERR_OVERFLOW;
  return CONV2D_OK;
}

size_t gw_workspace_bytes(const GWArgs& a) {
  return size_t(a.nchunks) * size_t(a.TM) * size_t(a.TN) * kTileElems * sizeof(float);
}

namespace {
struct Failure {
  std::string msg;
};
#define GW_REQUIRE(cond, ...)                                   \
  do {                                                          \
    if (!(cond)) {                                              \
      char buf_[512];                                           \
      std::snprintf(buf_, sizeof buf_, __VA_ARGS__);            \
      throw Failure{std::string(#cond) + ": " + buf_};          \
    }                                                           \
  } while (0)
}  // namespace

// Host replay of every workgroup and thread, through the kernel's own index
// functions and in its order (the pixel walk included), checked against the
// definition: for every stored row co and column (ci, t), each pixel of the
// chunk contributes grad_out[n, co, oh, ow] * x[n, ci, ih, iw] where the
// definition has that term and 0 elsewhere (a load past the buffer range
// reads 0); each LDS cell of a stage is written by exactly one thread; the
// products pair A and B cells of the same pixel and the lane's own row and
// slot; every partial-tile element is stored once; and the reduction takes
// every weight element from exactly one (row, slot).
int gw_check(const conv2d_params* p, int variant, char* msg, size_t len) {
  GWArgs a;
  int rc = gw_plan(p, kDefaultCUs, variant, &a);
  if (rc != CONV2D_OK) return rc;
  try {
    const int64_t tiles = int64_t(a.TM) * a.TN;
    const int64_t nparts = int64_t(a.nchunks) * tiles * kTileElems;
    std::vector<unsigned char> stored(size_t(nparts), 0);
    const int64_t go_bytes = int64_t(a.N) * a.Co * a.OHOW * 4;
    const int64_t x_bytes = int64_t(a.N) * a.Ci * a.H * a.W * 4;
    for (int bid = 0; bid < tiles * a.nchunks; ++bid) {
      const GWTile T = gw_tile(a, bid);
      GW_REQUIRE(T.chunk >= 0 && T.chunk < a.nchunks && T.tm < a.TM && T.tn < a.TN &&
                     T.nst >= 1 && T.p_begin < a.P,
                 "bid %d tile", bid);
      // per thread: the kernel's per-tile values and its pixel walk
      std::vector<GWPixel> px(kThreads);
      std::vector<int> bcol(size_t(kThreads) * kRowsPerThread), bdkh(bcol.size()),
          bdkw(bcol.size());
      std::vector<uint32_t> arow(bcol.size());
      for (int tid = 0; tid < kThreads; ++tid) {
        const int r0 = tid / kStagePx;
        for (int j = 0; j < kRowsPerThread; ++j) {
          const size_t k = size_t(tid) * kRowsPerThread + j;
          arow[k] = gw_a_row(a, T.co0 + r0 + kRowStep * j);
          int ci, kh, kw;
          gw_load_column(a, T.tn, r0 + kRowStep * j, &ci, &kh, &kw);
          GW_REQUIRE(ci >= 0 && ci < a.Ci && kh >= 0 && kh < a.KH && kw >= 0 && kw < a.KW,
                     "load column of slot %d", r0 + kRowStep * j);
          bdkh[k] = kh - a.PH;
          bdkw[k] = kw - a.PW;
          bcol[k] = a.mode == kColsTap ? int(uint32_t(ci) * uint32_t(a.H * a.W) * 4u)
                                       : ci * a.H * a.W + bdkh[k] * a.W + bdkw[k];
        }
        px[size_t(tid)] = gw_pixel_start(a, T.p_begin + (tid & (kStagePx - 1)));
      }
      for (int st = 0; st < T.nst; ++st) {
        std::vector<unsigned char> cell(2 * kTile * kPitch, 0);
        for (int tid = 0; tid < kThreads; ++tid) {
          const int cpx = tid & (kStagePx - 1), r0 = tid / kStagePx;
          GWPixel& x = px[size_t(tid)];
          const int pix = T.p_begin + st * kStagePx + cpx;
          GW_REQUIRE(x.p == pix, "pixel walk index %d, want %d", x.p, pix);
          const bool pin = x.p < T.p_end;
          // the definition's decomposition of this pixel
          const int64_t dn = pix / a.OHOW, dq = pix % a.OHOW, doh = dq / a.OW, dow = dq % a.OW;
          if (pin)
            GW_REQUIRE(x.n == dn && x.oh == doh && x.ow == dow, "pixel walk at %d", pix);
          const uint32_t abase = gw_a_base(a, pin, x);
          const size_t k0 = size_t(tid) * kRowsPerThread;
          const uint32_t bbase = gw_b_base(a, pin, x, bdkh[k0], bdkw[k0]);
          for (int j = 0; j < kRowsPerThread; ++j) {
            const int row = r0 + kRowStep * j;
            const size_t k = k0 + j;
            for (int op = 0; op < 2; ++op) {
              const int idx = op * kTile * kPitch + row * kPitch + cpx;
              GW_REQUIRE(cell[size_t(idx)] == 0, "stage %d cell written twice", st);
              cell[size_t(idx)] = 1;
            }
            const uint32_t ao = abase + arow[k];
            uint32_t bo;
            if (a.mode == kColsTap) {
              GW_REQUIRE(bdkh[k] == bdkh[k0] && bdkw[k] == bdkw[k0],
                         "tap tile: slots of one thread with different taps");
              bo = bbase + uint32_t(bcol[k]);
            } else {
              bo = gw_b_flat(a, pin, x, bcol[k], bdkh[k], bdkw[k]);
            }
            const int co = T.co0 + row;
            int ci, t;
            const bool col = gw_slot_column(a, T.tn, row, &ci, &t);
            if (co >= a.Co || !col) continue;   // never stored
            const int kh = t / a.KW, kw = t % a.KW;
            if (!pin) {
              GW_REQUIRE(int64_t(ao) >= go_bytes || int64_t(bo) >= x_bytes,
                         "pixel %d past the chunk contributes", pix);
              continue;
            }
            GW_REQUIRE(int64_t(ao) == ((dn * a.Co + co) * a.OHOW + dq) * 4,
                       "A element of co %d pixel %d", co, pix);
            const int64_t ih = doh * a.S - a.PH + kh, iw = dow * a.S - a.PW + kw;
            if (ih >= 0 && ih < a.H && iw >= 0 && iw < a.W) {
              GW_REQUIRE(int64_t(bo) == (((dn * a.Ci + ci) * a.H + ih) * a.W + iw) * 4,
                         "B element of column (%d, %d) pixel %d", ci, t, pix);
            } else {
              GW_REQUIRE(int64_t(bo) >= x_bytes, "B padding of column (%d, %d) pixel %d", ci, t,
                         pix);
            }
          }
          gw_pixel_next(a, &x);
        }
        for (int op = 0; op < 2; ++op)
          for (int row = 0; row < kTile; ++row)
            for (int c = 0; c < kStagePx; ++c)
              GW_REQUIRE(cell[size_t(op * kTile * kPitch + row * kPitch + c)] == 1,
                         "stage %d cell never written", st);
      }
      // products: each lane's A reads are its row, its B reads its slot, both
      // at the same pixels; then its stores
      for (int tid = 0; tid < kThreads; ++tid) {
        const int lane = tid & 63, wave = tid >> 6, wm = wave & 1, wn = wave >> 1;
        const int g = lane >> 4, c16 = lane & 15;
        for (int u = 0; u < kStagePx / 16; ++u)
          for (int m = 0; m < 2; ++m)
            for (int b = 0; b < 2; ++b) {
              const int ar = wm * kWaveRows + m * 16 + c16, br = wn * kWaveRows + b * 16 + c16;
              const int px0 = 16 * u + 4 * g;
              GW_REQUIRE(ar < kTile && br < kTile && px0 + 4 <= kStagePx &&
                             (ar * kPitch + px0) % 4 == 0 && (br * kPitch + px0) % 4 == 0,
                         "operand read");
            }
        for (int m = 0; m < 2; ++m)
          for (int b = 0; b < 2; ++b)
            for (int r = 0; r < 4; ++r) {
              const int row = wm * kWaveRows + m * 16 + 4 * g + r;
              const int slot = wn * kWaveRows + b * 16 + c16;
              const int64_t e = ((int64_t(T.chunk) * a.TM + T.tm) * a.TN + T.tn) * kTileElems +
                                row * kTile + slot;
              GW_REQUIRE(e >= 0 && e < nparts && stored[size_t(e)] == 0, "partial stored twice");
              stored[size_t(e)] = 1;
            }
      }
    }
    for (int64_t e = 0; e < nparts; ++e) GW_REQUIRE(stored[size_t(e)] == 1, "partial never stored");
    // the chunks cover every pixel once
    GW_REQUIRE(a.nchunks == 0 || (int64_t(a.nchunks - 1) * a.chunk_px < a.P &&
                                  int64_t(a.nchunks) * a.chunk_px >= a.P && a.chunk_px % kStagePx == 0),
               "chunks do not cover the pixels");
    // the reduction's workgroups cover the partial-tile elements in whole
    // groups of four, and write every weight element from exactly one (row,
    // slot)
    const int lanes = reduce_lanes(a.nchunks);
    GW_REQUIRE(lanes >= 1 && lanes <= kReduceMaxLanes && 256 % lanes == 0 &&
                   (tiles * kTileElems * lanes) % (4 * 256) == 0,
               "reduction grid");
    std::vector<unsigned char> dw_hit(size_t(int64_t(a.Co) * a.NC), 0);
    for (int64_t e = 0; e < tiles * kTileElems; ++e) {
      const int tile = int(e / kTileElems), rs = int(e % kTileElems);
      const int tm = tile / a.TN, tn = tile % a.TN;
      const int co = tm * kTile + rs / kTile;
      int ci, t;
      if (!gw_slot_column(a, tn, rs % kTile, &ci, &t) || co >= a.Co) continue;
      GW_REQUIRE(ci >= 0 && ci < a.Ci && t >= 0 && t < a.KHW, "slot column out of the weight");
      const size_t d = size_t((int64_t(co) * a.Ci + ci) * a.KHW + t);
      GW_REQUIRE(dw_hit[d] == 0, "weight element (%d, %d, %d) reduced twice", co, ci, t);
      dw_hit[d] = 1;
    }
    for (size_t d = 0; d < dw_hit.size(); ++d)
      GW_REQUIRE(dw_hit[d] == 1, "weight element %zu never reduced", d);
  } catch (const Failure& f) {
    if (msg && len) {
      std::strncpy(msg, f.msg.c_str(), len - 1);
      msg[len - 1] = 0;
    }
    return 1;
  }
  if (msg && len) msg[0] = 0;
  return CONV2D_OK;
}

// Pointer checks: inputs go, x; outputs dw and the workspace (16-byte
// aligned: the reduction reads it in 16-byte loads), which may not overlap
// each other or an input.
int gw_check_pointers(const float* go, const float* x, const float* dw, const void* ws,
                      size_t ws_bytes, const conv2d_params* p, const GWArgs& a) {
  const uint64_t n_go = uint64_t(p->batch) * p->out_channels * p->out_h * p->out_w;
  const uint64_t n_x = uint64_t(p->batch) * p->in_channels * p->in_h * p->in_w;
  const uint64_t n_dw = uint64_t(p->out_channels) * p->in_channels * p->kernel_h * p->kernel_w;
  const uint64_t ws_need = gw_workspace_bytes(a);
  if ((n_go && go == nullptr) || (n_x && x == nullptr) || (n_dw && dw == nullptr))
    return CONV2D_ERR_NULL_PTR;
  if (ws_need && (ws == nullptr || ws_bytes < ws_need || reinterpret_cast<uintptr_t>(ws) % 16))
    return CONV2D_ERR_WORKSPACE;
  auto overlap = [](const void* a0, uint64_t na, const void* b0, uint64_t nb) {
    if (na == 0 || nb == 0) return false;
    const uintptr_t a = reinterpret_cast<uintptr_t>(a0), b = reinterpret_cast<uintptr_t>(b0);
    return a < b + nb && b < a + na;
  };
  const uint64_t b_go = n_go * 4, b_x = n_x * 4, b_dw = n_dw * 4;
  if (overlap(dw, b_dw, go, b_go) || overlap(dw, b_dw, x, b_x) || overlap(ws, ws_need, go, b_go) ||
      overlap(ws, ws_need, x, b_x) || overlap(ws, ws_need, dw, b_dw))
    return CONV2D_ERR_ALIAS;
  return CONV2D_OK;
}

int device_cus_gw() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return kDefaultCUs;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < 1)
    return kDefaultCUs;
  return cus;
}

int run(const float* grad_out, const float* x, float* grad_weight, const conv2d_params* p,
        void* workspace, size_t workspace_bytes, void* stream, int variant) {
  if (p == nullptr) return CONV2D_ERR_NULL_PTR;
  GWArgs a;
  int rc = gw_plan(p, device_cus_gw(), variant, &a);
  if (rc != CONV2D_OK) return rc;
  rc = gw_check_pointers(grad_out, x, grad_weight, workspace, workspace_bytes, p, a);
  if (rc != CONV2D_OK) return rc;
  const int total = a.TM * a.TN * kTileElems;
  if (total == 0) return CONV2D_OK;
  a.go = grad_out;
  a.x = x;
  a.dw = grad_weight;
  a.part = static_cast<float*>(workspace);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (a.nchunks > 0) {
    if (a.mode == kColsTap)
      hipLaunchKernelGGL(grad_weight_mm_kernel<true>, dim3(a.TM * a.TN * a.nchunks),
                         dim3(kThreads), 0, st, a);
    else
      hipLaunchKernelGGL(grad_weight_mm_kernel<false>, dim3(a.TM * a.TN * a.nchunks),
                         dim3(kThreads), 0, st, a);
  }
  const int lanes = reduce_lanes(a.nchunks);
  hipLaunchKernelGGL(grad_weight_reduce_kernel, dim3(total * lanes / (4 * 256)), dim3(256), 0,
                     st, a, lanes);
  return hipGetLastError() == hipSuccess ? CONV2D_OK : CONV2D_ERR_HIP;
}

// ---------------------------------------------------------------------------
// Allocation-free entry point: the partial tiles go to a scratch array the
// library holds in device memory (each device its own copy, from the load of
// the code object until the process ends) instead of a caller's workspace.
// The array's name is only a stand-in in host code; its device address comes
// from hipGetSymbolAddress, once per device, with that device current.  The
// product kernel writes every partial element it reads back, so nothing has
// to be cleared between calls.

constexpr size_t kScratchBytes = CONV2D_GRAD_WEIGHT_NOALLOC_MAX_BYTES;
static_assert(kScratchBytes % 256 == 0, "whole 256-byte lines");
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

constexpr int kMaxScratchDevices = 64;

// Device address of the current device's scratch (nullptr on a HIP error).
void* scratch_address() {
  static std::mutex mu;
  static void* addr[kMaxScratchDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    addr[dev] = ptr;
  }
  return addr[dev];
}

int run_noalloc(const float* grad_out, const float* x, float* grad_weight,
                const conv2d_params* p, void* stream) {
  if (p == nullptr) return CONV2D_ERR_NULL_PTR;
  GWArgs a;
  int rc = gw_plan(p, device_cus_gw(), -1, &a);
  if (rc != CONV2D_OK) return rc;
  if (gw_workspace_bytes(a) > kScratchBytes) return CONV2D_ERR_SCRATCH;
  // the caller's tensors first (the scratch overlaps none of them), so that
  // every argument error is reported before any HIP call
  GWArgs tensors_only = a;
  tensors_only.nchunks = 0;
  rc = gw_check_pointers(grad_out, x, grad_weight, nullptr, 0, p, tensors_only);
  if (rc != CONV2D_OK) return rc;
  void* ws = scratch_address();
  if (ws == nullptr) return CONV2D_ERR_HIP;
  return run(grad_out, x, grad_weight, p, ws, kScratchBytes, stream, -1);
}

int workspace_size(const conv2d_params* p, int variant, size_t* bytes) {
  if (p == nullptr || bytes == nullptr) return CONV2D_ERR_NULL_PTR;
  GWArgs a;
  const int rc = gw_plan(p, device_cus_gw(), variant, &a);
  if (rc != CONV2D_OK) return rc;
  *bytes = gw_workspace_bytes(a);
  return CONV2D_OK;
}

}  // namespace gw
}  // namespace c2b

extern "C" int conv2d_grad_weight_workspace_size(const conv2d_params* p, size_t* bytes) {
  return c2b::gw::workspace_size(p, -1, bytes);
}

extern "C" int conv2d_grad_weight(const float* grad_out, const float* x, float* grad_weight,
                                  const conv2d_params* p, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  return c2b::gw::run(grad_out, x, grad_weight, p, workspace, workspace_bytes, stream, -1);
}

extern "C" int conv2d_grad_weight_noalloc(const float* grad_out, const float* x,
                                          float* grad_weight, const conv2d_params* p,
                                          void* stream) {
  return c2b::gw::run_noalloc(grad_out, x, grad_weight, p, stream);
}

extern "C" int conv2d_grad_weight_variant_workspace_size(const conv2d_params* p, int variant,
                                                         size_t* bytes) {
  return c2b::gw::workspace_size(p, variant, bytes);
}

extern "C" int conv2d_grad_weight_variant(const float* grad_out, const float* x,
                                          float* grad_weight, const conv2d_params* p,
                                          void* workspace, size_t workspace_bytes, void* stream,
                                          int variant) {
  return c2b::gw::run(grad_out, x, grad_weight, p, workspace, workspace_bytes, stream, variant);
}

extern "C" int conv2d_describe_grad_weight_plan(const conv2d_params* p, int variant,
                                                int32_t* info, int n) {
  if (p == nullptr || (info == nullptr && n > 0)) return CONV2D_ERR_NULL_PTR;
  c2b::gw::GWArgs a;
  const int rc = c2b::gw::gw_plan(p, c2b::gw::device_cus_gw(), variant, &a);
  if (rc != CONV2D_OK) return rc;
  const int32_t v = a.mode == c2b::gw::kColsFlat ? 0 : (a.TB == 1 ? 1 : a.TB == 2 ? 2 : 3);
  const int32_t vals[] = {v, a.CB, a.TB, a.TM, a.TN, a.nchunks, a.chunk_px};
  for (int i = 0; i < n && i < int(sizeof vals / sizeof vals[0]); ++i) info[i] = vals[i];
  return CONV2D_OK;
}

extern "C" int conv2d_check_indexing_grad_weight(const conv2d_params* p, char* msg,
                                                 size_t msg_len) {
  return c2b::gw::gw_check(p, -1, msg, msg_len);
}

extern "C" int conv2d_check_indexing_grad_weight_variant(const conv2d_params* p, int variant,
                                                         char* msg, size_t msg_len) {
  return c2b::gw::gw_check(p, variant, msg, msg_len);
}
