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
// columns c = ci*kH*kW + kh*kW + kw (the weight's own layout), contracted over
// all N*OH*OW pixels.
//
// How (v1, fp32):
//  * The contraction is split: every workgroup takes a 64 x 64 (co, c) tile
//    and one chunk of consecutive pixels, and writes its partial tile to a
//    caller-provided workspace; a second kernel adds the chunks' partial
//    tiles in a fixed order (deterministic) into grad_weight.  Workgroups are
//    dealt to the 8 XCDs in contiguous runs, so the tiles of one chunk share
//    an L2.
//  * A stage is 64 pixels.  Its operands go to LDS through registers:
//    A[co][px] = grad_out, B[c][px] = the im2col of x, rows 64 + 4 floats
//    apart (each 16-lane group's 16-byte reads then hit distinct banks).
//    Each thread owns one pixel of the stage and 16 rows of each operand; the
//    pixel's (n, oh, ow) is decomposed once per stage and each column's
//    (ci, kh, kw) once per tile.  Loads outside the image read 0 (buffer
//    range).  Two stage buffers: stage s+1 is written after the products of
//    stage s, stage s+2 is loaded then; one barrier per stage.
//  * Products: v_mfma_f32_16x16x4_f32, the k index being the pixel; lane
//    group g reads pixels 4g .. 4g+3 of each 16-pixel unit from A and B with
//    one 16-byte read each.  Four waves, each 2 x 2 blocks of 16 x 16.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "plan.hpp"
#include "tile_index.hpp"

namespace c2b {
namespace gw {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kTile = 64;                 // rows and columns of a tile
constexpr int kStagePx = 64;              // pixels of a stage
constexpr int kPitch = kStagePx + 4;      // floats between operand rows in LDS
constexpr int kThreads = 256;             // four waves
constexpr int kRowsPerThread = kTile * kStagePx / kThreads;   // 16 per operand
constexpr int kWaveRows = 32;             // each wave: 2 x 2 blocks of 16 x 16
constexpr int kTargetGroupsPerCU = 2;     // workgroups the split aims at, per CU
constexpr uint32_t kPad = 0x80000000u;    // byte offset past every buffer range

// By-value kernel arguments.
struct GWArgs {
  const float* go;
  const float* x;
  float* part;   // workspace: [nchunks][Co][NC]
  float* dw;     // [Co][NC]
  int32_t N, Ci, H, W, Co, KH, KW, S, PH, PW, OH, OW;
  int32_t NC;         // Ci * KH * KW
  int32_t OHOW;
  int32_t P;          // N * OH * OW pixels
  int32_t chunk_px;   // pixels per chunk (a multiple of kStagePx)
  int32_t nchunks;
  int32_t TM, TN;     // tiles along co and along columns
  uint32_t m_KHW, m_KW;   // fast_div reciprocals
};

// Tile of a workgroup: (chunk, co tile, column tile), the index dealt so that
// each XCD (workgroups x, x + 8, ...) takes one contiguous run.
struct GWTile {
  int chunk, co0, c0, p_begin, p_end, nst;
};

C2B_HD GWTile gw_tile(const GWArgs& a, int bid) {
  const int T = a.TM * a.TN * a.nchunks;
  const int q = T >> 3, r = T & 7, x = bid & 7, k = bid >> 3;
  int t = x * q + imin(x, r) + k;
  GWTile g;
  const int tn = t % a.TN;
  t /= a.TN;
  const int tm = t % a.TM;
  g.chunk = t / a.TM;
  g.co0 = tm * kTile;
  g.c0 = tn * kTile;
  g.p_begin = g.chunk * a.chunk_px;
  g.p_end = imin(g.p_begin + a.chunk_px, a.P);
  g.nst = (g.p_end - g.p_begin + kStagePx - 1) / kStagePx;
  return g;
}

// Column c -> its part of the x offset, ci*H*W + (kh - PH)*W + (kw - PW), and
// (kh << 16) | kw; khw = -1 for a column past NC.
C2B_HD void gw_column(const GWArgs& a, int c, int* xcol, int* khw) {
  if (c >= a.NC) {
    *xcol = 0;
    *khw = -1;
    return;
  }
  const int ci = fast_div(c, a.m_KHW);
  const int rem = c - ci * a.KH * a.KW;
  const int kh = fast_div(rem, a.m_KW);
  const int kw = rem - kh * a.KW;
  *xcol = ci * a.H * a.W + (kh - a.PH) * a.W + (kw - a.PW);
  *khw = (kh << 16) | kw;
}

// Pixel p -> (n, q = oh*OW + ow, oh, ow); false if p is past the chunk (the
// decomposition is then that of a pixel the caller does not use).  No branch
// (see gw_a_offset).
C2B_HD bool gw_pixel(const GWArgs& a, int p, int p_end, int* n, int* q, int* oh, int* ow) {
  *n = p / a.OHOW;
  *q = p - *n * a.OHOW;
  *oh = *q / a.OW;
  *ow = *q - *oh * a.OW;
  return p < p_end;
}

// Byte offsets into grad_out / x of the A element (row co) and the B element
// (column with xcol, khw) at pixel (n, q, oh, ow); kPad if the element is 0.
// Computed without branches (a select at the end): a branch per element
// would put a wait for the loads in flight at every join.
C2B_HD uint32_t gw_a_offset(const GWArgs& a, bool pin, int n, int q, int co) {
  const uint32_t off = uint32_t(((n * a.Co + co) * a.OHOW + q) * 4);
  return (pin & (co < a.Co)) ? off : kPad;
}
C2B_HD uint32_t gw_b_offset(const GWArgs& a, bool pin, int n, int oh, int ow, int xcol,
                            int khw) {
  const int kh = khw >> 16, kw = khw & 0xffff;
  const int ih = oh * a.S + kh - a.PH, iw = ow * a.S + kw - a.PW;
  const bool term = pin & (khw >= 0) & ((unsigned)ih < (unsigned)a.H) & ((unsigned)iw < (unsigned)a.W);
  const uint32_t off = uint32_t((n * a.Ci * a.H * a.W + xcol + oh * a.S * a.W + ow * a.S) * 4);
  return term ? off : kPad;
}

__device__ __forceinline__ float load_f32(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
}

__global__ __launch_bounds__(kThreads, 2) void grad_weight_mm_kernel(const GWArgs a) {
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
  const int cpx = tid & (kStagePx - 1), r0 = tid / kStagePx;   // copy pixel, first row

  const __amdgpu_buffer_rsrc_t rsA = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(a.go), 0, a.N * a.Co * a.OHOW * 4, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsB = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(a.x), 0, a.N * a.Ci * a.H * a.W * 4, 0x00020000);
  int xcol[kRowsPerThread], khw[kRowsPerThread];
#pragma unroll
  for (int j = 0; j < kRowsPerThread; ++j) gw_column(a, T.c0 + r0 + 4 * j, &xcol[j], &khw[j]);

  float sa[kRowsPerThread], sb[kRowsPerThread];
  // all offsets first, then all loads back to back
  auto load_stage = [&](int st) __attribute__((always_inline)) {
    int n, q, oh, ow;
    const bool pin = gw_pixel(a, T.p_begin + st * kStagePx + cpx, T.p_end, &n, &q, &oh, &ow);
    uint32_t oa[kRowsPerThread], ob[kRowsPerThread];
#pragma unroll
    for (int j = 0; j < kRowsPerThread; ++j) {
      oa[j] = gw_a_offset(a, pin, n, q, T.co0 + r0 + 4 * j);
      ob[j] = gw_b_offset(a, pin, n, oh, ow, xcol[j], khw[j]);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < kRowsPerThread; ++j) {
      sa[j] = load_f32(rsA, oa[j]);
      sb[j] = load_f32(rsB, ob[j]);
    }
  };
  auto write_stage = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < kRowsPerThread; ++j) {
      lds(buf, 0)[(r0 + 4 * j) * kPitch + cpx] = sa[j];
      lds(buf, 1)[(r0 + 4 * j) * kPitch + cpx] = sb[j];
    }
  };

  f32x4 acc[2][2];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[m][b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  // 16-pixel unit u: lane group g supplies pixels 16u + 4g .. +3 of its A row
  // (co) and its B column; MFMA q takes pixel 16u + 4g + q from every group
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

  load_stage(0);
  write_stage(0);
  if (T.nst > 1) load_stage(1);
  __syncthreads();
  for (int st = 0; st < T.nst; ++st) {
    compute(st);
    if (st + 1 < T.nst) write_stage((st + 1) & 1);
    if (st + 2 < T.nst) load_stage(st + 2);
    __syncthreads();
  }

  // partial tile: register r of block (m, b) holds row co0 + wm*32 + m*16 +
  // 4g + r, column c0 + wn*32 + b*16 + c16
  float* part = a.part + (size_t)T.chunk * a.Co * a.NC;
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int c = T.c0 + wn * kWaveRows + b * 16 + c16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int co = T.co0 + wm * kWaveRows + m * 16 + 4 * g + r;
        if (co < a.Co && c < a.NC) part[(size_t)co * a.NC + c] = acc[m][b][r];
      }
    }
}

// grad_weight[e] = the sum over chunks of the partial tiles, in a fixed
// order: eight interleaved partial sums (chunks k, k + 8, ...), so that eight
// loads are in flight per thread, added pairwise at the end.
__global__ __launch_bounds__(256) void grad_weight_reduce_kernel(const GWArgs a) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  const int total = a.Co * a.NC;
  if (e >= total) return;
  const float* src = a.part + e;
  float s[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) s[i] = 0.0f;
  int k = 0;
  for (; k + 8 <= a.nchunks; k += 8) {
#pragma unroll
    for (int i = 0; i < 8; ++i) s[i] += src[(size_t)(k + i) * total];
  }
  for (int i = 0; k < a.nchunks; ++k, ++i) s[i] += src[(size_t)k * total];
  a.dw[e] = ((s[0] + s[1]) + (s[2] + s[3])) + ((s[4] + s[5]) + (s[6] + s[7]));
}

// ---------------------------------------------------------------------------
// Host side: plan, workspace size, replay.

constexpr int64_t kI31 = int64_t(1) << 31;

// Plan of a shape for `cus` compute units; CONV2D_OK or an error code.
int gw_plan(const conv2d_params* p, int cus, GWArgs* a) {
  int rc = validate_shape(p);
  if (rc != CONV2D_OK) return rc;
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
  // whole-tensor byte offsets (chunks cross images) and fast_div bounds
  if (P >= kI31 || int64_t(p->batch) * p->out_channels * OHOW * 4 >= kI31 ||
      int64_t(p->batch) * p->in_channels * p->in_h * p->in_w * 4 >= kI31 ||
      NC * KHW >= kI31 || (NC + kTile) * KHW >= kI31)
    return CONV2D_ERR_OVERFLOW;
  a->NC = int32_t(NC);
  a->OHOW = int32_t(OHOW);
  a->P = int32_t(P);
  a->m_KHW = fast_div_magic(uint32_t(std::max<int64_t>(KHW, 1)));
  a->m_KW = fast_div_magic(uint32_t(std::max<int32_t>(a->KW, 1)));
  a->TM = int32_t((int64_t(a->Co) + kTile - 1) / kTile);
  a->TN = int32_t((NC + kTile - 1) / kTile);
  if (cus < 1) cus = kDefaultCUs;
  if (P == 0 || a->TM == 0 || a->TN == 0) {
    a->chunk_px = kStagePx;
    a->nchunks = 0;   // no pixel: grad_weight is zeros (no tile, or no output)
    return CONV2D_OK;
  }
  const int64_t target = int64_t(kTargetGroupsPerCU) * cus;
  const int64_t tiles = int64_t(a->TM) * a->TN;
  int64_t chunk = (P * tiles + target - 1) / target;
  chunk = std::max<int64_t>(kStagePx, (chunk + kStagePx - 1) / kStagePx * kStagePx);
  a->chunk_px = int32_t(std::min<int64_t>(chunk, (P + kStagePx - 1) / kStagePx * kStagePx));
  a->nchunks = int32_t((P + a->chunk_px - 1) / a->chunk_px);
  if (tiles * a->nchunks >= kI31 || int64_t(a->nchunks) * a->Co * NC * 4 >= (int64_t(1) << 40))
    return CONV2D_ERR_OVERFLOW;
  return CONV2D_OK;
}

size_t gw_workspace_bytes(const GWArgs& a) {
  return size_t(a.nchunks) * size_t(a.Co) * size_t(a.NC) * sizeof(float);
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

// Host replay of every workgroup and thread: each copy reads the grad_out /
// x element of the definition (or 0 where the definition has no term), each
// LDS cell of a stage is written by exactly one thread, the products pair A
// and B cells of the same pixel and the lane's own row and column, and every
// (chunk, co, column) partial is stored exactly once.
int gw_check(const conv2d_params* p, char* msg, size_t len) {
  GWArgs a;
  int rc = gw_plan(p, kDefaultCUs, &a);
  if (rc != CONV2D_OK) return rc;
  try {
    const int64_t nparts = int64_t(a.nchunks) * a.Co * a.NC;
    std::vector<unsigned char> stored(size_t(nparts), 0);
    const int64_t go_size = int64_t(a.N) * a.Co * a.OHOW, x_size = int64_t(a.N) * a.Ci * a.H * a.W;
    for (int bid = 0; bid < a.TM * a.TN * a.nchunks; ++bid) {
      const GWTile T = gw_tile(a, bid);
      GW_REQUIRE(T.chunk >= 0 && T.chunk < a.nchunks && T.co0 < a.Co && T.c0 < a.NC && T.nst >= 1,
                 "bid %d tile", bid);
      // per stage: which pixel each LDS column holds, and which cells are written
      for (int st = 0; st < T.nst; ++st) {
        std::vector<unsigned char> cell(2 * kTile * kPitch, 0);
        for (int tid = 0; tid < kThreads; ++tid) {
          const int cpx = tid & (kStagePx - 1), r0 = tid / kStagePx;
          int n = 0, q = 0, oh = 0, ow = 0;
          const int pix = T.p_begin + st * kStagePx + cpx;
          const bool pin = gw_pixel(a, pix, T.p_end, &n, &q, &oh, &ow);
          GW_REQUIRE(!pin || (pix >= T.p_begin && pix < a.P), "pixel %d", pix);
          for (int j = 0; j < kRowsPerThread; ++j) {
            const int row = r0 + 4 * j;
            GW_REQUIRE(row < kTile, "row %d", row);
            for (int op = 0; op < 2; ++op) {
              const int idx = op * kTile * kPitch + row * kPitch + cpx;
              GW_REQUIRE(cell[size_t(idx)] == 0, "stage %d cell written twice", st);
              cell[size_t(idx)] = 1;
            }
            // A: grad_out[n, co, oh, ow] or 0
            const int co = T.co0 + row;
            const uint32_t ao = gw_a_offset(a, pin, n, q, co);
            if (pin && co < a.Co) {
              GW_REQUIRE(ao == uint32_t(((int64_t(n) * a.Co + co) * a.OHOW +
                                         int64_t(oh) * a.OW + ow) * 4) &&
                             int64_t(ao / 4) < go_size,
                         "A element of co %d pixel %d", co, pix);
            } else {
              GW_REQUIRE(ao == kPad, "A padding");
            }
            // B: x[n, ci, s*oh - ph + kh, s*ow - pw + kw] or 0, against the
            // column's (ci, kh, kw) taken from the weight layout
            const int c = T.c0 + row;
            int xcol, khw;
            gw_column(a, c, &xcol, &khw);
            const uint32_t bo = gw_b_offset(a, pin, n, oh, ow, xcol, khw);
            bool term = false;
            int64_t want = 0;
            if (pin && c < a.NC) {
              const int KHW = a.KH * a.KW, ci = c / KHW, kh = (c % KHW) / a.KW, kw = c % a.KW;
              const int ih = oh * a.S - a.PH + kh, iw = ow * a.S - a.PW + kw;
              term = ih >= 0 && ih < a.H && iw >= 0 && iw < a.W;
              want = ((int64_t(n) * a.Ci + ci) * a.H + ih) * a.W + iw;
            }
            if (term) {
              GW_REQUIRE(bo == uint32_t(want * 4) && want < x_size, "B element of column %d pixel %d",
                         c, pix);
            } else {
              GW_REQUIRE(bo == kPad, "B padding of column %d pixel %d", c, pix);
            }
          }
        }
        for (int op = 0; op < 2; ++op)
          for (int row = 0; row < kTile; ++row)
            for (int px = 0; px < kStagePx; ++px)
              GW_REQUIRE(cell[size_t(op * kTile * kPitch + row * kPitch + px)] == 1,
                         "stage %d cell never written", st);
      }
      // products: each lane's A reads are its row, its B reads its column,
      // and both at the same pixel; then its stores
      for (int tid = 0; tid < kThreads; ++tid) {
        const int lane = tid & 63, wave = tid >> 6, wm = wave & 1, wn = wave >> 1;
        const int g = lane >> 4, c16 = lane & 15;
        for (int u = 0; u < kStagePx / 16; ++u)
          for (int m = 0; m < 2; ++m)
            for (int b = 0; b < 2; ++b) {
              const int arow = wm * kWaveRows + m * 16 + c16, brow = wn * kWaveRows + b * 16 + c16;
              const int px0 = 16 * u + 4 * g;
              GW_REQUIRE(arow < kTile && brow < kTile && px0 + 4 <= kStagePx &&
                             (arow * kPitch + px0) % 4 == 0 && (brow * kPitch + px0) % 4 == 0,
                         "operand read");
            }
        for (int m = 0; m < 2; ++m)
          for (int b = 0; b < 2; ++b) {
            const int c = T.c0 + wn * kWaveRows + b * 16 + c16;
            for (int r = 0; r < 4; ++r) {
              const int co = T.co0 + wm * kWaveRows + m * 16 + 4 * g + r;
              if (co >= a.Co || c >= a.NC) continue;
              const int64_t e = (int64_t(T.chunk) * a.Co + co) * a.NC + c;
              GW_REQUIRE(e >= 0 && e < nparts && stored[size_t(e)] == 0, "partial stored twice");
              stored[size_t(e)] = 1;
            }
          }
      }
    }
    for (int64_t e = 0; e < nparts; ++e) GW_REQUIRE(stored[size_t(e)] == 1, "partial never stored");
    // the chunks cover every pixel once
    GW_REQUIRE(a.nchunks == 0 || (int64_t(a.nchunks - 1) * a.chunk_px < a.P &&
                                  int64_t(a.nchunks) * a.chunk_px >= a.P && a.chunk_px % kStagePx == 0),
               "chunks do not cover the pixels");
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

// Pointer checks: inputs go, x; outputs dw and the workspace, which may not
// overlap each other or an input.
int gw_check_pointers(const float* go, const float* x, const float* dw, const void* ws,
                      size_t ws_bytes, const conv2d_params* p, const GWArgs& a) {
  const uint64_t n_go = uint64_t(p->batch) * p->out_channels * p->out_h * p->out_w;
  const uint64_t n_x = uint64_t(p->batch) * p->in_channels * p->in_h * p->in_w;
  const uint64_t n_dw = uint64_t(p->out_channels) * p->in_channels * p->kernel_h * p->kernel_w;
  const uint64_t ws_need = gw_workspace_bytes(a);
  if ((n_go && go == nullptr) || (n_x && x == nullptr) || (n_dw && dw == nullptr))
    return CONV2D_ERR_NULL_PTR;
  if (ws_need && (ws == nullptr || ws_bytes < ws_need)) return CONV2D_ERR_WORKSPACE;
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

}  // namespace gw
}  // namespace c2b

extern "C" int conv2d_grad_weight_workspace_size(const conv2d_params* p, size_t* bytes) {
  if (p == nullptr || bytes == nullptr) return CONV2D_ERR_NULL_PTR;
  c2b::gw::GWArgs a;
  const int rc = c2b::gw::gw_plan(p, c2b::gw::device_cus_gw(), &a);
  if (rc != CONV2D_OK) return rc;
  *bytes = c2b::gw::gw_workspace_bytes(a);
  return CONV2D_OK;
}

extern "C" int conv2d_grad_weight(const float* grad_out, const float* x, float* grad_weight,
                                  const conv2d_params* p, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  using namespace c2b::gw;
  if (p == nullptr) return CONV2D_ERR_NULL_PTR;
  GWArgs a;
  int rc = gw_plan(p, device_cus_gw(), &a);
  if (rc != CONV2D_OK) return rc;
  rc = gw_check_pointers(grad_out, x, grad_weight, workspace, workspace_bytes, p, a);
  if (rc != CONV2D_OK) return rc;
  const int total = a.Co * a.NC;
  if (total == 0) return CONV2D_OK;
  a.go = grad_out;
  a.x = x;
  a.dw = grad_weight;
  a.part = static_cast<float*>(workspace);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (a.nchunks > 0)
    hipLaunchKernelGGL(grad_weight_mm_kernel, dim3(a.TM * a.TN * a.nchunks), dim3(kThreads), 0,
                       st, a);
  hipLaunchKernelGGL(grad_weight_reduce_kernel, dim3((total + 255) / 256), dim3(256), 0, st, a);
  return hipGetLastError() == hipSuccess ? CONV2D_OK : CONV2D_ERR_HIP;
}

extern "C" int conv2d_check_indexing_grad_weight(const conv2d_params* p, char* msg,
                                                 size_t msg_len) {
  return c2b::gw::gw_check(p, msg, msg_len);
}
