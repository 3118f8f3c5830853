// Forward convolution for few input channels as an im2col GEMM on CDNA4
// (gfx950) matrix cores, and its host replay.
//
// The forward cross-correlation (the map of the stride > 1 im2col branch of
// meganeura 0.2.0, conv2d_grad_input_gemm_coop.wgsl, read forwards):
//   y[n, co, oh, ow] = sum over c = (ci, kh, kw) of
//       w[co, c] * x[n, ci, s*oh - padding_h + kh, s*ow - padding_w + kw]
// (x zero outside the image) is a GEMM with M = Co rows, N = N*OH*OW pixels
// and K = Ci*kH*kW, contracted over the weight layout's own columns c.  The
// input-gradient kernel family contracts over 16-channel groups, so with 3
// input channels 13 of 16 products are zero; here the contraction index is
// (ci, kh, kw) itself and nothing is padded but the last stage.
//
// How (fp32): a workgroup (four waves as 2 x 2, each 32 x 32 of
// v_mfma_f32_16x16x4_f32) takes 64 output channels x 64 pixels; a stage is
// 32 columns c.  W rows and im2col columns go to LDS through registers as
// [row][c], rows 36 floats apart (16-byte reads of 16 rows hit distinct
// banks).  A copy thread owns one im2col column (pixel) or weight row for
// the whole tile and 8 consecutive c of it per stage; the c's (ci, kh, kw)
// are wave-uniform.  Elements the definition lacks read 0 (offset past the
// buffer range); pixels past the last and rows past Co load clamped real
// ones, whose products are never stored.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "plan.hpp"
#include "tile_index.hpp"

namespace c2b {
namespace fg {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kTile = 64;        // output channels and pixels of a tile
constexpr int kStageK = 32;      // contraction columns per stage
constexpr int kPitch = kStageK + 4;
constexpr int kThreads = 256;
constexpr uint32_t kPad = 0x80000000u;
constexpr int64_t kI31 = int64_t(1) << 31;
constexpr int kMaxChannels = 16;   // the path takes Ci below this

struct FGArgs {
  const float* x;
  const float* w;
  float* y;
  int32_t N, Ci, H, W, Co, KH, KW, S, PH, PW, OH, OW;
  int32_t KHW, NC, OHOW, P;
  int32_t TM, TP;   // channel tiles, pixel tiles
};

// Tile of workgroup bid: pixel tiles fastest (consecutive workgroups share
// the weight rows and neighbouring x rows).
C2B_HD void fg_tile(const FGArgs& a, int bid, int* tm, int* tp) {
  *tp = bid % a.TP;
  *tm = bid / a.TP;
}

// Copy roles: thread tid copies row tid % 64 (a weight row for A, a pixel for
// B) and contraction columns 8 (tid / 64) .. +7 of each stage.
C2B_HD int fg_row(int tid) { return tid % 64; }
C2B_HD int fg_col8(int tid) { return 8 * (tid / 64); }

// Byte offset of w[co][c] (co clamped to a real row), kPad for c >= NC.
C2B_HD uint32_t fg_w_offset(const FGArgs& a, int co, int c) {
  return c < a.NC ? (uint32_t(imin(co, a.Co - 1)) * uint32_t(a.NC) + uint32_t(c)) * 4u : kPad;
}

// Pixel p (clamped to a real one) -> image and the x offset of its window
// origin (kh = kw = 0), and its (s*oh - ph, s*ow - pw).
struct FGPixel {
  int n, q, ih0, iw0;
};
C2B_HD FGPixel fg_pixel(const FGArgs& a, int p) {
  p = imin(p, a.P - 1);
  FGPixel x;
  x.n = p / a.OHOW;
  x.q = p - x.n * a.OHOW;
  const int oh = x.q / a.OW, ow = x.q - oh * a.OW;
  x.ih0 = oh * a.S - a.PH;
  x.iw0 = ow * a.S - a.PW;
  return x;
}

// Byte offset of the im2col element (c, pixel): x[n, ci, ih0 + kh, iw0 + kw]
// or kPad where the definition has no term (or c >= NC).
C2B_HD uint32_t fg_x_offset(const FGArgs& a, const FGPixel& px, int c) {
  const int ci = c / a.KHW, r = c - ci * a.KHW, kh = r / a.KW, kw = r - kh * a.KW;
  const int ih = px.ih0 + kh, iw = px.iw0 + kw;
  const bool term = (c < a.NC) & ((unsigned)ih < (unsigned)a.H) & ((unsigned)iw < (unsigned)a.W);
  const uint32_t off =
      ((uint32_t(px.n) * uint32_t(a.Ci) + uint32_t(ci)) * uint32_t(a.H * a.W) +
       uint32_t(ih * a.W + iw)) * 4u;
  return term ? off : kPad;
}

__device__ __forceinline__ float load_f32(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
}

__global__ __launch_bounds__(kThreads, 4) void forward_gemm_kernel(const FGArgs a) {
  __shared__ f32x4 lds4[2 * 2 * kTile * kPitch / 4];   // [buffer][A, B][row][c]
  auto lds = [&](int buf, int op) __attribute__((always_inline)) {
    return reinterpret_cast<float*>(lds4) + (buf * 2 + op) * kTile * kPitch;
  };
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int g = lane >> 4, c16 = lane & 15;
  int tm, tp;
  fg_tile(a, blockIdx.x, &tm, &tp);
  const int co0 = tm * kTile, p0 = tp * kTile;
  const int nst = (a.NC + kStageK - 1) / kStageK;

  const __amdgpu_buffer_rsrc_t rsW = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(a.w), 0, a.Co * a.NC * 4, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsX = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(a.x), 0, a.N * a.Ci * a.H * a.W * 4, 0x00020000);
  const int row = fg_row(tid), c8 = __builtin_amdgcn_readfirstlane(fg_col8(tid));
  const FGPixel px = fg_pixel(a, p0 + row);

  float sa[8], sb[8];
  auto load_stage = [&](int st) __attribute__((always_inline)) {
    uint32_t oa[8], ob[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int c = st * kStageK + c8 + e;
      oa[e] = fg_w_offset(a, co0 + row, c);
      ob[e] = fg_x_offset(a, px, c);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      sa[e] = load_f32(rsW, oa[e]);
      sb[e] = load_f32(rsX, ob[e]);
    }
  };
  auto write_stage = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      *reinterpret_cast<f32x4*>(lds(buf, 0) + row * kPitch + c8 + 4 * h) =
          f32x4{sa[4 * h], sa[4 * h + 1], sa[4 * h + 2], sa[4 * h + 3]};
      *reinterpret_cast<f32x4*>(lds(buf, 1) + row * kPitch + c8 + 4 * h) =
          f32x4{sb[4 * h], sb[4 * h + 1], sb[4 * h + 2], sb[4 * h + 3]};
    }
  };

  f32x4 acc[2][2];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[m][b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  auto compute = [&](int st) __attribute__((always_inline)) {
    const float* As = lds(st & 1, 0);
    const float* Bs = lds(st & 1, 1);
#pragma unroll
    for (int u = 0; u < kStageK / 16; ++u) {
      f32x4 av[2], bv[2];
#pragma unroll
      for (int m = 0; m < 2; ++m)
        av[m] = *reinterpret_cast<const f32x4*>(As + (wm * 32 + m * 16 + c16) * kPitch +
                                                 16 * u + 4 * g);
#pragma unroll
      for (int b = 0; b < 2; ++b)
        bv[b] = *reinterpret_cast<const f32x4*>(Bs + (wn * 32 + b * 16 + c16) * kPitch +
                                                 16 * u + 4 * g);
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
  if (nst > 1) load_stage(1);
  __syncthreads();
  for (int st = 0; st < nst; ++st) {
    compute(st);
    if (st + 1 < nst) write_stage((st + 1) & 1);
    if (st + 2 < nst) load_stage(st + 2);
    __syncthreads();
  }

  // register r of block (m, b): channel co0 + wm*32 + m*16 + 4g + r, pixel
  // p0 + wn*32 + b*16 + c16
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int p = p0 + wn * 32 + b * 16 + c16;
    if (p >= a.P) continue;
    const int n = p / a.OHOW, q = p - n * a.OHOW;
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int co = co0 + wm * 32 + m * 16 + 4 * g + r;
        if (co < a.Co) a.y[(size_t(n) * a.Co + co) * a.OHOW + q] = acc[m][b][r];
      }
  }
}

// ---------------------------------------------------------------------------
// Host side.

int fg_plan(const conv2d_params* p, FGArgs* a);

// fp32 shapes with 1 to 15 input channels whose tensors fit this kernel's
// whole-tensor 32-bit offsets (fg_plan); every other shape, including
// larger batches of the same layer, goes to the implicit-GEMM family, which
// offsets per image.
bool fg_applies(const conv2d_params* p, int f16) {
  if (p == nullptr || f16 || p->in_channels < 1 || p->in_channels >= uint32_t(kMaxChannels))
    return false;
  FGArgs a;
  return fg_plan(p, &a) == CONV2D_OK;
}

int fg_plan(const conv2d_params* p, FGArgs* a) {
  const int rc = validate_shape(p);
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
  const int64_t KHW = int64_t(a->KH) * a->KW, NC = int64_t(a->Ci) * KHW;
  const int64_t OHOW = int64_t(a->OH) * a->OW, P = int64_t(a->N) * OHOW;
  if (P >= kI31 || int64_t(a->N) * a->Ci * a->H * a->W * 4 >= kI31 ||
      int64_t(a->Co) * NC * 4 >= kI31 || NC + kStageK >= kI31 ||
      int64_t(a->N) * a->Co * OHOW >= kI31)
    return CONV2D_ERR_OVERFLOW;
  a->KHW = int32_t(KHW);
  a->NC = int32_t(NC);
  a->OHOW = int32_t(OHOW);
  a->P = int32_t(P);
  a->TM = int32_t((a->Co + kTile - 1) / kTile);
  a->TP = int32_t((P + kTile - 1) / kTile);
  if (int64_t(a->TM) * a->TP >= kI31) return CONV2D_ERR_OVERFLOW;
  return CONV2D_OK;
}

namespace {
struct Failure {
  std::string msg;
};
#define FG_REQUIRE(cond, ...)                                   \
  do {                                                          \
    if (!(cond)) {                                              \
      char buf_[512];                                           \
      std::snprintf(buf_, sizeof buf_, __VA_ARGS__);            \
      throw Failure{std::string(#cond) + ": " + buf_};          \
    }                                                           \
  } while (0)
}  // namespace

// Host replay: every tile once; per stage every LDS cell written once, each
// stored row / pixel's element the definition's (0 where it has no term or
// past NC); every output element stored once.
int fg_check(const conv2d_params* p, char* msg, size_t len) {
  FGArgs a;
  const int rc = fg_plan(p, &a);
  if (rc != CONV2D_OK) return rc;
  try {
    const int64_t w_bytes = int64_t(a.Co) * a.NC * 4, x_bytes = int64_t(a.N) * a.Ci * a.H * a.W * 4;
    const int nst = (a.NC + kStageK - 1) / kStageK;
    std::vector<unsigned char> stored(size_t(int64_t(a.N) * a.Co * a.OHOW), 0);
    for (int bid = 0; bid < a.TM * a.TP; ++bid) {
      int tm, tp;
      fg_tile(a, bid, &tm, &tp);
      FG_REQUIRE(tm < a.TM && tp < a.TP, "tile of %d", bid);
      const int co0 = tm * kTile, p0 = tp * kTile;
      for (int st = 0; st < nst; ++st) {
        std::vector<unsigned char> cell(2 * kTile * kStageK, 0);
        for (int tid = 0; tid < kThreads; ++tid) {
          const int row = fg_row(tid), c8 = fg_col8(tid);
          FG_REQUIRE(tid / 64 == (tid & ~63) / 64, "uniform columns");
          const FGPixel px = fg_pixel(a, p0 + row);
          for (int e = 0; e < 8; ++e) {
            const int lc = c8 + e, c = st * kStageK + lc;
            FG_REQUIRE(lc < kStageK, "column");
            for (int op = 0; op < 2; ++op) {
              unsigned char& cv = cell[size_t(op * kTile * kStageK + row * kStageK + lc)];
              FG_REQUIRE(cv == 0, "cell written twice");
              cv = 1;
            }
            const uint32_t ow = fg_w_offset(a, co0 + row, c);
            if (co0 + row < a.Co) {
              FG_REQUIRE(c < a.NC ? int64_t(ow) == (int64_t(co0 + row) * a.NC + c) * 4
                                  : int64_t(ow) >= w_bytes,
                         "w element (%d, %d)", co0 + row, c);
            }
            const int pix = p0 + row;
            if (pix < a.P && c < a.NC) {
              const int n = pix / a.OHOW, q = pix % a.OHOW, oh = q / a.OW, ow_ = q % a.OW;
              const int ci = c / a.KHW, kh = (c % a.KHW) / a.KW, kw = c % a.KW;
              const int ih = oh * a.S - a.PH + kh, iw = ow_ * a.S - a.PW + kw;
              const uint32_t ox = fg_x_offset(a, px, c);
              if (ih >= 0 && ih < a.H && iw >= 0 && iw < a.W)
                FG_REQUIRE(int64_t(ox) == (((int64_t(n) * a.Ci + ci) * a.H + ih) * a.W + iw) * 4,
                           "x element of pixel %d column %d", pix, c);
              else
                FG_REQUIRE(int64_t(ox) >= x_bytes, "x padding of pixel %d column %d", pix, c);
            } else if (c >= a.NC) {
              FG_REQUIRE(int64_t(fg_x_offset(a, px, c)) >= x_bytes, "x past NC");
            }
          }
        }
        for (size_t i = 0; i < cell.size(); ++i) FG_REQUIRE(cell[i] == 1, "cell never written");
      }
      for (int tid = 0; tid < kThreads; ++tid) {
        const int lane = tid & 63, wave = tid >> 6, wm = wave & 1, wn = wave >> 1;
        const int g = lane >> 4, c16 = lane & 15;
        for (int b = 0; b < 2; ++b) {
          const int pp = p0 + wn * 32 + b * 16 + c16;
          if (pp >= a.P) continue;
          for (int m = 0; m < 2; ++m)
            for (int r = 0; r < 4; ++r) {
              const int co = co0 + wm * 32 + m * 16 + 4 * g + r;
              if (co >= a.Co) continue;
              const size_t e = size_t((int64_t(pp / a.OHOW) * a.Co + co) * a.OHOW + pp % a.OHOW);
              FG_REQUIRE(stored[e] == 0, "output stored twice");
              stored[e] = 1;
            }
        }
      }
    }
    for (size_t e = 0; e < stored.size(); ++e) FG_REQUIRE(stored[e] == 1, "output never stored");
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

// The forward convolution on this path (pointers already checked).
int fg_launch(const float* x, const float* w, float* y, const conv2d_params* p, void* stream) {
  FGArgs a;
  const int rc = fg_plan(p, &a);
  if (rc != CONV2D_OK) return rc;
  if (int64_t(a.N) * a.Co * a.OHOW == 0) return CONV2D_OK;
  a.x = x;
  a.w = w;
  a.y = y;
  hipLaunchKernelGGL(forward_gemm_kernel, dim3(a.TM * a.TP), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), a);
  return hipGetLastError() == hipSuccess ? CONV2D_OK : CONV2D_ERR_HIP;
}

}  // namespace fg
}  // namespace c2b
