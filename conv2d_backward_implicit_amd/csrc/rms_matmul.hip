// RMSNorm-fused matrix product C = RmsNorm(X, g) x W on CDNA4 (gfx950)
// matrix cores, its host replay, and its C-ABI entry points.
//
// What is computed (meganeura 0.2.0, src/shaders/matmul_rms_norm.wgsl: the
// header comment, the per-row rsqrt prologue and the normalise-on-load A
// staging):
//   r[i] = 1 / sqrt(sum_k x[i, k]^2 / K + eps),
//   C[i, j] = sum_k x[i, k] * r[i] * g[k] * W[k, j].
// The page makes a separate pass over each X row for r[i], then stages
// x * r * g.  Here one pass does both: while X tiles are staged the row sums
// of squares are accumulated from the same registers, g is applied on the
// way to LDS, and r[i] multiplies the finished row in the epilogue (r[i]
// is a per-row factor of the sum, so the result is the same up to fp32
// rounding order).
//
// How (fp32):
//  * One workgroup (256 threads, four waves as 2 x 2) per 128 x 128 output
//    tile; each wave 64 x 64 as 4 x 4 blocks of v_mfma_f32_16x16x4_f32.
//    Tiles are dealt to the 8 XCDs in contiguous runs, column tiles fastest,
//    so the tiles of one row block share an L2.
//  * A stage is 32 columns of K.  X rows and W^T rows go to LDS through
//    registers as [row][k] with rows 36 floats apart: the 16-byte reads of
//    16 lanes (16 rows, one k quad) then hit distinct banks.  X: a thread
//    loads 4 consecutive k of 4 rows (8 lanes per row, coalesced along k)
//    and writes x * g as one 16-byte LDS store per row.  W: a thread loads
//    4 consecutive k rows of one column (64 lanes along n, coalesced) and
//    writes them transposed as one 16-byte store.  Columns k >= K read 0
//    (offset past the buffer range); rows past M and columns past N load a
//    clamped real row or column, whose products are never stored.
//  * Two stage buffers, one barrier per stage: stage s+1 is written after the
//    products of stage s, stage s+2 is loaded then.
//  * Products: lane group q4 of a 16-lane block reads k = 16u + 4q4 .. +3 of
//    its row (A) and of its column (B) with one 16-byte read each; MFMA q
//    takes k = 16u + 4q4 + q from every group.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "rms_norm_matmul.h"

#if defined(__HIPCC__)
#define RMM_HD __host__ __device__ __forceinline__
#else
#define RMM_HD inline
#endif

namespace rmm {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kBM = 128, kBN = 128;         // output tile
constexpr int kBK = 32;                     // k per stage
constexpr int kPitch = kBK + 4;             // floats between LDS rows
constexpr int kThreads = 256;
constexpr int kWave = 64;                   // each wave: 64 x 64 (4 x 4 blocks)
constexpr int kARows = 4;                   // X rows per copy thread (32 apart)
constexpr int kBQuads = 4;                  // W k-quads per copy thread (2 apart)
constexpr uint32_t kPad = 0x80000000u;      // byte offset past every buffer range
constexpr int64_t kI31 = int64_t(1) << 31;

RMM_HD int imin(int a, int b) { return a < b ? a : b; }

struct Args {
  const float* x;
  const float* g;
  const float* w;
  float* out;
  int32_t M, N, K;
  float eps;
  int32_t TM, TN;   // row and column tiles
};

// Tile of workgroup bid: each XCD (workgroups x, x + 8, ...) takes one
// contiguous run of tiles, ordered in groups of kGroupRows row blocks (row
// blocks fastest within a group) so that the tiles resident at once share
// both their X rows and their W columns in L2.
constexpr int kGroupRows = 8;

RMM_HD void tile_of(const Args& a, int bid, int* tm, int* tn) {
  const int T = a.TM * a.TN;
  const int q = T >> 3, r = T & 7, x = bid & 7, k = bid >> 3;
  const int t = x * q + imin(x, r) + k;
  const int grp = t / (kGroupRows * a.TN), first = grp * kGroupRows;
  const int gm = imin(kGroupRows, a.TM - first), within = t - grp * kGroupRows * a.TN;
  *tm = first + within % gm;
  *tn = within / gm;
}

// Copy thread roles.  X: k quad kq = tid % 8 of rows tid / 8 + 32 p.
// W: column tid % 128, k quads tid / 128 + 2 p.
RMM_HD int a_row(int tid, int p) { return tid / 8 + 32 * p; }
RMM_HD int a_kq(int tid) { return tid % 8; }
RMM_HD int b_col(int tid) { return tid % 128; }
RMM_HD int b_kq(int tid, int p) { return tid / 128 + 2 * p; }

// Byte offset of x[row][k] (row clamped to a real one), kPad for k >= K.
RMM_HD uint32_t x_offset(const Args& a, int row, int k) {
  const uint32_t off = (uint32_t(imin(row, a.M - 1)) * uint32_t(a.K) + uint32_t(k)) * 4u;
  return k < a.K ? off : kPad;
}
// Byte offset of w[k][col] (col clamped to a real one), kPad for k >= K.
RMM_HD uint32_t w_offset(const Args& a, int k, int col) {
  const uint32_t off = (uint32_t(k) * uint32_t(a.N) + uint32_t(imin(col, a.N - 1))) * 4u;
  return k < a.K ? off : kPad;
}

__device__ __forceinline__ float load_f32(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
}

__global__ __launch_bounds__(kThreads, 2) void rms_matmul_kernel(const Args a) {
  // [stage buffer][A, B][row * kPitch + k], 16-byte aligned
  __shared__ f32x4 lds4[2 * 2 * kBM * kPitch / 4];
  __shared__ float rs_row[kBM];   // r[i] of the tile's rows
  auto lds = [&](int buf, int op) __attribute__((always_inline)) {
    return reinterpret_cast<float*>(lds4) + (buf * 2 + op) * kBM * kPitch;
  };
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int q4 = lane >> 4, c16 = lane & 15;
  int tm, tn;
  tile_of(a, blockIdx.x, &tm, &tn);
  const int row0 = tm * kBM, col0 = tn * kBN;
  const int nst = (a.K + kBK - 1) / kBK;

  const __amdgpu_buffer_rsrc_t rsX = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(a.x), 0, a.M * a.K * 4, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsW = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(a.w), 0, a.K * a.N * 4, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsG = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(a.g), 0, a.K * 4, 0x00020000);

  const int akq = a_kq(tid), bcol = b_col(tid);
  float xs[kARows][4], ws[kBQuads][4], gs[4];
  float ss[kARows] = {0.0f, 0.0f, 0.0f, 0.0f};   // row sums of squares
  auto load_stage = [&](int st) __attribute__((always_inline)) {
    const int k0 = st * kBK;
    uint32_t ox[kARows][4], ow[kBQuads][4], og[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int k = k0 + 4 * akq + q;
      og[q] = k < a.K ? uint32_t(k) * 4u : kPad;
#pragma unroll
      for (int p = 0; p < kARows; ++p) ox[p][q] = x_offset(a, row0 + a_row(tid, p), k);
    }
#pragma unroll
    for (int p = 0; p < kBQuads; ++p)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        ow[p][q] = w_offset(a, k0 + 4 * b_kq(tid, p) + q, col0 + bcol);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < 4; ++q) gs[q] = load_f32(rsG, og[q]);
#pragma unroll
    for (int p = 0; p < kARows; ++p)
#pragma unroll
      for (int q = 0; q < 4; ++q) xs[p][q] = load_f32(rsX, ox[p][q]);
#pragma unroll
    for (int p = 0; p < kBQuads; ++p)
#pragma unroll
      for (int q = 0; q < 4; ++q) ws[p][q] = load_f32(rsW, ow[p][q]);
  };
  auto write_stage = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int p = 0; p < kARows; ++p) {
      f32x4 v;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        ss[p] += xs[p][q] * xs[p][q];
        v[q] = xs[p][q] * gs[q];
      }
      *reinterpret_cast<f32x4*>(lds(buf, 0) + a_row(tid, p) * kPitch + 4 * akq) = v;
    }
#pragma unroll
    for (int p = 0; p < kBQuads; ++p) {
      const f32x4 v = {ws[p][0], ws[p][1], ws[p][2], ws[p][3]};
      *reinterpret_cast<f32x4*>(lds(buf, 1) + bcol * kPitch + 4 * b_kq(tid, p)) = v;
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[m][b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  auto compute = [&](int st) __attribute__((always_inline)) {
    const float* As = lds(st & 1, 0);
    const float* Bs = lds(st & 1, 1);
#pragma unroll
    for (int u = 0; u < kBK / 16; ++u) {
      f32x4 av[4], bv[4];
#pragma unroll
      for (int m = 0; m < 4; ++m)
        av[m] = *reinterpret_cast<const f32x4*>(
            As + (wm * kWave + m * 16 + c16) * kPitch + 16 * u + 4 * q4);
#pragma unroll
      for (int b = 0; b < 4; ++b)
        bv[b] = *reinterpret_cast<const f32x4*>(
            Bs + (wn * kWave + b * 16 + c16) * kPitch + 16 * u + 4 * q4);
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
          for (int b = 0; b < 4; ++b)
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

  // r[i]: the 8 lanes of a row (tid % 8) add their partial sums
#pragma unroll
  for (int p = 0; p < kARows; ++p) {
    float v = ss[p];
    v += __shfl_xor(v, 1);
    v += __shfl_xor(v, 2);
    v += __shfl_xor(v, 4);
    if (akq == 0) rs_row[a_row(tid, p)] = 1.0f / sqrtf(v / float(a.K) + a.eps);
  }
  __syncthreads();

  // register r of block (m, b): row wm*64 + m*16 + 4*q4 + r, column
  // wn*64 + b*16 + c16
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int lr = wm * kWave + m * 16 + 4 * q4 + r;
      const int row = row0 + lr;
      if (row >= a.M) continue;
      const float f = rs_row[lr];
      float* orow = a.out + size_t(row) * a.N;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int col = col0 + wn * kWave + b * 16 + c16;
        if (col < a.N) orow[col] = acc[m][b][r] * f;
      }
    }
}


// ---------------------------------------------------------------------------
// Direct-to-LDS variant (K and N multiples of 4, 16-byte aligned pointers).
//
// The stage's X tile, W tile and g slice go from memory straight to LDS
// with buffer loads in their LDS form (lane i of a 16-byte load lands at
// M0 + 16 i, of a 4-byte load at M0 + 4 i): no registers or LDS writes on
// the way, so a stage's copies are a handful of instructions issued one
// stage ahead.  LDS layouts (per stage buffer):
//   A: [row][k] 128 x 32, k quad kq of row r at slot kq ^ ((r >> 1) & 7):
//      16 lanes reading 16 rows at one quad hit 16 distinct 4-bank groups;
//   B: [k][n] 32 x 128 as in memory: 16 lanes reading 16 consecutive n quads
//      at one k are conflict-free;
//   G: g[k0 .. k0 + 63] (32 used).
// Products: for k step t of a 16-k unit u, lane group q4 supplies
// k = 16u + 4 q4 + t; A: lane (row c16, q4) reads its row's quad (16-byte);
// B: lane (c16, q4) reads n = 4 c16 .. +3 at k (16-byte), one value for
// each of four MFMAs q, so MFMA q of a block covers columns 4 c16 + q.  The
// row sums of squares are taken from the raw A reads; g multiplies them.

constexpr int kDmaStageBytes = (kBM * kBK + kBK * kBN + 64) * 4;   // A, B, G

RMM_HD int dma_a_slot(int row, int kq) { return kq ^ ((row >> 1) & 7); }

// 16-byte load j (of 16 per stage) of the A tile, lane l: tile row and k quad.
RMM_HD void dma_a_src(int j, int l, int* row, int* kq) {
  *row = 8 * j + l / 8;
  *kq = dma_a_slot(*row, l % 8);   // the slot is its own inverse
}
// 16-byte load j (of 16) of the B tile, lane l: k row and n quad.
RMM_HD void dma_b_src(int j, int l, int* krow, int* nq) {
  *krow = 2 * j + l / 32;
  *nq = l % 32;
}
RMM_HD uint32_t dma_x_offset(const Args& a, int row0, int k0, int row, int kq) {
  const int k = k0 + 4 * kq;
  const uint32_t off =
      (uint32_t(imin(row0 + row, a.M - 1)) * uint32_t(a.K) + uint32_t(k)) * 4u;
  return k < a.K ? off : kPad;
}
RMM_HD uint32_t dma_w_offset(const Args& a, int k0, int col0, int krow, int nq) {
  const int k = k0 + krow;
  const uint32_t off = (uint32_t(k) * uint32_t(a.N) + uint32_t(col0 + 4 * nq)) * 4u;
  return k < a.K ? off : kPad;
}

typedef __attribute__((address_space(3))) void lds_void_t;

__global__ __launch_bounds__(kThreads, 2) void rms_matmul_dma_kernel(const Args a) {
  __shared__ f32x4 lds4[2 * kDmaStageBytes / 16];
  __shared__ float rs_row[kBM];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int q4 = lane >> 4, c16 = lane & 15;
  int tm, tn;
  tile_of(a, blockIdx.x, &tm, &tn);
  const int row0 = tm * kBM, col0 = tn * kBN;
  const int nst = (a.K + kBK - 1) / kBK;
  auto buf = [&](int b) __attribute__((always_inline)) {
    return reinterpret_cast<char*>(lds4) + b * kDmaStageBytes;
  };

  __amdgpu_buffer_rsrc_t rsX = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(a.x), 0, a.M * a.K * 4, 0x00020000);
  __amdgpu_buffer_rsrc_t rsW = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(a.w), 0, a.K * a.N * 4, 0x00020000);
  __amdgpu_buffer_rsrc_t rsG = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(a.g), 0, a.K * 4, 0x00020000);

  // this wave's loads: A and B loads 4 * wave .. 4 * wave + 3, and g (wave 0)
  auto issue = [&](int st) __attribute__((always_inline)) {
    const int k0 = st * kBK;
    char* base = buf(st & 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = 4 * wave + i;
      int row, kq, krow, nq;
      dma_a_src(j, lane, &row, &kq);
      dma_b_src(j, lane, &krow, &nq);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsX, (lds_void_t*)(base + j * 1024), 16, dma_x_offset(a, row0, k0, row, kq), 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsW, (lds_void_t*)(base + kBM * kBK * 4 + j * 1024), 16,
          dma_w_offset(a, k0, col0, krow, nq), 0, 0, 0);
    }
    if (wave == 0) {
      const int k = k0 + lane;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsG, (lds_void_t*)(base + (kBM * kBK + kBK * kBN) * 4), 4,
          k < a.K ? uint32_t(k) * 4u : kPad, 0, 0, 0);
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[m][q] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  float ss[4] = {0.0f, 0.0f, 0.0f, 0.0f};

  auto compute = [&](int st) __attribute__((always_inline)) {
    const char* base = buf(st & 1);
    const float* As = reinterpret_cast<const float*>(base);
    const float* Bs = reinterpret_cast<const float*>(base + kBM * kBK * 4);
    const float* Gs = reinterpret_cast<const float*>(base + (kBM * kBK + kBK * kBN) * 4);
#pragma unroll
    for (int u = 0; u < kBK / 16; ++u) {
      f32x4 av[4], bv[4];
      const f32x4 gv = *reinterpret_cast<const f32x4*>(Gs + 16 * u + 4 * q4);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int row = wm * kWave + m * 16 + c16;
        av[m] = *reinterpret_cast<const f32x4*>(As + row * kBK +
                                                 4 * dma_a_slot(row, 4 * u + q4));
      }
#pragma unroll
      for (int t = 0; t < 4; ++t)
        bv[t] = *reinterpret_cast<const f32x4*>(Bs + (16 * u + 4 * q4 + t) * kBN +
                                                 wn * kWave + 4 * c16);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
#pragma unroll
        for (int t = 0; t < 4; ++t) ss[m] += av[m][t] * av[m][t];
        av[m] *= gv;
      }
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            acc[m][q] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[m][t], bv[t][q], acc[m][q], 0,
                                                             0, 0);
    }
  };

  issue(0);
  __builtin_amdgcn_s_waitcnt(0);   // this wave's loads into LDS are done
  __syncthreads();
  for (int st = 0; st < nst; ++st) {
    if (st + 1 < nst) issue(st + 1);
    compute(st);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // r[i]: lanes c16 + 16 q4 (q4 = 0..3) hold the four k quads of one row
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    float v = ss[m];
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    if (wn == 0 && q4 == 0)
      rs_row[wm * kWave + m * 16 + c16] = 1.0f / sqrtf(v / float(a.K) + a.eps);
  }
  __syncthreads();

  // register r of block (m, q): row wm*64 + m*16 + 4*q4 + r, column
  // wn*64 + 4*c16 + q: four consecutive columns per lane, one 16-byte store
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int lr = wm * kWave + m * 16 + 4 * q4 + r;
      const int row = row0 + lr, col = col0 + wn * kWave + 4 * c16;
      if (row >= a.M || col >= a.N) continue;
      const float f = rs_row[lr];
      const f32x4 v = {acc[m][0][r] * f, acc[m][1][r] * f, acc[m][2][r] * f, acc[m][3][r] * f};
      *reinterpret_cast<f32x4*>(a.out + size_t(row) * a.N + col) = v;
    }
}

// ---------------------------------------------------------------------------
// Host side.

int plan(const rms_matmul_params* p, Args* a) {
  if (p == nullptr) return CONV2D_ERR_NULL_PTR;
  if (p->k == 0 || !(p->eps >= 0.0f) || !std::isfinite(p->eps)) return CONV2D_ERR_BAD_SHAPE;
  const int64_t M = p->m, N = p->n, K = p->k;
  if (M * K * 4 >= kI31 || K * N * 4 >= kI31 || M * N * 4 >= kI31 || M >= kI31 || N >= kI31 ||
      K + kBK >= kI31)
    return CONV2D_ERR_OVERFLOW;
  std::memset(a, 0, sizeof(*a));
  a->M = int32_t(M);
  a->N = int32_t(N);
  a->K = int32_t(K);
  a->eps = p->eps;
  a->TM = int32_t((M + kBM - 1) / kBM);
  a->TN = int32_t((N + kBN - 1) / kBN);
  if (int64_t(a->TM) * a->TN >= kI31) return CONV2D_ERR_OVERFLOW;
  return CONV2D_OK;
}

namespace {
struct Failure {
  std::string msg;
};
#define RMM_REQUIRE(cond, ...)                                  \
  do {                                                          \
    if (!(cond)) {                                              \
      char buf_[512];                                           \
      std::snprintf(buf_, sizeof buf_, __VA_ARGS__);            \
      throw Failure{std::string(#cond) + ": " + buf_};          \
    }                                                           \
  } while (0)
}  // namespace

// The direct-to-LDS kernel runs where every 16-byte quad of x and W lies in
// one row (K and N multiples of 4); the entry point also needs 16-byte
// aligned x, W and out.
bool dma_eligible(const Args& a) { return a.K % 4 == 0 && a.N % 4 == 0; }

// Replay of the direct-to-LDS kernel: which x / W / g element every load
// lane puts in every LDS cell of a stage (each cell once), then that every
// product read finds the definition's element there (0 past K), that the
// row sums of squares take every k of a row once, and every output element
// is stored once.
void check_dma(const Args& a) {
  const int nst = (a.K + kBK - 1) / kBK;
  const int64_t x_bytes = int64_t(a.M) * a.K * 4, w_bytes = int64_t(a.K) * a.N * 4;
  const int nA = kBM * kBK, nB = kBK * kBN, nG = 64;
  std::vector<unsigned char> stored(size_t(int64_t(a.M) * a.N), 0);
  // 16 loads of 1 KiB fill A, 16 fill B
  RMM_REQUIRE(kDmaStageBytes == (nA + nB + nG) * 4 && 16 * 1024 == nA * 4 && 16 * 1024 == nB * 4,
              "stage layout");
  for (int bid = 0; bid < a.TM * a.TN; ++bid) {
    int tm, tn;
    tile_of(a, bid, &tm, &tn);
    const int row0 = tm * kBM, col0 = tn * kBN;
    std::vector<int> ss_hits(size_t(kBM) * a.K, 0);
    for (int st = 0; st < nst; ++st) {
      const int k0 = st * kBK;
      // source of every LDS float of the stage: byte offset / 4 into x, W or
      // g, -1 for a zero (offset past the range), -2 for never written
      std::vector<int64_t> src(size_t(nA + nB + nG), -2);
      auto put = [&](int dst, int64_t off, int64_t range, int width) {
        for (int e = 0; e < width; ++e) {
          RMM_REQUIRE(dst + e >= 0 && dst + e < nA + nB + nG, "LDS cell %d", dst + e);
          RMM_REQUIRE(src[size_t(dst + e)] == -2, "LDS cell %d written twice", dst + e);
          src[size_t(dst + e)] = off >= range ? -1 : off / 4 + e;
        }
      };
      for (int wave = 0; wave < 4; ++wave)
        for (int i = 0; i < 4; ++i) {
          const int j = 4 * wave + i;
          for (int l = 0; l < 64; ++l) {
            int row, kq, krow, nq;
            dma_a_src(j, l, &row, &kq);
            dma_b_src(j, l, &krow, &nq);
            RMM_REQUIRE(row < kBM && kq < kBK / 4 && krow < kBK && nq < kBN / 4, "load roles");
            put(j * 256 + 4 * l, dma_x_offset(a, row0, k0, row, kq), x_bytes, 4);
            put(nA + j * 256 + 4 * l, dma_w_offset(a, k0, col0, krow, nq), w_bytes, 4);
          }
        }
      for (int l = 0; l < 64; ++l) {
        const int k = k0 + l;
        put(nA + nB + l, k < a.K ? int64_t(k) * 4 : int64_t(kPad), int64_t(a.K) * 4, 1);
      }
      for (size_t c = 0; c < src.size(); ++c) RMM_REQUIRE(src[c] != -2, "LDS cell never written");
      // product reads
      for (int tid = 0; tid < kThreads; ++tid) {
        const int lane = tid & 63, wave = tid >> 6, wm = wave & 1, wn = wave >> 1;
        const int q4 = lane >> 4, c16 = lane & 15;
        for (int u = 0; u < kBK / 16; ++u)
          for (int t = 0; t < 4; ++t) {
            const int k = k0 + 16 * u + 4 * q4 + t;
            const int64_t gs = src[size_t(nA + nB + 16 * u + 4 * q4 + t)];
            RMM_REQUIRE(k < a.K ? gs == k : gs == -1, "g at k %d", k);
            for (int m = 0; m < 4; ++m) {
              const int row = wm * kWave + m * 16 + c16;
              const int cell = row * kBK + 4 * dma_a_slot(row, 4 * u + q4) + t;
              RMM_REQUIRE(cell >= 0 && cell < nA && (cell - t) % 4 == 0, "A read");
              if (row0 + row < a.M) {
                const int64_t want = k < a.K ? int64_t(row0 + row) * a.K + k : -1;
                RMM_REQUIRE(src[size_t(cell)] == want, "x (%d, %d) read", row0 + row, k);
                if (wn == 0 && k < a.K) ss_hits[size_t(row) * a.K + k] += 1;
              }
            }
            for (int q = 0; q < 4; ++q) {
              const int col = wn * kWave + 4 * c16 + q;
              const int cell = nA + (16 * u + 4 * q4 + t) * kBN + col;
              RMM_REQUIRE(cell >= nA && cell < nA + nB && (cell - nA - q) % 4 == 0, "B read");
              if (col0 + col < a.N) {
                const int64_t want = k < a.K ? int64_t(k) * a.N + col0 + col : -1;
                RMM_REQUIRE(src[size_t(cell)] == want, "w (%d, %d) read", k, col0 + col);
              }
            }
          }
      }
    }
    for (int lr = 0; lr < kBM && row0 + lr < a.M; ++lr)
      for (int k = 0; k < a.K; ++k)
        RMM_REQUIRE(ss_hits[size_t(lr) * a.K + k] == 1, "row %d column %d summed %d times",
                    row0 + lr, k, ss_hits[size_t(lr) * a.K + k]);
    // the shuffles (xor 16, 32) combine the four lanes q4 of one row
    for (int tid = 0; tid < kThreads; ++tid)
      for (int sft = 16; sft < 64; sft <<= 1)
        RMM_REQUIRE(((tid ^ sft) & 15) == (tid & 15) && (tid ^ sft) / 64 == tid / 64,
                    "row-sum lanes");
    for (int tid = 0; tid < kThreads; ++tid) {
      const int lane = tid & 63, wave = tid >> 6, wm = wave & 1, wn = wave >> 1;
      const int q4 = lane >> 4, c16 = lane & 15;
      for (int m = 0; m < 4; ++m)
        for (int r = 0; r < 4; ++r) {
          const int row = row0 + wm * kWave + m * 16 + 4 * q4 + r;
          const int col = col0 + wn * kWave + 4 * c16;
          if (row >= a.M || col >= a.N) continue;
          RMM_REQUIRE(col % 4 == 0 && col + 4 <= a.N, "16-byte store");
          for (int q = 0; q < 4; ++q) {
            const size_t e = size_t(row) * a.N + col + q;
            RMM_REQUIRE(stored[e] == 0, "output (%d, %d) stored twice", row, col + q);
            stored[e] = 1;
          }
        }
    }
  }
  for (size_t e = 0; e < stored.size(); ++e)
    RMM_REQUIRE(stored[e] == 1, "output %zu never stored (direct-to-LDS kernel)", e);
}

// Host replay of every workgroup and copy thread through the kernel's own
// index functions, against the definition: for every stored output row and
// column, stage element k of the row is x[row][k] (0 past K) and of the
// column w[k][col] (0 past K); each LDS cell of a stage is written once;
// each row's sum of squares takes every k of that row once, from the 8
// lanes the epilogue's shuffles combine; products pair cells of one k; every
// output element is stored once.
int check(const rms_matmul_params* p, char* msg, size_t len) {
  Args a;
  const int rc = plan(p, &a);
  if (rc != CONV2D_OK) return rc;
  try {
    const int64_t x_bytes = int64_t(a.M) * a.K * 4, w_bytes = int64_t(a.K) * a.N * 4;
    const int nst = (a.K + kBK - 1) / kBK;
    std::vector<unsigned char> stored(size_t(int64_t(a.M) * a.N), 0);
    const int T = a.TM * a.TN;
    std::vector<unsigned char> seen(size_t(T), 0);
    for (int bid = 0; bid < T; ++bid) {
      int tm, tn;
      tile_of(a, bid, &tm, &tn);
      RMM_REQUIRE(tm >= 0 && tm < a.TM && tn >= 0 && tn < a.TN && !seen[size_t(tm * a.TN + tn)],
                  "workgroup %d tile", bid);
      seen[size_t(tm * a.TN + tn)] = 1;
      const int row0 = tm * kBM, col0 = tn * kBN;
      // sums of squares: which k each (row, lane-of-8) took
      std::vector<int> ss_hits(size_t(kBM) * a.K, 0);
      for (int st = 0; st < nst; ++st) {
        const int k0 = st * kBK;
        std::vector<unsigned char> cell(2 * kBM * kPitch, 0);
        for (int tid = 0; tid < kThreads; ++tid) {
          for (int p_ = 0; p_ < kARows; ++p_) {
            const int lr = a_row(tid, p_), row = row0 + lr;
            RMM_REQUIRE(lr < kBM, "A row %d", lr);
            for (int q = 0; q < 4; ++q) {
              const int lk = 4 * a_kq(tid) + q, k = k0 + lk;
              RMM_REQUIRE(lk < kBK, "A k %d", lk);
              const int idx = lr * kPitch + lk;
              RMM_REQUIRE(cell[size_t(idx)] == 0, "A cell written twice");
              cell[size_t(idx)] = 1;
              const uint32_t off = x_offset(a, row, k);
              if (k < a.K) {
                if (row < a.M) {
                  RMM_REQUIRE(int64_t(off) == (int64_t(row) * a.K + k) * 4, "x element (%d, %d)",
                              row, k);
                  ss_hits[size_t(lr) * a.K + k] += 1;
                }
                RMM_REQUIRE(int64_t(off) < x_bytes, "x offset in range");
              } else {
                RMM_REQUIRE(int64_t(off) >= x_bytes, "x past K reads 0");
              }
            }
          }
          for (int p_ = 0; p_ < kBQuads; ++p_) {
            const int lc = b_col(tid), col = col0 + lc;
            for (int q = 0; q < 4; ++q) {
              const int lk = 4 * b_kq(tid, p_) + q, k = k0 + lk;
              RMM_REQUIRE(lk < kBK && lc < kBN, "B cell");
              const int idx = kBM * kPitch + lc * kPitch + lk;
              RMM_REQUIRE(cell[size_t(idx)] == 0, "B cell written twice");
              cell[size_t(idx)] = 1;
              const uint32_t off = w_offset(a, k, col);
              if (k < a.K) {
                if (col < a.N)
                  RMM_REQUIRE(int64_t(off) == (int64_t(k) * a.N + col) * 4, "w element (%d, %d)",
                              k, col);
                RMM_REQUIRE(int64_t(off) < w_bytes, "w offset in range");
              } else {
                RMM_REQUIRE(int64_t(off) >= w_bytes, "w past K reads 0");
              }
            }
          }
        }
        for (int op = 0; op < 2; ++op)
          for (int r = 0; r < kBM; ++r)
            for (int k = 0; k < kBK; ++k)
              RMM_REQUIRE(cell[size_t(op * kBM * kPitch + r * kPitch + k)] == 1,
                          "stage %d cell never written", st);
      }
      // the shuffles combine lanes tid ^ 1, ^ 2, ^ 4: the 8 lanes with the
      // same tid / 8, which own the same rows
      for (int tid = 0; tid < kThreads; ++tid)
        for (int s = 1; s < 8; s <<= 1)
          RMM_REQUIRE(a_row(tid ^ s, 0) == a_row(tid, 0) && (tid ^ s) / 64 == tid / 64,
                      "row-sum lanes");
      for (int lr = 0; lr < kBM && row0 + lr < a.M; ++lr)
        for (int k = 0; k < a.K; ++k)
          RMM_REQUIRE(ss_hits[size_t(lr) * a.K + k] == 1, "row %d column %d summed %d times",
                      row0 + lr, k, ss_hits[size_t(lr) * a.K + k]);
      // products and stores
      for (int tid = 0; tid < kThreads; ++tid) {
        const int lane = tid & 63, wave = tid >> 6, wm = wave & 1, wn = wave >> 1;
        const int q4 = lane >> 4, c16 = lane & 15;
        for (int u = 0; u < kBK / 16; ++u)
          for (int m = 0; m < 4; ++m) {
            const int ar = wm * kWave + m * 16 + c16, br = wn * kWave + m * 16 + c16;
            const int k = 16 * u + 4 * q4;
            RMM_REQUIRE(ar < kBM && br < kBN && k + 4 <= kBK && (ar * kPitch + k) % 4 == 0 &&
                            (br * kPitch + k) % 4 == 0,
                        "operand read");
          }
        for (int m = 0; m < 4; ++m)
          for (int r = 0; r < 4; ++r)
            for (int b = 0; b < 4; ++b) {
              const int row = row0 + wm * kWave + m * 16 + 4 * q4 + r;
              const int col = col0 + wn * kWave + b * 16 + c16;
              if (row >= a.M || col >= a.N) continue;
              const size_t e = size_t(row) * a.N + col;
              RMM_REQUIRE(stored[e] == 0, "output (%d, %d) stored twice", row, col);
              stored[e] = 1;
            }
      }
    }
    for (size_t e = 0; e < stored.size(); ++e)
      RMM_REQUIRE(stored[e] == 1, "output %zu never stored", e);
    if (dma_eligible(a)) check_dma(a);
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

}  // namespace rmm

extern "C" int rms_norm_matmul(const float* x, const float* norm_weight, const float* proj,
                               float* out, const rms_matmul_params* p, void* stream) {
  rmm::Args a;
  const int rc = rmm::plan(p, &a);
  if (rc != CONV2D_OK) return rc;
  const uint64_t nx = uint64_t(a.M) * a.K, nw = uint64_t(a.K) * a.N, no = uint64_t(a.M) * a.N;
  if ((nx && x == nullptr) || norm_weight == nullptr || (nw && proj == nullptr) ||
      (no && out == nullptr))
    return CONV2D_ERR_NULL_PTR;
  auto overlap = [](const void* a0, uint64_t na, const void* b0, uint64_t nb) {
    if (na == 0 || nb == 0) return false;
    const uintptr_t u = reinterpret_cast<uintptr_t>(a0), v = reinterpret_cast<uintptr_t>(b0);
    return u < v + nb && v < u + na;
  };
  if (overlap(out, no * 4, x, nx * 4) || overlap(out, no * 4, norm_weight, uint64_t(a.K) * 4) ||
      overlap(out, no * 4, proj, nw * 4))
    return CONV2D_ERR_ALIAS;
  if (no == 0) return CONV2D_OK;
  a.x = x;
  a.g = norm_weight;
  a.w = proj;
  a.out = out;
  auto aligned = [](const void* v) { return reinterpret_cast<uintptr_t>(v) % 16 == 0; };
  if (rmm::dma_eligible(a) && aligned(x) && aligned(proj) && aligned(out))
    hipLaunchKernelGGL(rmm::rms_matmul_dma_kernel, dim3(a.TM * a.TN), dim3(rmm::kThreads), 0,
                       static_cast<hipStream_t>(stream), a);
  else
    hipLaunchKernelGGL(rmm::rms_matmul_kernel, dim3(a.TM * a.TN), dim3(rmm::kThreads), 0,
                       static_cast<hipStream_t>(stream), a);
  return hipGetLastError() == hipSuccess ? CONV2D_OK : CONV2D_ERR_HIP;
}

extern "C" int rms_norm_matmul_check_indexing(const rms_matmul_params* p, char* msg,
                                              size_t msg_len) {
  return rmm::check(p, msg, msg_len);
}
