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
// contiguous run of tiles, column tiles fastest.
RMM_HD void tile_of(const Args& a, int bid, int* tm, int* tn) {
  const int T = a.TM * a.TN;
  const int q = T >> 3, r = T & 7, x = bid & 7, k = bid >> 3;
  const int t = x * q + imin(x, r) + k;
  *tm = t / a.TN;
  *tn = t - *tm * a.TN;
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
  hipLaunchKernelGGL(rmm::rms_matmul_kernel, dim3(a.TM * a.TN), dim3(rmm::kThreads), 0,
                     static_cast<hipStream_t>(stream), a);
  return hipGetLastError() == hipSuccess ? CONV2D_OK : CONV2D_ERR_HIP;
}

extern "C" int rms_norm_matmul_check_indexing(const rms_matmul_params* p, char* msg,
                                              size_t msg_len) {
  return rmm::check(p, msg, msg_len);
}
