// The input gradient of a 1x1, stride-1, unpadded convolution as one GEMM
// over the pixels of every image, on CDNA4 (gfx950) matrix cores, and its
// host replay.
//
// What is computed (meganeura 0.2.0, conv2d_grad_input_gemm_coop.wgsl,
// header comment, with kH = kW = 1, stride 1 and no padding, where the
// gather rule reads grad_out at the input pixel itself):
//   grad_input[n, ci, p] = sum over co of weight[co, ci] * grad_out[n, co, p]
// for every image n and pixel p = ih * W + iw.  Per image that is the
// page's C[Ci, H*W] = weight^T x grad_out[n].  Here the pixels of all images
// form one column axis q = n * H*W + p, so tiles run across image
// boundaries and no lane is spent on a per-image remainder.
//
// How:
//  * A[k][m] = weight[k, m] (k = co, m = ci) and B[k][q] = grad_out[n, k, p]
//    are both rows of consecutive elements along m or q in memory.  A tile is
//    128 input channels x 128 pixels, four waves of 64 x 64; a stage is 32
//    output channels.  The stage's A and B rows go from memory straight to
//    LDS with 16-byte buffer loads in their LDS form (lane i of a load lands
//    at M0 + 16 i; one load covers two 128-float rows): no staging registers
//    and no LDS writes.  With H*W and Ci multiples of 4, a 4-pixel or
//    4-channel quad never crosses an image or a row end.
//  * The products are short next to a stage's copy, so the copies run three
//    stages ahead: four stage buffers (128 KB), and a wave waits only for the
//    loads of the stage it is about to multiply.  One barrier per stage.
//  * Operands: a lane reads 4 consecutive channels (or pixels) of one k row
//    with one 16-byte read, and matrix instruction q of a block takes the
//    q-th of them, so block q of a wave covers channels (pixels) 4c + q,
//    c = 0 .. 15.  fp32: lane group g supplies k = 4s + g of 4-k step s to
//    v_mfma_f32_16x16x4_f32.  f16-staged: lane group g supplies k = 8g .. 8g
//    + 7, rounded to f16 (round to nearest even) as they leave LDS, to
//    v_mfma_f32_16x16x32_f16 with fp32 accumulation: each operand element
//    is rounded once before it is multiplied, as on the other paths.
//  * Epilogue: a lane holds 4 consecutive pixels of a channel (the four
//    pixel blocks) and stores them with one 16-byte store.  Every output
//    element belongs to exactly one tile and is written once.
//  * Workgroups are dealt to the 8 XCDs in contiguous runs of tiles, channel
//    tiles fastest, so the tiles that read the same grad_out columns meet in
//    one L2.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "pointwise.hpp"

namespace c2b {
namespace pw {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

typedef __attribute__((address_space(3))) void lds_void_t;

// BUFS stage buffers: 4 (loads three stages ahead, one workgroup per CU)
// or 2 (one stage ahead; 64 KiB, so two workgroups share a CU and cover
// each other's waits, which pays when there are more tiles than CUs).
template <bool F16, bool AROW, int BUFS>
__global__ __launch_bounds__(kThreads, BUFS == kBufsShared ? 2 : 1) void pointwise_gemm_kernel(
    const PWArgs a) {
  constexpr int kBufs = BUFS;
  __shared__ f32x4 lds4[kBufs * kStageBytes / 16];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int g = lane >> 4, c16 = lane & 15;
  int tm, tn;
  tile_of(a, blockIdx.x, &tm, &tn);
  const int m0 = tm * kBM, q0 = tn * kBN;
  const int nst = (a.K + kBK - 1) / kBK;
  auto buf = [&](int st) __attribute__((always_inline)) {
    return reinterpret_cast<char*>(lds4) + (st % kBufs) * kStageBytes;
  };
  const __amdgpu_buffer_rsrc_t rsA = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(a.w), 0, a.K * a.M * 4, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsB = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(a.go), 0, int(int64_t(a.Q) * a.K * 4), 0x00020000);
  // this lane's B quad is the same in every load of the wave (the k row
  // changes): its pixel's element offset, fixed for the tile
  const int64_t bbase = b_base(a, q0 + 4 * load_quad(lane));

  // loads of stage st: this wave's loads j = 4 wave + i of each operand
  auto issue = [&](int st) __attribute__((always_inline)) {
    char* base = buf(st);
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int j = kLoads * wave + i;
      const int krow = load_krow(j, lane);
      const uint32_t ao = AROW ? arow_offset(a, st, m0, arow_row(j, lane), arow_kq(j, lane))
                               : a_offset(a, st, m0, krow, load_quad(lane));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsA, (lds_void_t*)(base + j * 1024), 16, ao, 0,
                                               0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsB, (lds_void_t*)(base + kBK * kBM * 4 + j * 1024), 16,
          b_offset(a, st, bbase, krow), 0, 0, 0);
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) acc[x][y] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  // products of stage st: acc[qa][qb] is the block of channels 4c + qa and
  // pixels 4c + qb of the wave's 64 x 64
  // forward (AROW): block qa of the wave covers rows 16 qa + c16 (plain
  // order); a lane reads the k quads of its row at their swizzled slots
  auto arow_read = [&](const char* base, int qa, int kq) __attribute__((always_inline)) {
    const int row = wm * kWave + 16 * qa + c16;
    return *reinterpret_cast<const f32x4*>(base + row * (kBK * 4) +
                                           16 * (kq ^ a_swizzle(row)));
  };
  auto compute = [&](int st) __attribute__((always_inline)) {
    const char* base = buf(st);
    const float* As = reinterpret_cast<const float*>(base) + wm * kWave + 4 * c16;
    const float* Bs = reinterpret_cast<const float*>(base + kBK * kBM * 4) + wn * kWave + 4 * c16;
    if constexpr (AROW && F16) {
      // lane group g: k = 8g .. 8g+7, the row's quads 2g and 2g+1
      f32x4 bv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) bv[i] = *reinterpret_cast<const f32x4*>(Bs + (8 * g + i) * kBN);
      f16x8 ah[4], bh[4];
#pragma unroll
      for (int qa = 0; qa < 4; ++qa) {
        const f32x4 a0 = arow_read(base, qa, 2 * g), a1 = arow_read(base, qa, 2 * g + 1);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          ah[qa][i] = _Float16(a0[i]);
          ah[qa][4 + i] = _Float16(a1[i]);
        }
      }
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int i = 0; i < 8; ++i) bh[q][i] = _Float16(bv[i][q]);
#pragma unroll
      for (int qa = 0; qa < 4; ++qa)
#pragma unroll
        for (int qb = 0; qb < 4; ++qb)
          acc[qa][qb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[qa], bh[qb], acc[qa][qb], 0, 0, 0);
    } else if constexpr (AROW) {
      // 16-k halves h: lane group g reads its row's quad 4h + g; MFMA t of
      // the half takes k = 16h + 4g + t from both operands
#pragma unroll
      for (int h = 0; h < kBK / 16; ++h) {
        f32x4 av[4], bv[4];
#pragma unroll
        for (int qa = 0; qa < 4; ++qa) av[qa] = arow_read(base, qa, 4 * h + g);
#pragma unroll
        for (int t = 0; t < 4; ++t)
          bv[t] = *reinterpret_cast<const f32x4*>(Bs + (16 * h + 4 * g + t) * kBN);
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int qa = 0; qa < 4; ++qa)
#pragma unroll
            for (int qb = 0; qb < 4; ++qb)
              acc[qa][qb] =
                  __builtin_amdgcn_mfma_f32_16x16x4f32(av[qa][t], bv[t][qb], acc[qa][qb], 0, 0, 0);
      }
    } else if constexpr (F16) {
      f32x4 av[8], bv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        av[i] = *reinterpret_cast<const f32x4*>(As + (8 * g + i) * kBM);
        bv[i] = *reinterpret_cast<const f32x4*>(Bs + (8 * g + i) * kBN);
      }
      f16x8 ah[4], bh[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          ah[q][i] = _Float16(av[i][q]);
          bh[q][i] = _Float16(bv[i][q]);
        }
      }
#pragma unroll
      for (int qa = 0; qa < 4; ++qa)
#pragma unroll
        for (int qb = 0; qb < 4; ++qb)
          acc[qa][qb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[qa], bh[qb], acc[qa][qb], 0, 0, 0);
    } else {
#pragma unroll
      for (int s = 0; s < kBK / 4; ++s) {
        const f32x4 av = *reinterpret_cast<const f32x4*>(As + (4 * s + g) * kBM);
        const f32x4 bv = *reinterpret_cast<const f32x4*>(Bs + (4 * s + g) * kBN);
#pragma unroll
        for (int qa = 0; qa < 4; ++qa)
#pragma unroll
          for (int qb = 0; qb < 4; ++qb)
            acc[qa][qb] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[qa], bv[qb], acc[qa][qb], 0, 0, 0);
      }
    }
  };

  // stages 0 .. kBufs - 2 in flight; at stage st a wave waits for its own
  // loads of st (2 * kLoads loads per later stage may stay outstanding), the
  // barrier then covers every wave's loads of st and every read of stage
  // st - 1, whose buffer stage st + kBufs - 1 refills
  for (int st = 0; st < kBufs - 1 && st < nst; ++st) issue(st);
  for (int st = 0; st < nst; ++st) {
    const int ahead = imin(nst - 1 - st, kBufs - 2);
    if (ahead >= 2) __builtin_amdgcn_s_waitcnt(0x4F70);        // vmcnt <= 16
    else if (ahead == 1) __builtin_amdgcn_s_waitcnt(0x0F78);   // vmcnt <= 8
    else __builtin_amdgcn_s_waitcnt(0x0F70);                   // vmcnt = 0
    // a bare barrier: __syncthreads' release fence would wait for every
    // load in flight, later stages included.  The asm statements keep the
    // compiler from moving LDS accesses across it.
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (st + kBufs - 1 < nst) issue(st + kBufs - 1);
    compute(st);
  }

  // register r of acc[qa][qb]: product row 4g + r of block qa (channel
  // 16g + 4r + qa of the wave), column c16 of block qb (pixel 4 c16 + qb):
  // for fixed (qa, r) a lane holds 4 consecutive pixels, one 16-byte store
  const int q = q0 + wn * kWave + 4 * c16;
  if (q >= a.Q) return;
  const int n = q / a.P, p = q - n * a.P;
  float* gi_n = a.gi + (size_t)n * a.M * a.P + p;
#pragma unroll
  for (int qa = 0; qa < 4; ++qa)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      // product row 4g + r of block qa: strided (input gradient) or plain
      const int m = m0 + wm * kWave + (AROW ? 16 * qa + 4 * g + r : 16 * g + 4 * r + qa);
      if (m < a.M)
        *reinterpret_cast<f32x4*>(gi_n + (size_t)m * a.P) =
            f32x4{acc[qa][0][r], acc[qa][1][r], acc[qa][2][r], acc[qa][3][r]};
    }
}

// ---------------------------------------------------------------------------
// Host side.

// The path for a call: the shape above, and 16-byte aligned tensors (the
// loads and stores are 16 bytes wide).
bool pw_applies(const conv2d_params* p, const float* go, const float* w, const float* gi) {
  if (!pw_shape(p)) return false;
  auto aligned = [](const void* x) { return (reinterpret_cast<uintptr_t>(x) & 15u) == 0; };
  return aligned(go) && aligned(w) && aligned(gi);
}

// Launch (shape and pointers already validated, pw_applies true).
template <int BUFS>
void pw_launch_bufs(const PWArgs& a, int f16, int fwd, hipStream_t st) {
  const dim3 grid(a.TM * a.TN), block(kThreads);
  if (f16 && fwd)
    hipLaunchKernelGGL((pointwise_gemm_kernel<true, true, BUFS>), grid, block, 0, st, a);
  else if (f16)
    hipLaunchKernelGGL((pointwise_gemm_kernel<true, false, BUFS>), grid, block, 0, st, a);
  else if (fwd)
    hipLaunchKernelGGL((pointwise_gemm_kernel<false, true, BUFS>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((pointwise_gemm_kernel<false, false, BUFS>), grid, block, 0, st, a);
}

int pw_launch(const float* go, const float* w, float* gi, const conv2d_params* p, int f16,
              void* stream, int fwd, int cus) {
  PWArgs a;
  pw_plan(p, &a, fwd);
  a.go = go;
  a.w = w;
  a.gi = gi;
  if (a.TM == 0 || a.TN == 0) return CONV2D_OK;   // no output channel: nothing to write
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (int64_t(a.TM) * a.TN > cus)
    pw_launch_bufs<kBufsShared>(a, f16, fwd, st);
  else
    pw_launch_bufs<kBufs>(a, f16, fwd, st);
  return hipGetLastError() == hipSuccess ? CONV2D_OK : CONV2D_ERR_HIP;
}

namespace {
struct Failure {
  std::string msg;
};
#define PW_REQUIRE(cond, ...)                                   \
  do {                                                          \
    if (!(cond)) {                                              \
      char buf_[512];                                           \
      std::snprintf(buf_, sizeof buf_, __VA_ARGS__);            \
      throw Failure{std::string(#cond) + ": " + buf_};          \
    }                                                           \
  } while (0)
}  // namespace

// Host replay of the kernel's addressing (pw_shape must hold): every tile
// once; per stage, every LDS cell written by exactly one load lane with the
// definition's element (weight[k, m], grad_out[n, k, p]) or 0 past Co, Ci or
// the pixels; the product reads of every block pair the same k in A and B,
// each k of the stage once; every grad_input element stored once, by the
// lane holding its channel and pixel.
int pw_check(const conv2d_params* p, char* msg, size_t len, int fwd) {
  PWArgs a;
  pw_plan(p, &a, fwd);
  try {
    const int64_t a_bytes = int64_t(a.K) * a.M * 4, b_bytes = int64_t(a.Q) * a.K * 4;
    const int nst = (a.K + kBK - 1) / kBK;
    std::vector<unsigned char> tile_seen(size_t(a.TM) * a.TN, 0);
    std::vector<unsigned char> stored(size_t(int64_t(a.Q) * a.M), 0);
    // source element of an A / B cell: expected byte offset or -1 for 0
    auto a_src = [&](int st, int m0, int krow, int col) -> int64_t {
      const int k = st * kBK + krow, m = m0 + col;
      return (k < a.K && m < a.M) ? (int64_t(k) * a.M + m) * 4 : -1;
    };
    // forward: A[m][k] = weight[m * K + k]
    auto arow_src = [&](int st, int m0, int row, int kk) -> int64_t {
      const int k = st * kBK + kk, m = m0 + row;
      return (k < a.K && m < a.M) ? (int64_t(m) * a.K + k) * 4 : -1;
    };
    auto b_src = [&](int st, int q0, int krow, int col) -> int64_t {
      const int k = st * kBK + krow, q = q0 + col;
      if (k >= a.K || q >= a.Q) return -1;
      const int n = q / a.P, pp = q % a.P;
      return ((int64_t(n) * a.K + k) * a.P + pp) * 4;
    };
    for (int bid = 0; bid < a.TM * a.TN; ++bid) {
      int tm, tn;
      tile_of(a, bid, &tm, &tn);
      PW_REQUIRE(tm >= 0 && tm < a.TM && tn >= 0 && tn < a.TN, "tile of %d", bid);
      PW_REQUIRE(!tile_seen[size_t(tm) * a.TN + tn], "tile (%d, %d) twice", tm, tn);
      tile_seen[size_t(tm) * a.TN + tn] = 1;
      const int m0 = tm * kBM, q0 = tn * kBN;
      // stage addressing does not depend on the stage beyond k, so the
      // first, second and last stages stand for all of them
      for (int st : {0, 1, nst - 1}) {
        if (st < 0 || st >= nst) continue;
        std::vector<int64_t> cellA(kBK * kBM, -2), cellB(kBK * kBN, -2);
        if (fwd) {
          // A stage as [row][slot][4]: slot s of row r holds k quad
          // s ^ a_swizzle(r); kept in cellA[r * kBK + k]
          for (int wave = 0; wave < kThreads / 64; ++wave)
            for (int lane = 0; lane < 64; ++lane)
              for (int i = 0; i < kLoads; ++i) {
                const int j = kLoads * wave + i, row = arow_row(j, lane), kq = arow_kq(j, lane);
                const int byte = j * 1024 + 16 * lane;   // M0 + 16 lane
                PW_REQUIRE(byte / (kBK * 4) == row && (byte % (kBK * 4)) / 16 == (lane % 8),
                           "forward A lane layout");
                PW_REQUIRE((lane % 8) == (kq ^ a_swizzle(row)), "swizzle not an involution");
                const uint32_t oa = arow_offset(a, st, m0, row, kq);
                PW_REQUIRE(oa == kPad || int64_t(oa) + 16 <= a_bytes, "A load in range");
                for (int e = 0; e < 4; ++e) {
                  const int cell = row * kBK + 4 * kq + e;
                  PW_REQUIRE(cellA[cell] == -2, "A cell written twice");
                  const int64_t ea = arow_src(st, m0, row, 4 * kq + e);
                  const int64_t ga = oa == kPad ? -1 : int64_t(oa) + 4 * e;
                  PW_REQUIRE(ga == ea, "A cell (%d, %d) of tile %d stage %d", row, 4 * kq + e,
                             bid, st);
                  cellA[cell] = ea;
                }
              }
          // reads: block qa of wave row wm, lane (c16, g) reads its row's
          // k quads (f16: 2g and 2g + 1; fp32: 4h + g) at slot kq ^ swizzle
          for (int wm = 0; wm < 2; ++wm)
            for (int qa = 0; qa < 4; ++qa)
              for (int c16 = 0; c16 < 16; ++c16) {
                const int row = wm * kWave + 16 * qa + c16;
                for (int kq = 0; kq < kBK / 4; ++kq) {
                  const int slot = kq ^ a_swizzle(row);
                  PW_REQUIRE(slot >= 0 && slot < kBK / 4, "read slot");
                  for (int e = 0; e < 4; ++e)
                    PW_REQUIRE(cellA[row * kBK + 4 * kq + e] != -2, "read of an unwritten cell");
                }
              }
          // bank spread of one read instruction: the 16 lanes of a group
          // (consecutive rows, one k quad) cover 16 distinct 4-bank groups
          for (int qa = 0; qa < 4; ++qa)
            for (int kq = 0; kq < kBK / 4; ++kq) {
              unsigned used = 0;
              for (int c16 = 0; c16 < 16; ++c16) {
                const int row = 16 * qa + c16;
                const int grp = ((row * kBK * 4 + 16 * (kq ^ a_swizzle(row))) / 16) % 16;
                used |= 1u << grp;
              }
              PW_REQUIRE(used == 0xffffu, "forward A read conflicts (quad %d)", kq);
            }
        }
        for (int wave = 0; wave < kThreads / 64; ++wave)
          for (int lane = 0; lane < 64; ++lane) {
            const int64_t bbase = b_base(a, q0 + 4 * load_quad(lane));
            for (int i = 0; i < kLoads; ++i) {
              const int j = kLoads * wave + i, krow = load_krow(j, lane);
              const int quad = load_quad(lane);
              const uint32_t oa = fwd ? 0u : a_offset(a, st, m0, krow, quad);
              const uint32_t ob = b_offset(a, st, bbase, krow);
              for (int e = 0; e < 4; ++e) {
                const int byte = j * 1024 + 16 * lane + 4 * e;   // M0 + 16 lane
                const int cell = byte / 4, row = cell / kBM, col = cell % kBM;
                PW_REQUIRE(row == krow && col == 4 * quad + e, "lane layout");
                PW_REQUIRE(cellB[cell] == -2, "cell written twice");
                const int64_t eb = b_src(st, q0, row, col);
                cellB[cell] = eb;
                const int64_t gb = ob >= uint32_t(b_bytes) ? -1 : int64_t(ob) + 4 * e;
                PW_REQUIRE(gb == eb, "B cell (%d, %d) of tile %d stage %d", row, col, bid, st);
                PW_REQUIRE(ob == kPad || int64_t(ob) + 16 <= b_bytes, "B load in range");
                if (fwd) continue;
                PW_REQUIRE(cellA[cell] == -2, "cell written twice");
                const int64_t ea = a_src(st, m0, row, col);
                const int64_t ga = oa >= uint32_t(a_bytes) ? -1 : int64_t(oa) + 4 * e;
                // 16-byte loads are whole: an in-range load must hold the
                // definition's element, padding only where it has none
                PW_REQUIRE(ga == ea || (ga >= 0 && ea < 0 && m0 + col >= a.M),
                           "A cell (%d, %d) of tile %d stage %d", row, col, bid, st);
                PW_REQUIRE(oa == kPad || int64_t(oa) + 16 <= a_bytes, "A load in range");
                cellA[cell] = ea;
              }
            }
          }
        for (int c = 0; c < kBK * kBM; ++c) PW_REQUIRE(cellA[c] != -2, "cell never written");
      }
      // products: block (qa, qb) of wave (wm, wn) pairs A cell [k][wm 64 +
      // 4 c + qa] with B cell [k][wn 64 + 4 c' + qb]; lane (c16, g) supplies
      // k = 8g + i (f16) or 4s + g (fp32): over the lanes of a block each k
      // of the stage appears once per row and column
      for (int f16 = 0; f16 < 2; ++f16) {
        std::vector<int> seen(kBK, 0);
        for (int g = 0; g < 4; ++g)
          for (int i = 0; i < 8; ++i) {
            const int k = f16 ? 8 * g + i : 4 * i + g;
            PW_REQUIRE(k >= 0 && k < kBK, "k of a read");
            ++seen[k];
          }
        for (int k = 0; k < kBK; ++k) PW_REQUIRE(seen[k] == 1, "k %d read %d times", k, seen[k]);
      }
      // stores
      for (int wave = 0; wave < 4; ++wave)
        for (int lane = 0; lane < 64; ++lane) {
          const int wm = wave & 1, wn = wave >> 1, g = lane >> 4, c16 = lane & 15;
          const int q = q0 + wn * kWave + 4 * c16;
          if (q >= a.Q) continue;
          for (int qa = 0; qa < 4; ++qa)
            for (int r = 0; r < 4; ++r) {
              const int m = m0 + wm * kWave + (fwd ? 16 * qa + 4 * g + r : 16 * g + 4 * r + qa);
              // the accumulator row 4g + r of block qa is channel
              // strided(4g + r, qa) (input gradient) or row 16 qa + 4g + r
              // (forward: block qa read rows 16 qa + c16); its column c16
              // of block qb is pixel strided(c16, qb)
              PW_REQUIRE(m == m0 + wm * kWave +
                                  (fwd ? 16 * qa + 4 * g + r : strided(4 * g + r, qa)),
                         "store row");
              if (m >= a.M) continue;
              for (int qb = 0; qb < 4; ++qb) {
                PW_REQUIRE(q + qb == q0 + wn * kWave + strided(c16, qb), "store column");
                PW_REQUIRE((q + qb) / a.P == q / a.P, "a store crosses an image");
                const size_t e = size_t(q + qb) * a.M + m;
                PW_REQUIRE(!stored[e], "output (%d, %d) stored twice", m, q + qb);
                stored[e] = 1;
              }
            }
        }
    }
    for (size_t e = 0; e < stored.size(); ++e)
      PW_REQUIRE(stored[e], "output %zu never stored", e);
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

}  // namespace pw
}  // namespace c2b
