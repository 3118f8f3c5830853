// Convolution input-gradient as an implicit GEMM on CDNA4 (gfx950) matrix
// cores, and the C-ABI entry points that launch it.
//
// What is computed (meganeura 0.2.0, conv2d_grad_input_gemm_coop.wgsl, header
// comment): per batch item, C[Ci, H*W] = A[Ci, K] x B[K, H*W] with
// K = Co*kH*kW, A[ci, (co,kh,kw)] = weight[co, ci, kh, kw] (weight_T staging)
// and B the im2col of grad_out under the stride > 1 gather rule.
//
// How it is computed here (a re-design for gfx950, not the shader's scheme):
//  * Stride-residue classes (plan.hpp): every class is a dense stride-1
//    problem on a sub-image, so no structural zero is staged or multiplied.
//    Batch, class, pixel band and channel block are folded into one
//    one-dimensional grid.  Workgroups are dealt to the 8 XCDs round robin,
//    so the tile index is remapped (decode_tile) to give each XCD one
//    contiguous run of tiles: neighbours that share halo rows and weights
//    then meet in the same L2.
//  * B is never materialised: per stage a workgroup copies the grad_out
//    window its pixels read (band rows plus the kernel halo, zero outside the
//    image) into LDS once, then every tap reads that window at a fixed
//    offset, so each grad_out element crosses from L2/HBM once per stage
//    instead of once per tap.
//  * Window and weights reach LDS through registers (tile_index.hpp, copy
//    batches): each load instruction reads 64 consecutive cells of one
//    channel, and each lane writes the 4 channels of one cell to LDS with one
//    16-byte store; loads past a tensor's extent return 0, which supplies the
//    padding halo.  (Loads that write LDS directly were measured to stall the
//    matrix cores' LDS reads for the whole time they land.)  Two stage
//    buffers: at the end of stage s the lanes write stage s+1 (loaded a stage
//    earlier) into the buffer stage s-1 used and issue the loads of stage
//    s+2; one barrier per stage.
//  * The wave shape and the stage shape (channel groups x taps) come from the
//    planner's cost model of the schedule over all CUs, or, after
//    conv2d_tune, from measurement.
//  * Few input channels (cm variants, plan.hpp): the kernel's column taps
//    join the input channels in the 16 matrix rows, the contraction runs over
//    output channels x row taps, and the epilogue adds each pixel's
//    column-tap partial sums through LDS.
//  * fp32 path: v_mfma_f32_16x16x4_f32, four per (unit, block).  f16-staged
//    path: the same fp32 data in LDS, rounded to f16 (round to nearest even)
//    as it is read into registers -- every operand element is rounded exactly
//    once before it is multiplied -- and two units (32 values of k) per
//    v_mfma_f32_16x16x32_f16 (a lone last unit on v_mfma_f32_16x16x16_f16),
//    fp32 accumulators.
//  * Epilogue: masked stores straight to NCHW grad_input; every pixel of a
//    class is owned by exactly one tile, so grad_input is overwritten once,
//    with no race between workgroups.
//  * The same body, with the roles of the operands exchanged (plan.hpp),
//    runs the forward convolution (conv2d_forward_mm_kernel).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstring>
#include <mutex>
#include <utility>
#include <vector>

#include "pointwise.hpp"
#include "tile_index.hpp"

namespace c2b {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// Word 3 of a raw (untyped, unswizzled) buffer resource: 32-bit data format.
constexpr int kRawBufferFlags = 0x00020000;
// One fp32 value from a buffer (0 if `byte_offset` is past the range); the
// builtin returns the raw 32 bits.
__device__ __forceinline__ float load_f32(__amdgpu_buffer_rsrc_t rs, uint32_t byte_offset) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, byte_offset, 0, 0));
}

// Four fp32 values rounded to f16 (round to nearest even).
__device__ __forceinline__ f16x4 to_f16(f32x4 x) { return __builtin_convertvector(x, f16x4); }

__device__ __forceinline__ f16x8 join(f16x4 lo, f16x4 hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

template <bool FWD, bool F16, int WM, int WN, int MB, int NBW, int SF, bool CM, bool MC>
__device__ __forceinline__ void mm_body(const LaunchArgs& a) {
  static_assert(!CM || (WM == 1 && MB == 1), "cm: one matrix block of rows");
  static_assert(!FWD || !CM, "forward launches have no cm variant");
  static_assert(!MC || (!FWD && !CM && !F16), "multi-class: fp32 input gradient only");
  using G = MMGeom<WM, WN, MB, NBW, SF>;
  constexpr int MT = G::kMT, NW = G::kWaves, NJ = G::kBatches;
  constexpr int kStageFloats = SF;   // this instance's stage buffer
  __shared__ f32x4 lds4[2 * SF / 4];
  float* lds = reinterpret_cast<float*>(lds4);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int mg = wave % WM, ng = wave / WM;
  const int g = lane >> 4, c16 = lane & 15;
  const TileCtx c = decode_tile(a, blockIdx.x);
  const PhaseDesc& P = c.P;
  const int OHOW = a.OH * a.OW;
  const float* go_n = a.go + (size_t)c.n * a.Co * OHOW;
  const int nst = c.nstages;
  // copy batches (tile_index.hpp): batch wave + NW*j of every stage is this
  // wave's j-th; its 64 lanes load 4 channels each and write 16 bytes to LDS
  const int NB = stage_batches(P);
  const int WB = window_blocks(P);
  const uint32_t wch = window_channel_bytes(a), tch = weight_channel_bytes(a);

  uint32_t off[NJ];   // per-lane source offsets of this wave's batches
  f32x4 stg[NJ];      // a stage's batches between their loads and LDS writes
  int wgroup = -1;    // tap group the weight offsets are for
  struct StageSrc {
    __amdgpu_buffer_rsrc_t rg, rw;
    int nco;   // contraction channels of the stage
  };
  // (Every lambda here is forced inline: an outlined one becomes a real call
  // with its own stack frame.)
  auto stage_src = [&](int st) __attribute__((always_inline)) {
    int co0, grp;
    stage_split(c, st, &co0, &grp);
    const int nco = imin(16 * P.cg, a.Co - co0);
    StageSrc sc;
    sc.nco = nco;
    sc.rg = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(go_n + (size_t)co0 * OHOW), 0,
                                              nco * OHOW * 4, kRawBufferFlags);
    // the stage's weights: its contraction channels, which on the input-
    // gradient path are whole leading rows of w; on a forward launch they
    // are interleaved with the other channels of every output channel, so
    // the range runs to the end of w
    const int wrange = FWD ? a.Ci * a.Co * a.KH * a.KW - co0 * a.wsk : nco * a.wsk;
    sc.rw = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(a.w + (size_t)co0 * a.wsk), 0,
                                              wrange * 4, kRawBufferFlags);
    return sc;
  };
  // Source offsets of this wave's batches: window blocks once per tile,
  // weight blocks whenever the tap group changes.  The empty asm makes the
  // lane index opaque, so the compiler cannot hoist the group-independent
  // part of every offset out of the stage loop (that would hold more
  // registers per batch).
  auto set_offsets = [&](int grp, bool window_too) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int k = wave + NW * j;
      if (k >= NB) break;
      int block, quad;
      batch_split(P, k, &block, &quad);
      if (block < WB) {
        if (window_too) off[j] = window_lane_offset(c, a, block, lane);
      } else {
        int ln = lane;
        asm volatile("" : "+v"(ln));
        off[j] = weight_lane_offset<MT, CM>(c, a, block - WB, ln, grp);
      }
    }
    wgroup = grp;
  };
  auto update_weight_offsets = [&](int st) __attribute__((always_inline)) {
    int co0, grp;
    stage_split(c, st, &co0, &grp);
    if (grp != wgroup) set_offsets(grp, false);
  };
  // Loads of this wave's batches of stage st into stg[]: four channels per
  // lane, each load reading 64 consecutive cells of one channel.
  auto load_stage = [&](int st) __attribute__((always_inline)) {
    const StageSrc sc = stage_src(st);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int k = wave + NW * j;
      if (k >= NB) break;
      int block, quad;
      batch_split(P, k, &block, &quad);
      const bool win = block < WB;
      const __amdgpu_buffer_rsrc_t rs = win ? sc.rg : sc.rw;
      const uint32_t ch = win ? wch : tch;
      const uint32_t o = off[j] + 4u * uint32_t(quad) * ch;
      uint32_t o0 = o, o1 = o + ch, o2 = o + 2u * ch, o3 = o + 3u * ch;
      if (FWD && !win) {
        // forward: weights of channels past the stage's last one are not
        // cut by the buffer range (see stage_src), so they read 0 explicitly
        const int c0 = 4 * quad;
        if (c0 >= sc.nco) o0 = kPadOffset;
        if (c0 + 1 >= sc.nco) o1 = kPadOffset;
        if (c0 + 2 >= sc.nco) o2 = kPadOffset;
        if (c0 + 3 >= sc.nco) o3 = kPadOffset;
      }
      stg[j] = f32x4{load_f32(rs, o0), load_f32(rs, o1), load_f32(rs, o2), load_f32(rs, o3)};
    }
  };
  // LDS writes of stg[] into stage buffer buf (16 bytes per lane).
  auto write_stage = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int k = wave + NW * j;
      if (k >= NB) break;
      int block, quad;
      batch_split(P, k, &block, &quad);
      const int f = batch_lds_float(P, block, quad, lane);
      if (f >= 0) *reinterpret_cast<f32x4*>(lds + buf * kStageFloats + f) = stg[j];
    }
  };

  // Stage 0 is copied now; stage 1 is loaded now and written at the end of
  // stage 0.
  set_offsets(0, true);
  if (nst > 0) {
    load_stage(0);
    write_stage(0);
  }
  if (nst > 1) {
    update_weight_offsets(1);
    load_stage(1);
  }

  // byte offsets within a stage buffer: block b's window cell (quad g,
  // first tap of the class), and block m's weights (quad g, t = 0) within
  // the weight region
  int bb[NBW];
#pragma unroll
  for (int b = 0; b < NBW; ++b)
    bb[b] = (g * P.slots + (MC   ? window_pixel(c, mm_local(b, ng, c16, WN))
                            : CM ? window_base_cm(c, mm_local(b, ng, c16, WN))
                                 : window_base(c, mm_local(b, ng, c16, WN)))) * 16;
  int aq[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m) aq[m] = (g * P.qp + mm_channel(m, mg, c16, MB) * 4 * P.pt) * 4;

  // one accumulator set, or (multi-class) one per class
  constexpr int NCL = MC ? kMCClasses : 1;
  f32x4 accs[NCL][MB][NBW];
#pragma unroll
  for (int k = 0; k < NCL; ++k)
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
      for (int b = 0; b < NBW; ++b) accs[k][m][b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  auto& acc = accs[0];

  // Blocks of this wave that hold at least one of the tile's pixels (or cm
  // points): a prefix of its NBW blocks.  A tile whose pixel count is not a
  // multiple of the lane tile leaves the last block of some waves empty;
  // those waves skip that block's reads and products (one uniform branch per
  // unit; fewer empty blocks are rare and are multiplied as padding).
  bool last_on = true;
  {
    const int npts = CM ? cm_points(c) : c.npx;
    last_on = NBW == 1 || ((NBW - 1) * WN + ng) * 16 < npts;
  }

  // All addresses, then all reads of one unit: the scheduling barriers keep
  // the compiler from recycling a read's target register as the next
  // address, which would serialise the reads.
  auto read_unit = [&](const char* Hb, const char* Ab, int wo, int ao, f32x4(&bv)[NBW],
                       f32x4(&aw)[MB]) __attribute__((always_inline)) {
    const f32x4* ba[NBW];
#pragma unroll
    for (int b = 0; b < NBW; ++b) ba[b] = reinterpret_cast<const f32x4*>(Hb + bb[b] + wo);
    const f32x4* aa[MB];
#pragma unroll
    for (int m = 0; m < MB; ++m) aa[m] = reinterpret_cast<const f32x4*>(Ab + aq[m] + ao);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int m = 0; m < MB; ++m) aw[m] = *aa[m];
#pragma unroll
    for (int b = 0; b < NBW - 1; ++b) bv[b] = *ba[b];
    if (last_on) bv[NBW - 1] = *ba[NBW - 1];
    __builtin_amdgcn_sched_barrier(0);
  };
  // Products of one unit: blocks 0 .. NBW-2, then the last block if it holds
  // a pixel (every accumulator still takes its four k values in order).
  auto mma_f32 = [&](f32x4(&ac)[MB][NBW], const f32x4(&bv)[NBW],
                     const f32x4(&aw)[MB]) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int b = 0; b < NBW - 1; ++b)
          ac[m][b] = __builtin_amdgcn_mfma_f32_16x16x4f32(aw[m][q], bv[b][q], ac[m][b], 0, 0, 0);
    if (last_on) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int m = 0; m < MB; ++m)
          ac[m][NBW - 1] = __builtin_amdgcn_mfma_f32_16x16x4f32(aw[m][q], bv[NBW - 1][q],
                                                               ac[m][NBW - 1], 0, 0, 0);
    }
  };
  auto mma_f16_pair = [&](const f32x4(&bv0)[NBW], const f32x4(&aw0)[MB],
                          const f32x4(&bv1)[NBW],
                          const f32x4(&aw1)[MB]) __attribute__((always_inline)) {
    f16x8 ah[MB];
#pragma unroll
    for (int m = 0; m < MB; ++m) ah[m] = join(to_f16(aw0[m]), to_f16(aw1[m]));
#pragma unroll
    for (int b = 0; b < NBW; ++b) {
      if (b == NBW - 1 && !last_on) break;
      const f16x8 bh = join(to_f16(bv0[b]), to_f16(bv1[b]));
#pragma unroll
      for (int m = 0; m < MB; ++m)
        acc[m][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[m], bh, acc[m][b], 0, 0, 0);
    }
  };
  auto mma_f16_single = [&](const f32x4(&bv)[NBW],
                            const f32x4(&aw)[MB]) __attribute__((always_inline)) {
    f16x4 ah[MB];
#pragma unroll
    for (int m = 0; m < MB; ++m) ah[m] = to_f16(aw[m]);
#pragma unroll
    for (int b = 0; b < NBW; ++b) {
      if (b == NBW - 1 && !last_on) break;
      const f16x4 bh = to_f16(bv[b]);
#pragma unroll
      for (int m = 0; m < MB; ++m)
        acc[m][b] = __builtin_amdgcn_mfma_f32_16x16x16f16(ah[m], bh, acc[m][b], 0, 0, 0);
    }
  };

  // Multiply stage st out of buffer st&1 (the copies run after it, in the
  // stage loop below).  Units run channel group by channel group, taps in
  // class order inside a group (cm variants: row taps only).
  // Multi-class stage st: for each channel group, each class, each tap
  // (j, l) of the class (kernel tap (rh + 2j, rw + 2l)): the class's blocks
  // at its window offset, into its accumulator set.
  auto compute_mc = [&](int st) __attribute__((always_inline)) {
    const char* Hb = reinterpret_cast<const char*>(lds + (st & 1) * kStageFloats);
    const char* Ab = Hb + P.wfl * 4;
#pragma unroll 1
    for (int cgi = 0; cgi < P.cg; ++cgi) {
#pragma unroll
      for (int k = 0; k < NCL; ++k) {
        const MCClass& K = a.mcls[k];
        // (opaque: otherwise the compiler keeps every class's window offset
        // added to every block's read base, in registers, across the stage
        // loop)
        int wk = cgi * P.slots * 64 + (K.e * c.roww + K.f) * 16;
        asm volatile("" : "+s"(wk));
        // (not unrolled: unrolled tap loops hold several units' operands)
#pragma unroll 1
        for (int j = 0; j < K.th; ++j)
#pragma unroll 1
          for (int l = 0; l < K.tw; ++l) {
            const int kidx = (K.rh + 2 * j) * a.KW + (K.rw + 2 * l);
            f32x4 bv[NBW], aw[MB];
            read_unit(Hb, Ab, wk + tap_window_offset(c, j, l) * 16,
                      cgi * P.qp * 16 + kidx * 16, bv, aw);
            mma_f32(accs[k], bv, aw);
          }
      }
    }
  };
  auto compute = [&](int st) __attribute__((always_inline)) {
    if constexpr (MC) {
      compute_mc(st);
      return;
    }
    const int buf = st & 1;
    int co0, grp;
    stage_split(c, st, &co0, &grp);
    (void)co0;
    const int tap0 = grp * P.tg;
    const int ntg = imin(P.tg, c.ntaps - tap0);
    const int units = P.cg * ntg;
    const char* Hb = reinterpret_cast<const char*>(lds + buf * kStageFloats);
    const char* Ab = Hb + P.wfl * 4;
    const int twl = CM ? 1 : P.tw;   // taps per window row in the tap loop
    const int j0 = tap0 / twl, l0 = tap0 - j0 * twl;
    int cgi = 0, t = 0, j = j0, l = l0;
    auto wo = [&]() __attribute__((always_inline)) {
      return cgi * P.slots * 64 + tap_window_offset(c, j, l) * 16;
    };
    auto ao = [&]() __attribute__((always_inline)) { return cgi * P.qp * 16 + t * 16; };
    auto advance = [&]() __attribute__((always_inline)) {
      if (++t == ntg) {
        t = 0;
        ++cgi;
        j = j0;
        l = l0;
      } else if (++l == twl) {
        l = 0;
        ++j;
      }
    };
    if constexpr (!F16) {
      for (int u = 0; u < units; ++u) {
        f32x4 bv[NBW], aw[MB];
        read_unit(Hb, Ab, wo(), ao(), bv, aw);
        mma_f32(acc, bv, aw);
        advance();
      }
    } else {
      int u = 0;
      for (; u + 2 <= units; u += 2) {
        f32x4 bv0[NBW], aw0[MB], bv1[NBW], aw1[MB];
        read_unit(Hb, Ab, wo(), ao(), bv0, aw0);
        advance();
        read_unit(Hb, Ab, wo(), ao(), bv1, aw1);
        advance();
        mma_f16_pair(bv0, aw0, bv1, aw1);
      }
      if (u < units) {
        f32x4 bv[NBW], aw[MB];
        read_unit(Hb, Ab, wo(), ao(), bv, aw);
        mma_f16_single(bv, aw);
      }
    }
  };
  __syncthreads();   // stage 0 is in LDS
  for (int st = 0; st < nst; ++st) {
    compute(st);
    // stage st+1 (loaded one stage ago) into the buffer stage st-1 used, then
    // the loads of stage st+2, which have all of stage st+1 to land
    if (st + 1 < nst) write_stage((st + 1) & 1);
    if (st + 2 < nst) {
      update_weight_offsets(st + 2);
      load_stage(st + 2);
    }
    __syncthreads();   // stage st+1 is in LDS, buffer st&1 may be refilled
  }

  float* gi_n = a.gi + (size_t)c.n * a.Ci * (a.H * a.W);
  const size_t HW = (size_t)a.H * a.W;
  if constexpr (CM) {
    // cm epilogue: register r of block b holds matrix row 4g + r (input
    // channel ci0 + row / twm, column tap row mod twm) at point
    // (b*WN + ng)*16 + c16.  The rows go to LDS (the stage buffers are free
    // after the last barrier), then every pixel (i', j') of the tile adds its
    // tw column taps: tap l of the pixel sits at window column
    // j' + tw - 1 - l of the pixel's row.
    if (nst == 0) {
      // a class no tap reaches: zeros
      const int rows = c.R - P.th + 1;
      for (int cl = 0; cl < a.cit && c.ci0 + cl < a.Ci; ++cl)
        for (int q = tid; q < rows * P.wb; q += 64 * WM * WN) {
          const int r = fast_div(q, P.m_wb), jj = q - r * P.wb;
          const int col = c.band * P.wb + jj;
          if (col >= P.wp) continue;
          gi_n[(c.ci0 + cl) * HW + (P.ih0 + a.S * (c.i_start + r)) * a.W + P.iw0 + a.S * col] =
              0.0f;
        }
      return;
    }
    constexpr int QP = 16 * NBW * WN + 4;   // floats per matrix row in LDS
    static_assert(16 * QP <= 2 * SF, "cm rows fit the stage buffers");
#pragma unroll
    for (int b = 0; b < NBW; ++b) {
      const int local = mm_local(b, ng, c16, WN);
#pragma unroll
      for (int r = 0; r < 4; ++r) lds[(4 * g + r) * QP + local] = acc[0][b][r];
    }
    __syncthreads();
    const int rows = c.R - P.th + 1;
    for (int cl = 0; cl < a.cit && c.ci0 + cl < a.Ci; ++cl) {
      float* gi_c = gi_n + (c.ci0 + cl) * HW;
      const float* qrow = lds + cl * a.twm * QP;
      for (int q = tid; q < rows * P.wb; q += 64 * WM * WN) {
        const int r = fast_div(q, P.m_wb), jj = q - r * P.wb;
        const int col = c.band * P.wb + jj;
        if (col >= P.wp) continue;
        const int pt0 = r * c.roww + jj + P.tw - 1;   // column tap 0
        float v = 0.0f;
        for (int l = 0; l < P.tw; ++l) v += qrow[l * QP + pt0 - l];
        gi_c[(P.ih0 + a.S * (c.i_start + r)) * a.W + P.iw0 + a.S * col] = v;
      }
    }
    return;
  }
  if constexpr (MC) {
    // register r of block (m, b) of class k holds input channel
    // (mg*MB + m)*16 + 4g + r at the block's grid point.  The two classes of
    // a row class hold adjacent columns there, so a lane stores them
    // together (8 bytes) and 16 lanes fill whole lines; with an odd width
    // (or a grad_input not 8-byte aligned) the pair is stored as two floats.
    const bool pairs =
        (a.W & 1) == 0 && (reinterpret_cast<uintptr_t>(a.gi) & 7) == 0;
    // (an opaque copy of the lane's column, so that the store addresses are
    // formed here rather than hoisted above the stage loop, where they
    // would hold registers the accumulators need)
    int c16e = c16;
    asm volatile("" : "+v"(c16e));
#pragma unroll
    for (int hk = 0; hk < 2; ++hk)
#pragma unroll
      for (int b = 0; b < NBW; ++b) {
        int ih, col0;
        bool even_ok, odd_ok;
        if (!mc_pair_pixel(c, a, hk, mm_local(b, ng, c16e, WN), &ih, &col0, &even_ok, &odd_ok))
          continue;
        const bool k0_even = a.mcls[2 * hk].iw0 == 0;
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int cc = c.ci0 + (mg * MB + m) * 16 + 4 * g + r;
            if (cc >= a.Ci) continue;
            const float v0 = accs[2 * hk][m][b][r], v1 = accs[2 * hk + 1][m][b][r];
            const float ve = k0_even ? v0 : v1, vo = k0_even ? v1 : v0;
            float* dst = gi_n + cc * HW + ih * a.W + col0;
            if (pairs && even_ok && odd_ok) {
              *reinterpret_cast<float2*>(dst) = make_float2(ve, vo);
            } else {
              if (even_ok) dst[0] = ve;
              if (odd_ok) dst[1] = vo;
            }
          }
      }
    return;
  }
  // epilogue: register r of block (m, b) holds input channel
  // (mg*MB + m)*16 + 4g + r, pixel (b*WN + ng)*16 + c16
#pragma unroll
  for (int b = 0; b < NBW; ++b) {
    const int po = output_offset(c, a, mm_local(b, ng, c16, WN));
    if (po < 0) continue;
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int cc = c.ci0 + (mg * MB + m) * 16 + 4 * g + r;
        if (cc < a.Ci) gi_n[cc * HW + po] = acc[m][b][r];
      }
  }
}

// The input-gradient kernel, one instantiation per variant.
template <bool F16, int WM, int WN, int MB, int NBW, int SF, bool CM, bool MC>
__global__ __launch_bounds__(64 * WM * WN, SF == kStageFloatsHalf ? 2 : 1) void grad_input_mm_kernel(
    const LaunchArgs a) {
  mm_body<false, F16, WM, WN, MB, NBW, SF, CM, MC>(a);
}

// The forward convolution on the same body (roles exchanged, plan.hpp), one
// instantiation per variant without cm.
template <bool F16, int WM, int WN, int MB, int NBW, int SF>
__global__ __launch_bounds__(64 * WM * WN, SF == kStageFloatsHalf ? 2 : 1) void conv2d_forward_mm_kernel(
    const LaunchArgs a) {
  mm_body<true, F16, WM, WN, MB, NBW, SF, false, false>(a);
}

template <int V>
void launch_variant(const LaunchArgs& la, hipStream_t st) {
  constexpr Variant v = kVariants[V];
  if constexpr (v.cm == 0 && v.mc == 0) {
    if (la.fwd) {
      hipLaunchKernelGGL((conv2d_forward_mm_kernel<v.f16 != 0, v.wm, v.wn, v.mb, v.nbw,
                                                   stage_floats(v)>),
                         dim3(la.total_tiles), dim3(64 * v.wm * v.wn), 0, st, la);
      return;
    }
  }
  hipLaunchKernelGGL((grad_input_mm_kernel<v.f16 != 0, v.wm, v.wn, v.mb, v.nbw, stage_floats(v),
                                           v.cm != 0, v.mc != 0>),
                     dim3(la.total_tiles), dim3(64 * v.wm * v.wn), 0, st, la);
}

template <int... Vs>
void launch_dispatch(const LaunchArgs& la, hipStream_t st, std::integer_sequence<int, Vs...>) {
  ((la.variant == Vs ? launch_variant<Vs>(la, st) : void()), ...);
}

// Compute units of the current device, read once per device.
int device_cus() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cus_of[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return kDefaultCUs;
  if (dev >= 0 && dev < kMaxDevices) {
    const int known = cus_of[dev].load(std::memory_order_relaxed);
    if (known > 0) return known;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < 1)
    return kDefaultCUs;
  if (dev >= 0 && dev < kMaxDevices) cus_of[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

// Launch plans of recent shapes (host memory only), so that a repeated call
// skips the planner's search.  Keyed by the shape, the operation, the path,
// the variant (-1: the model's choice) and the CU count; at most
// kPlanCacheSize entries, least recently used evicted.  A cached plan is only
// a memo of build_plan: evicting one changes no result.
struct PlanKey {
  conv2d_params p;
  int op, f16, variant, cus;
};
struct PlanEntry {
  PlanKey key;
  std::vector<LaunchArgs> launches;
};
constexpr size_t kPlanCacheSize = 64;

// The variant chosen for a shape by conv2d_tune or conv2d_select_variant
// (key variant field -1): the default entry point's plan for that shape.
// Never evicted, so a choice stays in force for the rest of the process; at
// most kMaxSelections shapes (a further selection returns
// CONV2D_ERR_UNSUPPORTED and leaves the model's choice in force).
struct Selection {
  PlanKey key;
  int variant;
};
constexpr size_t kMaxSelections = 4096;

std::mutex& plan_cache_mutex() {
  static std::mutex mu;
  return mu;
}
std::vector<PlanEntry>& plan_cache() {
  static std::vector<PlanEntry> cache;
  return cache;
}
std::vector<Selection>& selections() {
  static std::vector<Selection> sel;
  return sel;
}

PlanKey plan_key(const conv2d_params* p, int op, int f16, int variant, int cus) {
  PlanKey key;
  std::memset(&key, 0, sizeof(key));
  key.p = *p;
  key.op = op;
  key.f16 = f16;
  key.variant = variant;
  key.cus = cus;
  return key;
}

bool same_key(const PlanKey& a, const PlanKey& b) { return std::memcmp(&a, &b, sizeof(a)) == 0; }

// Insert a plan as the most recently used entry (callers hold no lock).
void store_plan(const PlanKey& key, const std::vector<LaunchArgs>& launches) {
  std::lock_guard<std::mutex> lock(plan_cache_mutex());
  std::vector<PlanEntry>& cache = plan_cache();
  for (size_t i = 0; i < cache.size(); ++i)
    if (same_key(cache[i].key, key)) {
      cache.erase(cache.begin() + long(i));
      break;
    }
  if (cache.size() >= kPlanCacheSize) cache.erase(cache.begin());
  cache.push_back(PlanEntry{key, launches});
}

// Selected variant of a shape's default plan, or -1 (the model's choice).
int selected_variant(const conv2d_params* p, int op, int f16, int cus) {
  const PlanKey key = plan_key(p, op, f16, -1, cus);
  std::lock_guard<std::mutex> lock(plan_cache_mutex());
  for (const Selection& s : selections())
    if (same_key(s.key, key)) return s.variant;
  return -1;
}

// Make `variant` the default plan's variant for a shape (-1: back to the
// model's choice).
int select_variant(const conv2d_params* p, int op, int f16, int cus, int variant) {
  const PlanKey key = plan_key(p, op, f16, -1, cus);
  std::lock_guard<std::mutex> lock(plan_cache_mutex());
  std::vector<Selection>& sel = selections();
  for (size_t i = 0; i < sel.size(); ++i)
    if (same_key(sel[i].key, key)) {
      if (variant < 0) sel.erase(sel.begin() + long(i));
      else sel[i].variant = variant;
      return CONV2D_OK;
    }
  if (variant < 0) return CONV2D_OK;
  if (sel.size() >= kMaxSelections) return CONV2D_ERR_UNSUPPORTED;
  sel.push_back(Selection{key, variant});
  return CONV2D_OK;
}

// Plan of a shape with `variant` forced, or (variant -1) its default plan:
// the selected variant if there is one, else the model's choice.
int cached_plan(const conv2d_params* p, int op, int f16, int variant, int cus,
                std::vector<LaunchArgs>* out) {
  if (variant < 0) variant = selected_variant(p, op, f16, cus);
  const PlanKey key = plan_key(p, op, f16, variant, cus);
  {
    std::lock_guard<std::mutex> lock(plan_cache_mutex());
    std::vector<PlanEntry>& cache = plan_cache();
    for (size_t i = 0; i < cache.size(); ++i)
      if (same_key(cache[i].key, key)) {
        *out = cache[i].launches;
        if (i + 1 != cache.size()) {   // most recently used goes last
          PlanEntry e = std::move(cache[i]);
          cache.erase(cache.begin() + long(i));
          cache.push_back(std::move(e));
        }
        return CONV2D_OK;
      }
  }
  const int rc = build_plan(p, f16, cus, out, nullptr, variant, nullptr, op);
  if (rc != CONV2D_OK) return rc;
  store_plan(key, *out);
  return CONV2D_OK;
}

// Enqueue a plan's launches on `st` with the caller's buffers.
int enqueue(std::vector<LaunchArgs>& launches, const float* go, const float* w, float* gi,
            hipStream_t st) {
  for (LaunchArgs& la : launches) {
    la.go = go;
    la.w = w;
    la.gi = gi;
    if (la.total_tiles == 0) continue;
    launch_dispatch(la, st, std::make_integer_sequence<int, kNumVariants>());
  }
  return hipGetLastError() == hipSuccess ? CONV2D_OK : CONV2D_ERR_HIP;
}

int launch(const float* go, const float* w, float* gi, const conv2d_params* p, int f16,
           int variant, void* stream, int op = kOpGradInput) {
  int rc = validate_shape(p);
  if (rc != CONV2D_OK) return rc;
  rc = check_pointers(go, w, gi, p, op);
  if (rc != CONV2D_OK) return rc;
  // 1x1, stride 1, unpadded: the GEMM over all images' pixels (forced
  // variants still reach the kernel family)
  const int fwd = op == kOpForward ? 1 : 0;
  if (variant < 0 && pw::pw_route(p, fwd, f16) && pw::pw_applies(p, go, w, gi))
    return pw::pw_launch(go, w, gi, p, f16, stream, fwd, device_cus());
  std::vector<LaunchArgs> launches;
  rc = cached_plan(p, op, f16, variant, device_cus(), &launches);
  if (rc != CONV2D_OK) return rc;
  return enqueue(launches, go, w, gi, static_cast<hipStream_t>(stream));
}

// Tuning: the variants of the path whose modelled makespan is within
// kTuneSpread of the best (at most kTuneCandidates) each run once as a
// warm-up, then kTuneRounds rounds go over all of them in turn, timing
// kTuneReps runs of each with events on the caller's buffers and stream; a
// candidate's time is its fastest round, so a clock that is still rising
// (or a stray slow run) falls on every candidate alike.  The fastest becomes
// the shape's default plan.
constexpr int kTuneCandidates = 8;
constexpr double kTuneSpread = 1.3;
constexpr int kTuneRounds = 3;
constexpr int kTuneReps = 2;

int tune(const float* go, const float* w, float* gi, const conv2d_params* p, int f16,
         void* stream, int* variant_out, int op = kOpGradInput) {
  int rc = validate_shape(p);
  if (rc != CONV2D_OK) return rc;
  rc = check_pointers(go, w, gi, p, op);
  if (rc != CONV2D_OK) return rc;
  const int fwd = op == kOpForward ? 1 : 0;
  if (pw::pw_route(p, fwd, f16) && pw::pw_applies(p, go, w, gi)) {
    // the 1x1 GEMM has no variant to choose: run it once
    rc = pw::pw_launch(go, w, gi, p, f16, stream, fwd, device_cus());
    if (rc != CONV2D_OK) return rc;
    if (hipStreamSynchronize(static_cast<hipStream_t>(stream)) != hipSuccess)
      return CONV2D_ERR_HIP;
    if (variant_out) *variant_out = -1;
    return CONV2D_OK;
  }
  const int cus = device_cus();
  std::vector<std::pair<double, int>> cand;
  for (int v = 0; v < kNumVariants; ++v) {
    if (kVariants[v].f16 != f16) continue;
    double cost = 0.0;
    if (build_plan(p, f16, cus, nullptr, nullptr, v, &cost, op) == CONV2D_OK)
      cand.push_back({cost, v});
  }
  // the model's choice (built here, not through the selection in force)
  std::vector<LaunchArgs> launches;
  rc = build_plan(p, f16, cus, &launches, nullptr, -1, nullptr, op);
  if (rc != CONV2D_OK) return rc;
  int best_v = launches.empty() ? -1 : launches[0].variant;
  std::sort(cand.begin(), cand.end());
  if (cand.size() > size_t(kTuneCandidates)) cand.resize(kTuneCandidates);
  hipStream_t st = static_cast<hipStream_t>(stream);
  std::vector<LaunchArgs> best_plan = launches;
  if (!launches.empty() && cand.size() > 1) {
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
      if (e0) (void)hipEventDestroy(e0);
      return CONV2D_ERR_HIP;
    }
    // the candidates' plans, each run once as a warm-up
    std::vector<std::vector<LaunchArgs>> plans;
    for (const auto& c : cand) {
      if (c.first > kTuneSpread * cand[0].first) break;
      std::vector<LaunchArgs> plan;
      rc = build_plan(p, f16, cus, &plan, nullptr, c.second, nullptr, op);
      if (rc != CONV2D_OK) break;
      rc = enqueue(plan, go, w, gi, st);
      if (rc != CONV2D_OK) break;
      plans.push_back(std::move(plan));
    }
    std::vector<float> fastest(plans.size(), 0.0f);
    for (int round = 0; rc == CONV2D_OK && round < kTuneRounds; ++round)
      for (size_t i = 0; i < plans.size(); ++i) {
        rc = CONV2D_ERR_HIP;
        if (hipEventRecord(e0, st) != hipSuccess) break;
        int r = 0;
        for (; r < kTuneReps; ++r)
          if (enqueue(plans[i], go, w, gi, st) != CONV2D_OK) break;
        if (r < kTuneReps) break;
        float ms = 0.0f;
        if (hipEventRecord(e1, st) != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
            hipEventElapsedTime(&ms, e0, e1) != hipSuccess)
          break;
        rc = CONV2D_OK;
        if (round == 0 || ms < fastest[i]) fastest[i] = ms;
      }
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    if (rc != CONV2D_OK) return rc;
    for (size_t i = 0; i < plans.size(); ++i)
      if (i == 0 || fastest[i] < fastest[0]) {
        fastest[0] = fastest[i];
        best_plan = plans[i];
      }
    best_v = best_plan[0].variant;
  }
  if (best_v >= 0) {
    rc = select_variant(p, op, f16, cus, best_v);
    if (rc != CONV2D_OK) return rc;
    store_plan(plan_key(p, op, f16, best_v, cus), best_plan);
  }
  if (!best_plan.empty()) {
    // leave the output holding the result of the chosen plan
    rc = enqueue(best_plan, go, w, gi, st);
    if (rc != CONV2D_OK) return rc;
  }
  if (variant_out) *variant_out = best_v;
  return CONV2D_OK;
}

// The variant the default entry point of a path uses for a shape now (-1 if
// the shape launches nothing).
int planned_variant(const conv2d_params* p, int f16, int* variant_out, int op = kOpGradInput) {
  if (pw::pw_route(p, op == kOpForward, f16)) {   // the 1x1 GEMM (aligned tensors)
    *variant_out = -1;
    return CONV2D_OK;
  }
  std::vector<LaunchArgs> launches;
  const int rc = cached_plan(p, op, f16, -1, device_cus(), &launches);
  if (rc != CONV2D_OK) return rc;
  *variant_out = launches.empty() ? -1 : launches[0].variant;
  return CONV2D_OK;
}

}  // namespace c2b

extern "C" int conv2d_grad_input(const float* grad_out, const float* weight, float* grad_input,
                                 const conv2d_params* p, void* stream) {
  return c2b::launch(grad_out, weight, grad_input, p, 0, -1, stream);
}

extern "C" int conv2d_grad_input_f16(const float* grad_out, const float* weight,
                                     float* grad_input, const conv2d_params* p, void* stream) {
  return c2b::launch(grad_out, weight, grad_input, p, 1, -1, stream);
}

extern "C" int conv2d_grad_input_variant(const float* grad_out, const float* weight,
                                         float* grad_input, const conv2d_params* p, int variant,
                                         void* stream) {
  if (p == nullptr) return CONV2D_ERR_NULL_PTR;
  if (variant < 0 || variant >= c2b::kNumVariants) return CONV2D_ERR_UNSUPPORTED;
  return c2b::launch(grad_out, weight, grad_input, p, c2b::kVariants[variant].f16, variant,
                     stream);
}

extern "C" int conv2d_tune(const float* grad_out, const float* weight, float* grad_input,
                           const conv2d_params* p, int f16, void* stream, int* variant_out) {
  return c2b::tune(grad_out, weight, grad_input, p, f16 ? 1 : 0, stream, variant_out);
}

extern "C" int conv2d_planned_variant(const conv2d_params* p, int f16, int* variant_out) {
  if (p == nullptr || variant_out == nullptr) return CONV2D_ERR_NULL_PTR;
  const int rc = c2b::validate_shape(p);
  if (rc != CONV2D_OK) return rc;
  return c2b::planned_variant(p, f16 ? 1 : 0, variant_out);
}

namespace c2b {
// A variant for a shape's default plan: -1, or a variant of the path that
// tiles the shape.
int select_checked(const conv2d_params* p, int op, int f16, int variant) {
  if (p == nullptr) return CONV2D_ERR_NULL_PTR;
  int rc = validate_shape(p);
  if (rc != CONV2D_OK) return rc;
  if (variant < -1 || variant >= kNumVariants) return CONV2D_ERR_UNSUPPORTED;
  // the 1x1 GEMM has no variant to choose (-1 still clears a choice)
  if (pw::pw_route(p, op == kOpForward, f16) && variant >= 0) return CONV2D_ERR_UNSUPPORTED;
  const int cus = device_cus();
  if (variant >= 0) {
    rc = build_plan(p, f16, cus, nullptr, nullptr, variant, nullptr, op);
    if (rc != CONV2D_OK) return rc;
  }
  return select_variant(p, op, f16, cus, variant);
}
}  // namespace c2b

extern "C" int conv2d_select_variant(const conv2d_params* p, int f16, int variant) {
  return c2b::select_checked(p, c2b::kOpGradInput, f16 ? 1 : 0, variant);
}

namespace c2b {
namespace fg {   // forward_gemm.hip: the few-input-channel forward
bool fg_applies(const conv2d_params* p, int f16);
int fg_launch(const float* x, const float* w, float* y, const conv2d_params* p, void* stream);
}  // namespace fg
}  // namespace c2b

extern "C" int conv2d_forward(const float* x, const float* weight, float* y,
                              const conv2d_params* p, void* stream) {
  // fewer than 16 input channels: the im2col GEMM over (ci, kh, kw), which
  // pads no contraction channel (forced variants still reach this family)
  if (c2b::fg::fg_applies(p, 0)) {
    int rc = c2b::validate_shape(p);
    if (rc == CONV2D_OK) rc = c2b::check_pointers(x, weight, y, p, c2b::kOpForward);
    return rc == CONV2D_OK ? c2b::fg::fg_launch(x, weight, y, p, stream) : rc;
  }
  return c2b::launch(x, weight, y, p, 0, -1, stream, c2b::kOpForward);
}

extern "C" int conv2d_forward_f16(const float* x, const float* weight, float* y,
                                  const conv2d_params* p, void* stream) {
  return c2b::launch(x, weight, y, p, 1, -1, stream, c2b::kOpForward);
}

extern "C" int conv2d_forward_variant(const float* x, const float* weight, float* y,
                                      const conv2d_params* p, int variant, void* stream) {
  if (p == nullptr) return CONV2D_ERR_NULL_PTR;
  if (variant < 0 || variant >= c2b::kNumVariants) return CONV2D_ERR_UNSUPPORTED;
  return c2b::launch(x, weight, y, p, c2b::kVariants[variant].f16, variant, stream,
                     c2b::kOpForward);
}

extern "C" int conv2d_tune_forward(const float* x, const float* weight, float* y,
                                   const conv2d_params* p, int f16, void* stream,
                                   int* variant_out) {
  // shapes on the im2col GEMM have no variant to choose: run it once
  if (c2b::fg::fg_applies(p, f16 ? 1 : 0)) {
    const int rc = conv2d_forward(x, weight, y, p, stream);
    if (rc != CONV2D_OK) return rc;
    if (hipStreamSynchronize(static_cast<hipStream_t>(stream)) != hipSuccess)
      return CONV2D_ERR_HIP;
    if (variant_out) *variant_out = -1;
    return CONV2D_OK;
  }
  return c2b::tune(x, weight, y, p, f16 ? 1 : 0, stream, variant_out, c2b::kOpForward);
}

extern "C" int conv2d_planned_forward_variant(const conv2d_params* p, int f16, int* variant_out) {
  if (p == nullptr || variant_out == nullptr) return CONV2D_ERR_NULL_PTR;
  const int rc = c2b::validate_shape(p);
  if (rc != CONV2D_OK) return rc;
  if (c2b::fg::fg_applies(p, f16 ? 1 : 0)) {   // the im2col GEMM, not a variant
    *variant_out = -1;
    return CONV2D_OK;
  }
  return c2b::planned_variant(p, f16 ? 1 : 0, variant_out, c2b::kOpForward);
}

extern "C" int conv2d_select_forward_variant(const conv2d_params* p, int f16, int variant) {
  // a shape on the im2col GEMM has no variant to choose (-1 still clears one)
  if (c2b::fg::fg_applies(p, f16 ? 1 : 0) && variant >= 0) return CONV2D_ERR_UNSUPPORTED;
  return c2b::select_checked(p, c2b::kOpForward, f16 ? 1 : 0, variant);
}
