// Index arithmetic of the implicit-GEMM kernels, shared by the kernels and
// by the host-side index checker (index_check.hip), so that the checker
// replays exactly the addresses the kernels form.
//
// Terms (see plan.hpp for the stride-residue classes, the stages and the
// forward launches, whose roles are named here as on the input-gradient
// path):
//  * tile: MT input channels x up to NTL consecutive pixels of one band of
//    one class sub-image of one image;
//  * window: the grad_out rows/columns a tile's pixels read through all taps
//    of the class, R rows of roww elements, staged in LDS per output channel;
//  * stage: 16*cg output channels x up to tg taps of the class.
#pragma once

#include "plan.hpp"

#if defined(__HIP__) || defined(__HIPCC__)
#include <hip/hip_runtime.h>
#define C2B_HD __host__ __device__ __forceinline__
#else
#define C2B_HD inline
#endif

namespace c2b {

// Everything one workgroup derives from its index.
struct TileCtx {
  PhaseDesc P;
  int n, band, ci0, p0, npx;
  int i_start, R, roww, oh_base, ow_base;
  int ntaps, nstages;
};

C2B_HD int imin(int a, int b) { return a < b ? a : b; }

// floor(n / d) as one multiply-high: m = ceil(2^31 / d) (fast_div_magic),
// exact whenever n * d < 2^31 (n*m/2^31 exceeds n/d by less than n/2^31,
// which cannot reach the next multiple of 1/d).  The planner bounds every
// numerator it is used with.
C2B_HD int fast_div(int n, uint32_t m) {
#if defined(__HIP_DEVICE_COMPILE__)
  return int(__umulhi(uint32_t(n) << 1, m));
#else
  return int((uint64_t(uint32_t(n) << 1) * m) >> 32);
#endif
}

C2B_HD uint32_t fast_div_magic(uint32_t d) {
  return uint32_t(((uint64_t(1) << 31) + d - 1) / d);
}

// Contiguous runs per XCD: the dispatcher deals workgroups round-robin over
// the 8 XCDs, so of `count` workgroups the ones with l = x mod 8 (one XCD)
// take the x-th of 8 contiguous runs of the tiles.
C2B_HD int xcd_run(int l, int count) {
  const int q = count >> 3, r = count & 7, x = l & 7, k = l >> 3;
  return x * q + imin(x, r) + k;
}

// Tile of a workgroup.  Each XCD takes contiguous runs of tiles, channel
// tile fastest, so that tiles that share grad_out rows and weights share
// that XCD's L2.  Classes (stride > 1) occupy consecutive workgroup ranges,
// heaviest first, and each class's range is dealt over the XCDs on its own.
// With `ilv` (classes of equal stage counts) the whole launch is dealt at
// once, image by image and inside an image class by class: the classes of
// one image read the same grad_out planes, which then stay in the XCD's L2
// while they all run, instead of coming back from memory once per class.
C2B_HD TileCtx decode_tile(const LaunchArgs& a, int bid) {
  TileCtx c;
  int pi = 0, t;
  if (a.ilv) {
    const int u = xcd_run(bid, a.total_tiles);
    const int n = u / a.img_total, v = u - n * a.img_total;
    for (int i = 1; i < a.nphases; ++i)
      if (v >= a.ph[i].img_begin) pi = i;
    t = n * a.ph[pi].img_tiles + (v - a.ph[pi].img_begin);
  } else {
    // class pi's workgroups start at N * img_begin (its tiles run image by
    // image)
    for (int i = 1; i < a.nphases; ++i)
      if (bid >= a.N * a.ph[i].img_begin) pi = i;
    t = xcd_run(bid - a.N * a.ph[pi].img_begin, a.ph[pi].tiles);
  }
  c.P = a.ph[pi];
  const PhaseDesc& P = c.P;
  const int ciblk = t % a.ciblocks;
  t /= a.ciblocks;
  const int ptile = t % P.ptiles;
  t /= P.ptiles;
  c.band = t % P.nbands;
  c.n = t / P.nbands;
  c.ci0 = ciblk * a.cit;
  const int bandpix = P.hp * P.wb;
  c.p0 = ptile * P.ntv;
  const int pend = imin(c.p0 + P.ntv, bandpix);
  c.npx = pend - c.p0;
  // cm: row taps only; multi-class: every kernel tap, in the weight's order
  c.ntaps = a.cm ? P.th : P.mct > 0 ? P.mct : P.th * P.tw;
  c.nstages = c.ntaps > 0 ? P.nchunks * P.ngroups : 0;
  c.i_start = c.p0 / P.wb;
  // window: the source rows / columns of the tile's rows and band through
  // every tap, sampled every ss (1 except on forward launches)
  c.R = ((pend - 1) / P.wb - c.i_start) * P.ss + P.th;
  c.roww = (P.wb - 1) * P.ss + P.tw;
  c.oh_base = c.i_start * P.ss + P.ch - (P.th - 1);
  c.ow_base = c.band * P.wb * P.ss + P.cw - (P.tw - 1);
  return c;
}

// Offset (oh*OW + ow) within a grad_out channel plane of window slot f, or
// -1 if the slot is outside the image (zero padding) or outside the window.
C2B_HD int window_slot_offset(const TileCtx& c, const LaunchArgs& a, int f) {
  if (c.ntaps == 0 || f >= c.R * c.roww) return -1;
  const int r = fast_div(f, c.P.m_roww);
  const int col = f - r * c.roww;
  const int oh = c.oh_base + r;
  const int ow = c.ow_base + col;
  if ((unsigned)oh < (unsigned)a.OH && (unsigned)ow < (unsigned)a.OW) return oh * a.OW + ow;
  return -1;
}

// Window slot a tile-local pixel reads for the class's first tap (j = l = 0);
// tap (j, l) reads j*roww + l slots before it.  Lanes past the tile's pixels
// get a slot whose tap offsets all stay inside the window.
C2B_HD int window_base(const TileCtx& c, int local) {
  const PhaseDesc& P = c.P;
  if (c.ntaps == 0) return 0;
  if (local >= c.npx) return (P.th - 1) * c.roww + P.tw - 1;
  // row within the tile's first row: (p0 mod wb + local) / wb
  const int q0 = c.p0 - c.i_start * P.wb + local;
  const int dr = fast_div(q0, P.m_wb);
  const int jb = q0 - dr * P.wb;
  return (dr * P.ss + P.th - 1) * c.roww + jb * P.ss + P.tw - 1;
}

// cm (column taps in the matrix rows): the tile's lanes are the points
// (r, u) of its class rows r < R - th + 1 and window columns u < roww, in
// row-major order; the window slot a point reads for row tap j = 0.  Lanes
// past the points get a slot whose row-tap offsets stay inside the window.
C2B_HD int cm_points(const TileCtx& c) { return (c.R - c.P.th + 1) * c.roww; }
C2B_HD int window_base_cm(const TileCtx& c, int local) {
  const PhaseDesc& P = c.P;
  if (c.ntaps == 0) return 0;
  if (local >= cm_points(c)) return (P.th - 1) * c.roww;
  const int r = fast_div(local, P.m_roww);
  return (r + P.th - 1) * c.roww + (local - r * c.roww);
}

// Multi-class tiles (Variant::mc): the window position (dr, jb) of a
// tile-local grid point, as the slot dr * roww + jb; class k's pixel there
// reads slot + e * roww + f - (j * roww + l) at its tap (j, l).  Lanes past
// the tile's points get slot 0, from which every class's taps stay inside
// the window (0 <= e - j, f - l and e - j < R, f - l < roww).
C2B_HD int window_pixel(const TileCtx& c, int local) {
  const PhaseDesc& P = c.P;
  if (c.ntaps == 0 || local >= c.npx) return 0;
  const int q0 = c.p0 - c.i_start * P.wb + local;
  const int dr = fast_div(q0, P.m_wb);
  return dr * c.roww + (q0 - dr * P.wb);
}

// Plane offset ih*W + iw of class k's pixel at a tile-local grid point of a
// multi-class tile, or -1 (past the tile's points or the class's extent).
C2B_HD int mc_output_offset(const TileCtx& c, const LaunchArgs& a, const MCClass& k,
                            int local) {
  const PhaseDesc& P = c.P;
  if (local >= c.npx) return -1;
  const int q0 = c.p0 - c.i_start * P.wb + local;
  const int dr = fast_div(q0, P.m_wb);
  const int ip = c.i_start + dr;
  const int jj = c.band * P.wb + (q0 - dr * P.wb);
  if (ip >= k.hp || jj >= k.wp) return -1;
  return (k.ih0 + 2 * ip) * a.W + k.iw0 + 2 * jj;
}

// Multi-class stores: the two classes of row class hk (mcls[2 hk] and
// mcls[2 hk + 1], whose first columns iw0 are 0 and 1) hold, at a grid point
// (i', j'), the two adjacent pixels (ih, 2j') and (ih, 2j' + 1) of input row
// ih = ih0 + 2i'.  Fills the row and the even column and which of the pair
// lie inside their class; false past the tile's points or the rows.
C2B_HD bool mc_pair_pixel(const TileCtx& c, const LaunchArgs& a, int hk, int local, int* ih,
                          int* col0, bool* even_ok, bool* odd_ok) {
  const PhaseDesc& P = c.P;
  if (local >= c.npx) return false;
  const MCClass& k0 = a.mcls[2 * hk];
  const MCClass& k1 = a.mcls[2 * hk + 1];
  const int q0 = c.p0 - c.i_start * P.wb + local;
  const int dr = fast_div(q0, P.m_wb);
  const int ip = c.i_start + dr;
  const int jj = c.band * P.wb + (q0 - dr * P.wb);
  if (ip >= k0.hp) return false;
  *ih = k0.ih0 + 2 * ip;
  *col0 = 2 * jj;
  const bool first_even = k0.iw0 == 0;   // which class holds the even column
  *even_ok = jj < (first_even ? k0.wp : k1.wp);
  *odd_ok = jj < (first_even ? k1.wp : k0.wp);
  return *even_ok || *odd_ok;
}

// Window slot offset of tap (j, l) relative to window_base.
C2B_HD int tap_window_offset(const TileCtx& c, int j, int l) { return -(j * c.roww + l); }

// Plane offset ih*W + iw of the grad_input pixel of a tile-local lane, or -1.
C2B_HD int output_offset(const TileCtx& c, const LaunchArgs& a, int local) {
  const PhaseDesc& P = c.P;
  if (local >= c.npx) return -1;
  const int q0 = c.p0 - c.i_start * P.wb + local;
  const int dr = fast_div(q0, P.m_wb);
  const int ip = c.i_start + dr;
  const int jj = c.band * P.wb + (q0 - dr * P.wb);
  if (jj >= P.wp) return -1;
  const int ih = P.ih0 + a.S * ip;
  const int iw = P.iw0 + a.S * jj;
  return ih * a.W + iw;
}

// Flat weight index kh*KW + kw of the tap-th tap of the class.
C2B_HD int tap_kidx(const PhaseDesc& P, const LaunchArgs& a, int tap) {
  const int j = fast_div(tap, P.m_tw);
  const int l = tap - j * P.tw;
  return (P.rh + P.kstep * j) * a.KW + (P.rw + P.kstep * l);
}

// Stage st -> (first output channel, tap group); tap-group-major.
C2B_HD void stage_split(const TileCtx& c, int st, int* co0, int* grp) {
  *grp = st / c.P.nchunks;
  *co0 = (st - *grp * c.P.nchunks) * 16 * c.P.cg;
}

// ---------------------------------------------------------------------------
// Kernel geometry.
//   wave w: channel group mg = w % WM, pixel group ng = w / WM; lane: k group
//   g = lane / 16, c16 = lane % 16.  Channel block m of the wave covers input
//   channels (mg*MB + m)*16 + [0, 16); pixel block b covers tile-local pixels
//   (b*WN + ng)*16 + [0, 16).  In every unit (16 output channels at one tap)
//   lane group g supplies output channels 4g .. 4g+3 of the unit's group.
// A stage buffer (SF floats, two of them at fixed offsets) holds:
//   window  [quad cq < 4cg][slot < slots][4 channels] at float 0: a lane
//           reads its 4 channels of one slot with one 16-byte read; slots is
//           a multiple of 16, so the four lane groups sit a multiple of
//           256 bytes apart, and a tap shift is a plain subtraction of slots;
//   weights [quad cq][ci < MT][t < pt][4 channels] at float wfl, quads qp
//           floats apart (a multiple of 64): a lane reads the 4 channels of
//           one (ci, tap) with one 16-byte read; pt is odd, so the 16 lanes
//           of a group (consecutive ci) hit 16 disjoint sets of 4 banks.
// Both are filled by copy batches (below): coalesced loads into registers,
// then one 16-byte LDS write per lane.
template <int WM, int WN, int MB, int NBW, int SF>
struct MMGeom {
  static constexpr int kThreads = 64 * WM * WN;
  static constexpr int kMT = 16 * WM * MB;            // channels per tile
  static constexpr int kNTL = 16 * NBW * WN;          // pixel lanes per tile
  static constexpr int kSF = SF;                      // floats per stage buffer
  static constexpr int kWaves = WM * WN;
  // copy batches per wave and stage (the planner only picks stage shapes
  // whose batches fit: at most kWaves * kBatches of them)
  static constexpr int kBatches = (SF / 256 + kWaves - 1) / kWaves;
  static_assert(SF % 256 == 0, "whole copy batches");
};

// Tile-local pixel of block b of pixel group ng, lane c16.
C2B_HD int mm_local(int b, int ng, int c16, int wn) { return (b * wn + ng) * 16 + c16; }

// Tile-local input channel of block m of channel group mg, lane c16.
C2B_HD int mm_channel(int m, int mg, int c16, int mb) { return (mg * mb + m) * 16 + c16; }

// Window cell f = (cq*slots + slot)*4 + c of a stage buffer: grad_out offset
// ch*OH*OW + oh*OW + ow (ch = 4cq + c) relative to the stage's first output
// channel, or -1 if the cell is padding (outside the image or the window).
C2B_HD int mm_window_cell(const TileCtx& c, const LaunchArgs& a, int f) {
  const PhaseDesc& P = c.P;
  if (c.ntaps == 0 || f >= P.wfl) return -1;
  const int cq = fast_div(f, P.m_slots4);
  const int r = f - cq * 4 * P.slots;
  const int slot = r >> 2, ch = 4 * cq + (r & 3);
  const int off = window_slot_offset(c, a, slot);
  return off < 0 ? -1 : ch * (a.OH * a.OW) + off;
}

// Offset within one output channel's weight row (ci*kH*kW + kh*kW + kw) of
// matrix row m at tap t of tap group `grp`, or -1 if that cell is padding.
// Matrix row m is input channel ci0 + m; with cm it is input channel
// ci0 + m / twm at column tap m mod twm, and the taps are the row taps.
template <int MT, bool CM>
C2B_HD int weight_source(const TileCtx& c, const LaunchArgs& a, int m, int t, int grp) {
  const PhaseDesc& P = c.P;
  if (c.ntaps == 0 || m >= MT || t >= P.tg) return -1;
  const int tap = grp * P.tg + t;
  if (tap >= c.ntaps) return -1;
  int ci, kidx;
  if (P.mct > 0) {   // multi-class: tap t of the stage is kernel tap t
    ci = c.ci0 + m;
    kidx = tap;
  } else if (CM) {
    const int cl = m / a.twm, l = m - cl * a.twm;
    if (l >= P.tw || cl >= a.cit) return -1;
    ci = c.ci0 + cl;
    kidx = (P.rh + P.kstep * tap) * a.KW + (P.rw + P.kstep * l);
  } else {
    ci = c.ci0 + m;
    kidx = tap_kidx(P, a, tap);
  }
  if (ci >= a.Ci) return -1;
  return ci * a.wsm + kidx;
}

// Weight cell e = cq*qp + (m*pt + t)*4 + c (e counted from the start of the
// weight region) of tap group `grp`: offset of the weight of contraction
// channel 4cq + c at matrix row m, tap grp*tg + t (weight_source), relative
// to the stage's first contraction channel, or -1 if the cell is padding.
template <int MT, bool CM>
C2B_HD int mm_weight_cell(const TileCtx& c, const LaunchArgs& a, int e, int grp) {
  const PhaseDesc& P = c.P;
  if (c.ntaps == 0 || e < 0 || e >= 4 * P.cg * P.qp) return -1;
  const int cq = fast_div(e, P.m_qp);
  const int r = e - cq * P.qp;
  const int m = fast_div(r, P.m_pt4);
  const int r2 = r - m * 4 * P.pt;
  const int t = r2 >> 2, co = 4 * cq + (r2 & 3);
  const int src = weight_source<MT, CM>(c, a, m, t, grp);
  if (src < 0) return -1;
  return co * a.wsk + src;
}

// ---------------------------------------------------------------------------
// Copy batches.  A stage buffer's window holds 4*cg channel quads of `slots`
// slots (4 channels each); its weights hold 4*cg quads of qp/4 (ci, tap)
// pairs (4 output channels each).  A batch fills 64 consecutive slots (a
// window block) or pairs (a weight block) of one quad: lane l loads the 4
// channels of slot / pair 64*block + l with 4 loads, one per channel -- the
// 64 lanes of a load read consecutive grad_out pixels of one row segment,
// or consecutive taps of consecutive input channels -- and stores them to
// LDS with one 16-byte write.  Blocks [0, WB) are window blocks, [WB, WB+PB)
// weight blocks; batch k of a stage is block k mod (WB+PB) of quad
// k / (WB+PB), and wave w copies batches w, w + waves, w + 2*waves, ...
// A lane's source offset depends on the quad only through a per-channel
// constant (a grad_out plane, or a weight row), added to a per-lane offset.
// Padding lanes (outside the image or the window, past the tap group or the
// tile's channels) get kPadOffset: 2^31 plus any channel constant (below
// 2^31, as the planner bounds a stage's byte ranges) stays at or beyond every
// buffer resource's range, so such loads return 0.
constexpr uint32_t kPadOffset = 0x80000000u;

C2B_HD int window_blocks(const PhaseDesc& P) { return (P.slots + 63) / 64; }
C2B_HD int weight_blocks(const PhaseDesc& P) { return (P.qp / 4 + 63) / 64; }
C2B_HD int copy_blocks(const PhaseDesc& P) { return window_blocks(P) + weight_blocks(P); }
C2B_HD int stage_batches(const PhaseDesc& P) { return 4 * P.cg * copy_blocks(P); }

// Batch k -> (block, quad).
C2B_HD void batch_split(const PhaseDesc& P, int k, int* block, int* quad) {
  *quad = fast_div(k, P.m_blocks);
  *block = k - *quad * copy_blocks(P);
}

// Byte offset, within a grad_out channel plane, of the pixel of window slot
// 64*block + lane (kPadOffset if padding).
C2B_HD uint32_t window_lane_offset(const TileCtx& c, const LaunchArgs& a, int block, int lane) {
  const PhaseDesc& P = c.P;
  const int slot = 64 * block + lane;
  if (c.ntaps == 0 || slot >= c.R * c.roww) return kPadOffset;
  const int r = fast_div(slot, P.m_roww);
  const int oh = c.oh_base + r, ow = c.ow_base + (slot - r * c.roww);
  if ((unsigned)oh >= (unsigned)a.OH || (unsigned)ow >= (unsigned)a.OW) return kPadOffset;
  return uint32_t((oh * a.OW + ow) * 4);
}

// Byte offset, within a weight row of one output channel, of weight pair
// 64*wblock + lane (matrix row, tap) of tap group `grp` (kPadOffset if
// padding).
template <int MT, bool CM>
C2B_HD uint32_t weight_lane_offset(const TileCtx& c, const LaunchArgs& a, int wblock, int lane,
                                   int grp) {
  const PhaseDesc& P = c.P;
  if (c.ntaps == 0) return kPadOffset;
  const int pr = 64 * wblock + lane;
  const int m = fast_div(pr, P.m_pt);
  const int src = weight_source<MT, CM>(c, a, m, pr - m * P.pt, grp);
  return src < 0 ? kPadOffset : uint32_t(src * 4);
}

// Bytes between consecutive contraction channels: source planes, or weights.
C2B_HD uint32_t window_channel_bytes(const LaunchArgs& a) { return uint32_t(4 * a.OH * a.OW); }
C2B_HD uint32_t weight_channel_bytes(const LaunchArgs& a) { return uint32_t(4 * a.wsk); }

// Stage-buffer float of the 16-byte LDS write of lane `lane` of a batch, or
// -1 if the lane is past its quad's slots / pairs (no write).
C2B_HD int batch_lds_float(const PhaseDesc& P, int block, int quad, int lane) {
  const int WB = window_blocks(P);
  if (block < WB) {
    const int slot = 64 * block + lane;
    return slot < P.slots ? (quad * P.slots + slot) * 4 : -1;
  }
  const int pr = 64 * (block - WB) + lane;
  return pr < P.qp / 4 ? P.wfl + quad * P.qp + pr * 4 : -1;
}

}  // namespace c2b
