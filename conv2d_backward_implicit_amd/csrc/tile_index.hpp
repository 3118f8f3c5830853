// Index arithmetic of the input-gradient kernels, shared by the kernels and
// by the host-side index checker (index_check.hip), so that the checker
// replays exactly the addresses the kernels form.
//
// Terms (see plan.hpp for the stride-residue classes):
//  * tile: 64 input channels x up to 256 consecutive pixels of one band of
//    one class sub-image of one image;
//  * window: the grad_out rows/columns a tile's pixels read through all taps
//    of the class, R rows of roww elements, staged in LDS per output channel;
//  * stage: CK output channels x up to TAPS taps of the class.
#pragma once

#include "plan.hpp"

#if defined(__HIP__) || defined(__HIPCC__)
#include <hip/hip_runtime.h>
#define C2B_HD __host__ __device__ __forceinline__
#else
#define C2B_HD inline
#endif

namespace c2b {

constexpr int kThreads = 256;

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

// Index of the class of workgroup `bid` within the launch.
C2B_HD int phase_of(const LaunchArgs& a, int bid) {
  int pi = 0;
  for (int i = 1; i < a.nphases; ++i)
    if (bid >= a.ph[i].tile_begin) pi = i;
  return pi;
}

// Tile of a workgroup.  Inside a class, the workgroups whose index is
// x mod 8 (one XCD: the dispatcher deals workgroups round-robin over the 8
// XCDs) take one contiguous run of tiles, channel tile fastest, so tiles
// that share grad_out rows and weights share that XCD's L2.
// ck: output channels per stage (0: the class's own stage depth, P.ckr).
template <int MT>
C2B_HD TileCtx decode_tile(const LaunchArgs& a, int bid, int ck) {
  TileCtx c;
  c.P = a.ph[phase_of(a, bid)];
  const PhaseDesc& P = c.P;
  int t;
  {
    const int l = bid - P.tile_begin, T = P.tiles;
    const int q = T >> 3, r = T & 7, x = l & 7, k = l >> 3;
    t = x * q + imin(x, r) + k;
  }
  const int ciblk = t % a.ciblocks;
  t /= a.ciblocks;
  const int ptile = t % P.ptiles;
  t /= P.ptiles;
  c.band = t % P.nbands;
  c.n = t / P.nbands;
  c.ci0 = ciblk * MT;
  const int bandpix = P.hp * P.wb;
  c.p0 = ptile * P.ntv;
  const int pend = imin(c.p0 + P.ntv, bandpix);
  c.npx = pend - c.p0;
  c.ntaps = P.th * P.tw;
  if (ck == 0) ck = P.ckr;
  c.nstages = c.ntaps > 0 ? ((a.Co + ck - 1) / ck) * P.ngroups : 0;
  c.i_start = c.p0 / P.wb;
  c.R = (pend - 1) / P.wb - c.i_start + P.th;
  c.roww = P.wb + P.tw - 1;
  c.oh_base = c.i_start + P.ch - (P.th - 1);
  c.ow_base = c.band * P.wb + P.cw - (P.tw - 1);
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
  return (dr + P.th - 1) * c.roww + jb + P.tw - 1;
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
  return (P.rh + a.S * j) * a.KW + (P.rw + a.S * l);
}

// Stage st -> (first output channel, tap group).
C2B_HD void stage_split(const TileCtx& c, int ck, int st, int* co0, int* g) {
  const int cchunk = st / c.P.ngroups;
  *g = st - cchunk * c.P.ngroups;
  *co0 = cchunk * ck;
}

// Weight staging cell e = (t, cg, ci), t-major, ci fastest; each cell holds
// CPC consecutive output channels (1 for fp32, 8 for f16).  Returns the offset
// of weight[cg*CPC, ci0 + ci, tap] relative to the stage's first output
// channel, or -1 if the cell is padding (no tap / channel beyond Ci).
template <int MT, int NCG, int TAPS, int CPC>
C2B_HD int weight_cell_offset(const TileCtx& c, const LaunchArgs& a, int e, int g) {
  constexpr int AE = TAPS * NCG * MT;
  if (e >= AE) return -1;
  const int t = e / (NCG * MT);
  const int cg = (e / MT) % NCG;
  const int ci = e % MT;
  const int tap = g * TAPS + t;
  if (tap >= c.ntaps || c.ci0 + ci >= a.Ci) return -1;
  return (cg * CPC * a.Ci + c.ci0 + ci) * (a.KH * a.KW) + tap_kidx(c.P, a, tap);
}

// First output channel (relative to the stage) of weight cell e.
template <int MT, int NCG, int CPC>
C2B_HD int weight_cell_channel(int e) { return ((e / MT) % NCG) * CPC; }

// LDS index of weight cell e: cells are stored [t][cg][pitch], ci fastest.
template <int MT, int NCG, int PITCH>
C2B_HD int weight_cell_lds(int e) {
  const int t = e / (NCG * MT);
  const int cg = (e / MT) % NCG;
  const int ci = e % MT;
  return (t * NCG + cg) * PITCH + ci;
}

// Compile-time geometry of one kernel instantiation.
//   fp32: one output channel per LDS cell, 2 k values per matrix instruction,
//         A rows padded by 32 floats so the two half-waves of a read sit 32
//         banks apart;
//   f16:  8 output channels per 16-byte cell, 16 k values per instruction.
template <bool F16, int MT, int CK, int TAPS, int SLAB>
struct KernelGeom {
  static constexpr int kCPC = F16 ? 8 : 1;               // channels per cell
  static constexpr int kKPerStep = F16 ? 16 : 2;         // k per instruction
  static constexpr int kNCG = CK / kCPC;                 // cell groups / stage
  static constexpr int kKSteps = CK / kKPerStep;         // k-steps per tap
  static constexpr int kPitch = F16 ? MT : MT + 32;      // A row pitch, cells
  static constexpr int kHS = (SLAB + kThreads - 1) / kThreads;  // window slots
  static constexpr int kAE = TAPS * kNCG * MT;           // A cells per stage
  static constexpr int kWS = (kAE + kThreads - 1) / kThreads;   // A slots
  static constexpr int kLdsA = TAPS * kNCG * kPitch;     // A cells in LDS
  static constexpr int kLdsH = kNCG * SLAB;              // window cells in LDS
  static_assert(CK % (2 * kCPC) == 0, "a k-step takes one cell group per half-wave");
  static_assert(kKSteps * 2 == kNCG, "k-steps cover the stage's cell groups");
};

// ---------------------------------------------------------------------------
// fp32 kernel family (8 waves, 16x16x4 fp32 matrix instructions).
//   wave w: channel group mg = w % WM (16 input channels), pixel group
//   ng = w / WM (WN groups); lane: k group g = lane / 16, c16 = lane % 16;
//   block b of the wave covers tile-local pixels (b*WN + ng)*16 + [0, 16);
//   k-step q (0..3) of a tap: lane group g supplies output channel 4g + q.
// A stage is 16 output channels x up to tg taps.  LDS (two buffers of each,
// at fixed offsets):
//   window  [quad cq = 0..3][slot][4 channels]  (16*slots floats): a lane
//           reads its group's 4 channels with one 16-byte read, 16 lanes read
//           16 consecutive 16-byte cells (every bank once), and a tap shift
//           is a plain subtraction of slots;
//   weights [co][ci][t] with channel pitch cp (= 4 mod 16 floats, so the
//           four lane groups, 4*cp apart, sit 16 banks apart).
// Both are filled by buffer loads that write LDS directly: each
// wave-instruction fills 64 consecutive floats, which here come from 16
// consecutive pixels of 4 channels, or from consecutive weights of one
// channel -- a few cache lines per instruction.
template <int WM, int WN, int NBW>
struct F32Geom {
  static constexpr int kThreads = 64 * WM * WN;
  static constexpr int kWN = WN;                      // waves along pixels
  static constexpr int kMT = 16 * WM;                 // channels per tile
  static constexpr int kNTL = 16 * NBW * WN;          // pixel lanes per tile
  // copy wave-instructions per wave and stage: every one is issued; cells
  // past the stage's window or weights read 0 and land inside the buffer
  static constexpr int kHS = (kF32WinFloats + kThreads - 1) / kThreads;
  static constexpr int kWS = (kF32WtFloats + kThreads - 1) / kThreads;
  static_assert(kF32WinFloats % 64 == 0 && kF32WtFloats % 64 == 0, "whole instructions");
};

// Tile-local pixel of block b of pixel group ng, lane c16.
C2B_HD int f32_local(int b, int ng, int c16, int wn) { return (b * wn + ng) * 16 + c16; }

// Window cell f = (cq*slots + slot)*4 + c of a stage: grad_out offset
// ch*OH*OW + oh*OW + ow (ch = 4cq + c) relative to the stage's first channel,
// or -1 if the cell is padding (outside the image or the window).
C2B_HD int f32_window_cell(const TileCtx& c, const LaunchArgs& a, int f) {
  const int slots = c.P.slabr;
  if (c.ntaps == 0 || f >= kF32StageCh * slots) return -1;
  const int cq = fast_div(f, c.P.m_slots4);
  const int r = f - cq * 4 * slots;
  const int slot = r >> 2, ch = 4 * cq + (r & 3);
  const int off = window_slot_offset(c, a, slot);
  return off < 0 ? -1 : ch * (a.OH * a.OW) + off;
}

// Weight cell e = co*cp + ci*tg + t of stage tap group `grp`: offset of
// weight[co, ci0 + ci, tap] relative to the stage's first output channel,
// or -1 if padding.
template <int MT>
C2B_HD int f32_weight_cell(const TileCtx& c, const LaunchArgs& a, int e, int grp) {
  const PhaseDesc& P = c.P;
  if (c.ntaps == 0 || e >= kF32StageCh * P.cp) return -1;
  const int co = fast_div(e, P.m_cp);
  const int r = e - co * P.cp;
  if (r >= MT * P.tg) return -1;
  const int ci = fast_div(r, P.m_tg), t = r - ci * P.tg;
  const int tap = grp * P.tg + t;
  if (tap >= c.ntaps || c.ci0 + ci >= a.Ci) return -1;
  return (co * a.Ci + c.ci0 + ci) * (a.KH * a.KW) + tap_kidx(P, a, tap);
}

// Accumulator register r of lane half h in a 32x32 block holds block row
// 8*(r/4) + 4*h + r%4 (column = lane mod 32) -- the C/D layout of the
// 32x32 matrix instructions used here.
C2B_HD int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

}  // namespace c2b
