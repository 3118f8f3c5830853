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
template <int MT, int CK>
C2B_HD TileCtx decode_tile(const LaunchArgs& a, int bid) {
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
  c.nstages = c.ntaps > 0 ? ((a.Co + CK - 1) / CK) * P.ngroups : 0;
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
  const int r = f / c.roww;
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
  const int q = c.p0 + local;
  const int ip = q / P.wb;
  const int jb = q - ip * P.wb;
  return (ip - c.i_start + P.th - 1) * c.roww + jb + P.tw - 1;
}

// Window slot offset of tap (j, l) relative to window_base.
C2B_HD int tap_window_offset(const TileCtx& c, int j, int l) { return -(j * c.roww + l); }

// Plane offset ih*W + iw of the grad_input pixel of a tile-local lane, or -1.
C2B_HD int output_offset(const TileCtx& c, const LaunchArgs& a, int local) {
  const PhaseDesc& P = c.P;
  if (local >= c.npx) return -1;
  const int q = c.p0 + local;
  const int ip = q / P.wb;
  const int jj = c.band * P.wb + (q - ip * P.wb);
  if (jj >= P.wp) return -1;
  const int ih = P.ih0 + a.S * ip;
  const int iw = P.iw0 + a.S * jj;
  return ih * a.W + iw;
}

// Flat weight index kh*KW + kw of the tap-th tap of the class.
C2B_HD int tap_kidx(const PhaseDesc& P, const LaunchArgs& a, int tap) {
  const int j = tap / P.tw;
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

// Accumulator register r of lane half h in a 32x32 block holds block row
// 8*(r/4) + 4*h + r%4 (column = lane mod 32) -- the C/D layout of the
// 32x32 matrix instructions used here.
C2B_HD int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

}  // namespace c2b
