// Launch planning for the conv2d input-gradient kernels (internal header).
//
// The planner is plain host C++: it validates a conv2d_params, splits the
// problem into stride-residue phases and tiles, and fills the by-value
// argument block each kernel launch receives.  The kernels only decode their
// tile from that block.
//
// Stride-residue phases.  In the gather rule of the shader's stride > 1
// im2col branch (meganeura 0.2.0, conv2d_grad_input_gemm_coop.wgsl), a tap
// (kh, kw) contributes to input pixel (ih, iw) only if ih + padding_h - kh and
// iw + padding_w - kw are both multiples of s.  Grouping input rows by
// rh = (ih + padding_h) mod s and kernel rows by kh mod s, only kernel rows
// with kh = rh (mod s) ever reach the rows of class rh (likewise for columns).
// Each class (rh, rw) is therefore a dense stride-1 problem on the sub-image
//   ih = ih0 + s*i',  iw = iw0 + s*j'
// with the sub-kernel kh = rh + s*j, kw = rw + s*l (j < th, l < tw), and the
// grad_out row it reads is oh = i' + ch - j (column ow = j' + cw - l), where
// ch = (ih0 + padding_h - rh) / s.  For s = 1 there is one class.  No
// structural zero is ever multiplied; classes that no tap reaches (s > kernel)
// are written as zeros.
#pragma once

#include <stdint.h>

namespace c2b {

constexpr int kMaxPhasesPerLaunch = 16;

// One stride-residue class and its tiling.
struct PhaseDesc {
  int32_t rh, rw;      // residues of (ih + padding_h), (iw + padding_w) mod s
  int32_t ih0, iw0;    // first input row / column of the class
  int32_t hp, wp;      // rows / columns of the class sub-image
  int32_t th, tw;      // sub-kernel taps per axis (0: class gets zeros)
  int32_t ch, cw;      // grad_out row = i' + ch - j, column = j' + cw - l
  int32_t wb;          // band width: sub-image columns per band
  int32_t nbands;      // bands per sub-image row, ceil(wp / wb)
  int32_t ntv;         // pixels per tile (<= the kernel's lane tile)
  int32_t ptiles;      // tiles per (image, band): ceil(hp * wb / ntv)
  int32_t ngroups;     // tap groups: ceil(th * tw / taps per stage)
  int32_t tiles;       // tiles of this class in the launch
  int32_t tile_begin;  // first workgroup index of this class in the launch
  int32_t ckr;         // output channels per stage (fp32 kernel)
  int32_t tg;          // taps per stage (fp32 kernel)
  int32_t slabr;       // window slots per channel in LDS (fp32 kernel)
  int32_t cp;          // LDS floats per output channel of staged weights (fp32 kernel)
  // reciprocals for per-lane division: m = ceil(2^31 / d), see fast_div
  uint32_t m_roww;     // d = wb + tw - 1
  uint32_t m_wb;       // d = wb
  uint32_t m_tw;       // d = tw
  uint32_t m_slots4;   // d = 4 * slabr
  uint32_t m_cp;       // d = cp
  uint32_t m_tg;       // d = tg
};

// By-value kernel argument block of one launch.
struct LaunchArgs {
  const float* go;
  const float* w;
  float* gi;
  int32_t N, Ci, H, W, Co, KH, KW, S, PH, PW, OH, OW;
  int32_t ciblocks;    // ceil(Ci / channel tile)
  int32_t nphases;     // classes in this launch, heaviest first
  int32_t total_tiles; // workgroups in this launch
  int32_t variant;     // kernel instantiation (host side only)
  PhaseDesc ph[kMaxPhasesPerLaunch];
};

// Compile-time tile shape of one kernel variant, as the planner sees it.
struct TileShape {
  int mt;     // input channels per workgroup
  int nt;     // pixel lanes per workgroup
  int ck;     // output channels staged per stage
  int taps;   // kernel taps staged per stage
  int slab;   // staged grad_out elements per output channel (halo window)
};

}  // namespace c2b

#include <vector>

#include "../../include/conv2d_bwd.h"

namespace c2b {

// Tile shapes of the two kernel families (the kernels static_assert that
// their template arguments match these).
constexpr TileShape kF32Tile{64, 256, 8, 9, 608};
constexpr TileShape kF16Tile{64, 256, 16, 9, 608};

// Shape checks shared by every entry point (no pointer is looked at).
int validate_shape(const conv2d_params* p);

// Full plan for one tile shape: validate, split into classes and tiles, and
// append one LaunchArgs per launch (pointers left null).  `info` may be null.
// Used by the f16-staged kernel.
int build_plan(const conv2d_params* p, const TileShape& ts,
               std::vector<LaunchArgs>* launches, conv2d_plan_info* info);

// fp32 kernel family: WM x WN waves, 16x16x4 fp32 matrix instructions; each
// wave owns 16 input channels x NBW blocks of 16 pixels.  WM waves along
// channels (64- or 128-channel tiles), WN waves along pixels (2, 3 or 4 waves
// per SIMD).
struct F32Variant {
  int wm;    // waves along channels: 4 (64-channel tiles) or 8 (128)
  int wn;    // waves along pixels
  int nbw;   // 16-pixel blocks per wave
};
constexpr F32Variant kF32Variants[] = {{4, 2, 4}, {4, 2, 8}, {4, 2, 13}, {4, 3, 9},
                                       {4, 4, 7}, {8, 1, 4}, {8, 1, 8}, {8, 1, 13},
                                       {8, 2, 7}};
constexpr int kNumF32Variants = int(sizeof(kF32Variants) / sizeof(kF32Variants[0]));
constexpr int kF32StageCh = 16;     // output channels per stage
constexpr int kF32MaxSlots = 640;   // window slots per channel (multiple of 16)
constexpr int kF32MaxCP = 608;      // staged weight floats per channel
constexpr int kF32WinFloats = kF32StageCh * kF32MaxSlots;   // one window buffer
constexpr int kF32WtFloats = kF32StageCh * kF32MaxCP;       // one weight buffer
constexpr int kF32LdsFloats = 2 * (kF32WinFloats + kF32WtFloats);   // 156 KiB
constexpr int kF32StageTaps = 9;    // kernel taps per stage
constexpr int kF32DefaultCUs = 256;

// Plan for the fp32 kernel family on a device with `num_cus` compute units:
// chooses the variant, tile sizes and stage depths per class (balancing the
// tiles over the compute units, heaviest first).
// force_variant >= 0 plans with that variant only (CONV2D_ERR_UNSUPPORTED if
// it cannot tile the shape); used by host-side checks of every variant.
int build_plan_f32(const conv2d_params* p, int num_cus, std::vector<LaunchArgs>* launches,
                   conv2d_plan_info* info, int force_variant = -1);

// Pointer checks: NULL inputs of non-empty tensors and output/input overlap.
int check_pointers(const float* go, const float* w, const float* gi,
                   const conv2d_params* p);

}  // namespace c2b
