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
//
// Stages.  A tile's contraction runs in stages; a stage is cg groups of 16
// output channels times up to tg taps of the class (a "unit" is one group at
// one tap: 16 values of k).  Its grad_out halo window and its weights are
// copied into one of two LDS stage buffers while the other buffer is
// multiplied.  Stages run tap-group-major: for each tap group, every chunk of
// 16*cg output channels.
//
// Forward convolution (the adjoint operator, same kernels).  With the kernel
// taps flipped, j = KH-1-kh and l = KW-1-kw, the forward convolution
//   y[n, co, oh, ow] = sum over ci, kh, kw of
//       x[n, ci, s*oh - padding_h + kh, s*ow - padding_w + kw] * w[co, ci, kh, kw]
// reads x row s*oh + ch - j with ch = KH-1-padding_h: the form of a class
// above with the output plane as the class sub-image, all KH x KW taps, and
// the window sampled every s rows and columns (PhaseDesc::ss).  A forward
// launch therefore runs the same kernels with the roles exchanged: the
// matrix rows are the output channels co, the contraction runs over the
// input channels ci and the taps, the window is cut from x and the results
// go to y (LaunchArgs::fwd).
#pragma once

#include <stdint.h>

namespace c2b {

constexpr int kMaxPhasesPerLaunch = 16;

// LDS floats of one stage buffer: two per workgroup, 156 KiB of the 160 KiB
// (kStageFloats), or half of that for variants that run two workgroups per
// CU (kStageFloatsHalf).
constexpr int kStageFloats = 19968;
constexpr int kStageFloatsHalf = 9984;
constexpr int kMaxStageTaps = 9;    // taps per stage
constexpr int kMaxStageGroups = 8;  // 16-channel groups per stage
constexpr int kDefaultCUs = 256;

// One stride-residue class and its tiling.
struct PhaseDesc {
  int32_t rh, rw;      // residues of (ih + padding_h), (iw + padding_w) mod s
  int32_t ih0, iw0;    // first input row / column of the class
  int32_t hp, wp;      // rows / columns of the class sub-image
  int32_t th, tw;      // sub-kernel taps per axis (0: class gets zeros)
  int32_t ch, cw;      // source row = ss*i' + ch - j, column = ss*j' + cw - l
  int32_t ss;          // source rows / columns per pixel step (1; forward: stride)
  int32_t kstep;       // kernel index of tap (j, l): (rh + kstep*j, rw + kstep*l)
  int32_t wb;          // band width: sub-image columns per band
  int32_t nbands;      // bands per sub-image row, ceil(wp / wb)
  int32_t ntv;         // pixels per tile (<= the kernel's lane tile)
  int32_t ptiles;      // tiles per (image, band): ceil(hp * wb / ntv)
  int32_t tiles;       // tiles of this class in the launch
  int32_t img_tiles;   // tiles of this class per image: tiles / N
  int32_t img_begin;   // first tile of this class in an image's run (see
                       // decode_tile): img_tiles of the classes before it
  int32_t cg;          // 16-channel groups per stage
  int32_t tg;          // taps per stage
  int32_t ngroups;     // tap groups, ceil(th * tw / tg)
  int32_t nchunks;     // output-channel chunks, ceil(Co / (16 * cg))
  int32_t slots;       // window slots per channel (multiple of 16)
  int32_t pt;          // weight pitch per input channel, in taps (odd, >= tg)
  int32_t qp;          // weight floats per channel quad (multiple of 64)
  int32_t wfl;         // window floats of a stage buffer: 16 * cg * slots
  int32_t used;        // floats of a stage buffer copied: wfl + 4 * cg * qp
  int32_t mct;         // multi-class union: taps of the stage contraction (kH * kW,
                       // in the weight's own order); 0 for any other class
  // reciprocals for per-lane division: m = ceil(2^31 / d), see fast_div
  uint32_t m_roww;     // d = roww = ss*(wb - 1) + tw
  uint32_t m_wb;       // d = wb
  uint32_t m_tw;       // d = tw
  uint32_t m_slots4;   // d = 4 * slots
  uint32_t m_qp;       // d = qp
  uint32_t m_pt4;      // d = 4 * pt
  uint32_t m_pt;       // d = pt
  uint32_t m_blocks;   // d = copy blocks of a quad (window + weight blocks)
};

// One stride-residue class of a multi-class launch (Variant::mc): its pixels
// are (ih0 + 2 i', iw0 + 2 j') for grid points i' < hp, j' < wp, its taps
// (rh + 2 j, rw + 2 l) for j < th, l < tw, and its pixel at window position
// (dr, jb) of a tile reads window row dr + e - j, column jb + f - l at tap
// (j, l).
struct MCClass {
  int32_t ih0, iw0, hp, wp, th, tw, rh, rw, e, f;
};
constexpr int kMCClasses = 4;   // multi-class launches: stride 2

// By-value kernel argument block of one launch.  For a forward launch
// (fwd = 1) the fields keep their input-gradient roles: go is x, gi is y, Ci
// and H x W are the output channels and plane, Co and OH x OW the input
// channels and plane, and S = 1 (the output plane is dense; the stride is the
// classes' ss).
struct LaunchArgs {
  const float* go;
  const float* w;
  float* gi;
  int32_t N, Ci, H, W, Co, KH, KW, S, PH, PW, OH, OW;
  int32_t fwd;         // 1: forward convolution launch (roles above)
  int32_t wsm, wsk;    // weight elements between matrix rows / contraction channels
  int32_t ciblocks;    // ceil(Ci / cit)
  int32_t cit;         // input channels per tile
  int32_t cm;          // 1: column taps in the matrix rows (see Variant::cm)
  int32_t twm;         // cm: matrix rows per input channel (widest class's tw)
  int32_t nphases;     // classes in this launch, heaviest first
  int32_t total_tiles; // workgroups in this launch
  int32_t ilv;         // 1: classes interleaved image by image (decode_tile)
  int32_t img_total;   // tiles per image over the launch's classes
  int32_t variant;     // kernel instantiation (host side only)
  int32_t mc;          // 1: multi-class launch (ph[0] is the union of mcls)
  PhaseDesc ph[kMaxPhasesPerLaunch];
  MCClass mcls[kMCClasses];
};

// One instantiation of the kernel family: WM x WN waves; wave (mg, ng) owns
// MB blocks of 16 input channels x NBW blocks of 16 pixels.  fp32 variants
// multiply on v_mfma_f32_16x16x4_f32, f16 variants on
// v_mfma_f32_16x16x32_f16 (pairs of units) and v_mfma_f32_16x16x16_f16.
//
// cm (column taps in the matrix rows, for few input channels): the 16 rows
// of a tile's matrix block are (input channel, column tap l) pairs, twm rows
// per channel, instead of 16 input channels; a stage's contraction runs over
// output channels x row taps j only, and its "pixels" are the points (class
// row, window column) of whole rows.  Each product row then holds, for one
// channel and one column tap, the partial sum over all output channels and
// row taps; the epilogue adds the tw partial sums of a pixel, which sit tw
// window columns apart, through LDS.  With Ci = 3 and a 4-column class this
// fills 12 of 16 rows, where one channel per row fills 3.
//
// mc (multi-class, stride 2): one tile covers the same grid points
// (i', j') of all four stride-residue classes, so the four classes share
// one grad_out window per stage (the union of the windows they read) and a
// stage holds all kH x kW taps of the weights.  Every wave multiplies every
// class: for its NBW blocks of grid points it keeps one accumulator set per
// class, and each unit (16 output channels at one tap) updates the set of
// the class the tap belongs to.  The epilogue stores each class's pixels.
struct Variant {
  int f16;   // 0: fp32 path, 1: f16-staged path
  int wm;    // waves along channels
  int wn;    // waves along pixels
  int mb;    // 16-channel blocks per wave
  int nbw;   // 16-pixel blocks per wave
  int half;  // 1: half-size stage buffers, two workgroups per CU
  int cm;    // 1: column taps in the matrix rows (wm = mb = 1)
  int mc;    // 1: all four classes of a stride-2 shape per tile
};

// Floats of one stage buffer of a variant.  Multi-class variants stage a
// window shared by four classes, so their stages are smaller; 52 copy
// batches keep each of 8 waves at 7 batches of staging registers (with
// more, the accumulators of four classes no longer fit in registers).  The
// one-block-row form (32 channels, 7 pixel blocks per wave) holds 8 operand
// reads per unit and stays at 46 batches (6 per wave).
constexpr int kStageFloatsMC = 13312;
constexpr int kStageFloatsMC1 = 11776;
constexpr int stage_floats(const Variant& v) {
  return v.mc ? (v.mb == 1 ? kStageFloatsMC1 : kStageFloatsMC)
              : v.half ? kStageFloatsHalf : kStageFloats;
}

// Copy batches (of 256 floats) one wave of a variant copies per stage at
// most; a stage shape is usable only if its batches fit in the waves.
constexpr int batches_per_wave(const Variant& v) {
  return (stage_floats(v) / 256 + v.wm * v.wn - 1) / (v.wm * v.wn);
}

constexpr Variant kVariants[] = {
    // fp32, one workgroup per CU
    {0, 4, 2, 1, 4, 0}, {0, 4, 2, 1, 8, 0}, {0, 4, 2, 1, 13, 0}, {0, 4, 3, 1, 9, 0},
    {0, 4, 4, 1, 7, 0}, {0, 8, 1, 1, 4, 0}, {0, 8, 1, 1, 8, 0}, {0, 8, 1, 1, 13, 0},
    {0, 8, 2, 1, 7, 0},
    // f16-staged, one workgroup per CU
    {1, 4, 2, 1, 8, 0}, {1, 2, 4, 2, 4, 0}, {1, 1, 8, 4, 2, 0}, {1, 2, 4, 4, 2, 0},
    {1, 2, 4, 4, 4, 0}, {1, 4, 2, 2, 4, 0}, {1, 2, 6, 2, 3, 0},
    // fp32, two workgroups per CU
    {0, 4, 2, 1, 7, 1}, {0, 4, 2, 1, 5, 1}, {0, 4, 2, 1, 8, 1},
    // one 16-channel block per tile (few input channels)
    {0, 1, 8, 1, 7, 0}, {0, 1, 12, 1, 5, 0}, {0, 1, 16, 1, 4, 0}, {1, 1, 12, 1, 5, 0},
    {1, 1, 8, 1, 7, 0},
    // column taps in the matrix rows (few input channels)
    {0, 1, 8, 1, 7, 0, 1}, {0, 1, 12, 1, 5, 0, 1}, {0, 1, 16, 1, 4, 0, 1},
    {0, 1, 8, 1, 4, 1, 1}, {1, 1, 8, 1, 7, 0, 1}, {1, 1, 12, 1, 5, 0, 1},
    {1, 1, 8, 1, 4, 1, 1},
    // all four classes of a stride-2 shape per tile (fp32), the four
    // classes' accumulators in registers: 8 waves of 64 channels x 4 blocks
    // or 32 channels x 7 blocks (pixel blocks then split 13 : 12 rather than
    // 14 : 12 between the SIMDs on 196-pixel tiles), or 12 waves of 32
    // channels x 5 blocks (three waves per SIMD, 13 : 12 as well)
    {0, 2, 4, 2, 4, 0, 0, 1}, {0, 2, 4, 1, 7, 0, 0, 1}, {0, 2, 6, 1, 5, 0, 0, 1}};
constexpr int kNumVariants = int(sizeof(kVariants) / sizeof(kVariants[0]));

}  // namespace c2b

#include <vector>

#include "../../include/conv2d_bwd.h"

namespace c2b {

// Shape checks shared by every entry point (no pointer is looked at).
int validate_shape(const conv2d_params* p);

// The two operations the kernels run.
enum Op { kOpGradInput = 0, kOpForward = 1 };

// Plan for the fp32 (f16 == 0) or f16-staged path on a device with
// `num_cus` compute units: chooses the variant, tile sizes and stage shapes
// per class (balancing the tiles over the compute units, heaviest first) and
// appends one LaunchArgs per launch (pointers left null).  `info` may be null.
// force_variant >= 0 plans with that variant only (CONV2D_ERR_UNSUPPORTED if
// it belongs to the other path or cannot tile the shape).
// `model_cost` (may be null) receives the modelled makespan of the plan.
// op = kOpForward plans the forward convolution (no cm variants).
int build_plan(const conv2d_params* p, int f16, int num_cus, std::vector<LaunchArgs>* launches,
               conv2d_plan_info* info, int force_variant = -1, double* model_cost = nullptr,
               int op = kOpGradInput);

// Pointer checks: NULL inputs of non-empty tensors and output/input overlap.
// Input gradient: inputs go, w, output gi.  Forward (op = kOpForward):
// inputs x (passed as go), w, output y (passed as gi).
int check_pointers(const float* go, const float* w, const float* gi,
                   const conv2d_params* p, int op = kOpGradInput);

}  // namespace c2b
