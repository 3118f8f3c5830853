// Host-side validation and launch planning (no HIP call in this file).
//
// Shape rules follow the `Params` struct of the shader this library
// re-designs (meganeura 0.2.0, conv2d_grad_input_gemm_coop.wgsl): one stride
// for both axes, separate paddings, out_h / out_w passed in.  Here out_h and
// out_w must equal the forward-convolution extents, so that grad_input is the
// exact adjoint of that forward convolution.
#include <algorithm>
#include <climits>
#include <cstdint>
#include <cstring>

#include "plan.hpp"
#include "pointwise.hpp"
#include "tile_index.hpp"

namespace c2b {

namespace {

constexpr int64_t kI31 = int64_t(1) << 31;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// First index i >= 0 with (i + pad) mod s == r.
int64_t first_of_class(int64_t r, int64_t pad, int64_t s) {
  return (((r - pad) % s) + s) % s;
}

}  // namespace

int validate_shape(const conv2d_params* p) {
  if (p == nullptr) return CONV2D_ERR_NULL_PTR;
  const int64_t N = p->batch, Ci = p->in_channels, H = p->in_h, W = p->in_w;
  const int64_t Co = p->out_channels, KH = p->kernel_h, KW = p->kernel_w;
  const int64_t S = p->stride, PH = p->padding_h, PW = p->padding_w;
  const int64_t OH = p->out_h, OW = p->out_w;
  if (S == 0 || KH == 0 || KW == 0) return CONV2D_ERR_BAD_SHAPE;
  if (H + 2 * PH < KH || W + 2 * PW < KW) return CONV2D_ERR_BAD_SHAPE;
  if (OH != (H + 2 * PH - KH) / S + 1) return CONV2D_ERR_BAD_SHAPE;
  if (OW != (W + 2 * PW - KW) / S + 1) return CONV2D_ERR_BAD_SHAPE;
  // every extent and per-image plane is indexed with 32-bit offsets; the
  // batch offset is 64-bit
  const int64_t dims[] = {N, Ci, H, W, Co, KH, KW, S, PH, PW, OH, OW};
  for (int64_t d : dims)
    if (d >= kI31) return CONV2D_ERR_OVERFLOW;
  if (H * W >= kI31 || OH * OW >= kI31) return CONV2D_ERR_OVERFLOW;
  if (Ci * H * W >= kI31 || Co * OH * OW >= kI31) return CONV2D_ERR_OVERFLOW;
  if (Co * Ci >= kI31 || Co * Ci * KH * KW >= kI31) return CONV2D_ERR_OVERFLOW;
  if (H + PH + KH >= kI31 || W + PW + KW >= kI31) return CONV2D_ERR_OVERFLOW;
  return CONV2D_OK;
}

int check_pointers(const float* go, const float* w, const float* gi,
                   const conv2d_params* p, int op) {
  if (p == nullptr) return CONV2D_ERR_NULL_PTR;
  // input-side and output-side element counts: forward reads x and writes y
  const uint64_t n_x = uint64_t(p->batch) * p->in_channels * p->in_h * p->in_w;
  const uint64_t n_y = uint64_t(p->batch) * p->out_channels * p->out_h * p->out_w;
  const uint64_t n_gi = op == kOpForward ? n_y : n_x;   // written
  const uint64_t n_go = op == kOpForward ? n_x : n_y;   // read
  const uint64_t n_w = uint64_t(p->out_channels) * p->in_channels * p->kernel_h *
                       p->kernel_w;
  if ((n_gi && gi == nullptr) || (n_go && go == nullptr) || (n_w && w == nullptr))
    return CONV2D_ERR_NULL_PTR;
  auto overlap = [](const float* a, uint64_t na, const float* b, uint64_t nb) {
    if (na == 0 || nb == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a);
    const uintptr_t b0 = reinterpret_cast<uintptr_t>(b);
    const uintptr_t a1 = a0 + na * sizeof(float);
    const uintptr_t b1 = b0 + nb * sizeof(float);
    return a0 < b1 && b0 < a1;
  };
  if (overlap(gi, n_gi, go, n_go) || overlap(gi, n_gi, w, n_w))
    return CONV2D_ERR_ALIAS;
  return CONV2D_OK;
}

// Non-empty stride-residue classes of a shape (geometry only, no tiling).
static void make_classes(const conv2d_params* p, std::vector<PhaseDesc>* out) {
  const int64_t H = p->in_h, W = p->in_w, KH = p->kernel_h, KW = p->kernel_w;
  const int64_t S = p->stride, PH = p->padding_h, PW = p->padding_w;
  for (int64_t rh = 0; rh < S; ++rh) {
    for (int64_t rw = 0; rw < S; ++rw) {
      PhaseDesc d;
      std::memset(&d, 0, sizeof(d));
      const int64_t ih0 = first_of_class(rh, PH, S);
      const int64_t iw0 = first_of_class(rw, PW, S);
      const int64_t hp = ih0 < H ? ceil_div(H - ih0, S) : 0;
      const int64_t wp = iw0 < W ? ceil_div(W - iw0, S) : 0;
      if (hp == 0 || wp == 0) continue;  // class has no pixel
      const int64_t th = rh < KH ? ceil_div(KH - rh, S) : 0;
      const int64_t tw = rw < KW ? ceil_div(KW - rw, S) : 0;
      d.rh = int32_t(rh);
      d.rw = int32_t(rw);
      d.ih0 = int32_t(ih0);
      d.iw0 = int32_t(iw0);
      d.hp = int32_t(hp);
      d.wp = int32_t(wp);
      d.ss = 1;
      d.kstep = int32_t(S);
      if (th > 0 && tw > 0) {
        d.th = int32_t(th);
        d.tw = int32_t(tw);
        d.ch = int32_t((ih0 + PH - rh) / S);
        d.cw = int32_t((iw0 + PW - rw) / S);
      }
      out->push_back(d);
    }
  }
}

// The forward convolution as one class over the output plane (plan.hpp):
// all KH x KW taps, flipped (kernel index (KH-1-j, KW-1-l)), window sampled
// every `stride` source rows and columns.
static void make_forward_class(const conv2d_params* p, std::vector<PhaseDesc>* out) {
  PhaseDesc d;
  std::memset(&d, 0, sizeof(d));
  d.rh = int32_t(p->kernel_h) - 1;
  d.rw = int32_t(p->kernel_w) - 1;
  d.kstep = -1;
  d.ss = int32_t(p->stride);
  d.hp = int32_t(p->out_h);
  d.wp = int32_t(p->out_w);
  d.th = int32_t(p->kernel_h);
  d.tw = int32_t(p->kernel_w);
  d.ch = int32_t(p->kernel_h) - 1 - int32_t(p->padding_h);
  d.cw = int32_t(p->kernel_w) - 1 - int32_t(p->padding_w);
  if (d.hp > 0 && d.wp > 0) out->push_back(d);
}

// The four classes of a stride-2 shape as one multi-class tiling
// (Variant::mc): `u` describes the tiling over the grid of class pixels
// (i', j') and the window all classes share, `mcls` each class.  Class k
// reads grad_out row i' + ch_k - j at tap j; over the classes and their taps
// these rows run from i' + lo to i' + max ch_k, lo = min (ch_k - th_k + 1),
// so the union window has th = max ch_k - lo + 1 rows per grid row and class
// k's tap j sits e_k - j rows into it, e_k = ch_k - lo (columns alike).
// False unless the shape has stride 2, all four classes have pixels and
// taps, and the kernel has at most kMaxStageTaps taps (one stage holds them
// all).
static bool make_mc_union(const conv2d_params* p, const std::vector<PhaseDesc>& classes,
                          PhaseDesc* u, MCClass* mcls) {
  if (p->stride != 2 || classes.size() != size_t(kMCClasses)) return false;
  if (int64_t(p->kernel_h) * p->kernel_w > kMaxStageTaps) return false;
  int32_t hch = INT32_MIN, hlo = INT32_MAX, wch = INT32_MIN, wlo = INT32_MAX, hp = 0, wp = 0;
  for (const PhaseDesc& d : classes) {
    if (d.th == 0 || d.tw == 0) return false;
    hch = std::max(hch, d.ch);
    hlo = std::min(hlo, d.ch - d.th + 1);
    wch = std::max(wch, d.cw);
    wlo = std::min(wlo, d.cw - d.tw + 1);
    hp = std::max(hp, d.hp);
    wp = std::max(wp, d.wp);
  }
  std::memset(u, 0, sizeof(*u));
  u->hp = hp;
  u->wp = wp;
  u->th = hch - hlo + 1;
  u->tw = wch - wlo + 1;
  u->ch = hch;
  u->cw = wch;
  u->ss = 1;
  u->kstep = 1;
  u->mct = int32_t(p->kernel_h * p->kernel_w);
  for (int k = 0; k < kMCClasses; ++k) {
    const PhaseDesc& d = classes[size_t(k)];
    mcls[k] = MCClass{d.ih0, d.iw0, d.hp, d.wp, d.th, d.tw, d.rh, d.rw, d.ch - hlo, d.cw - wlo};
  }
  return true;
}

static LaunchArgs launch_header(const conv2d_params* p, int64_t ciblocks, int64_t cit, int cm,
                                int64_t twm, int op) {
  LaunchArgs la;
  std::memset(&la, 0, sizeof(la));
  const int32_t KHW = int32_t(p->kernel_h * p->kernel_w);
  la.N = int32_t(p->batch);
  la.KH = int32_t(p->kernel_h);
  la.KW = int32_t(p->kernel_w);
  la.PH = int32_t(p->padding_h);
  la.PW = int32_t(p->padding_w);
  if (op == kOpForward) {   // roles exchanged (plan.hpp)
    la.fwd = 1;
    la.Ci = int32_t(p->out_channels);
    la.H = int32_t(p->out_h);
    la.W = int32_t(p->out_w);
    la.Co = int32_t(p->in_channels);
    la.S = 1;
    la.OH = int32_t(p->in_h);
    la.OW = int32_t(p->in_w);
    la.wsm = int32_t(p->in_channels) * KHW;   // w[co, ci, kh, kw]: co is the row
    la.wsk = KHW;
    la.ciblocks = int32_t(ciblocks);
    la.cit = int32_t(cit);
    return la;
  }
  la.Ci = int32_t(p->in_channels);
  la.H = int32_t(p->in_h);
  la.W = int32_t(p->in_w);
  la.Co = int32_t(p->out_channels);
  la.S = int32_t(p->stride);
  la.wsm = KHW;                               // ci is the row, co the channel
  la.wsk = int32_t(p->in_channels) * KHW;
  la.OH = int32_t(p->out_h);
  la.OW = int32_t(p->out_w);
  la.ciblocks = int32_t(ciblocks);
  la.cit = int32_t(cit);
  la.cm = cm;
  la.twm = int32_t(twm);
  return la;
}


// Reciprocals of a class's per-lane divisors, and the bounds under which the
// kernel's fast_div is exact (numerator x divisor < 2^31): numerators are
// stage-buffer cells (< kStageFloats), window slots (< slots), taps, and
// positions inside a band row plus one tile of pixels.
static int finalize_divisors(PhaseDesc* d) {
  const int64_t lim = int64_t(1) << 31;
  const int64_t roww = std::max<int64_t>((int64_t(d->wb) - 1) * d->ss + d->tw, 1);
  const int64_t wb = d->wb, tw = std::max(d->tw, 1);
  const int64_t slots4 = std::max<int64_t>(4 * int64_t(d->slots), 1);
  const int64_t qp = std::max(d->qp, 1), pt4 = std::max<int64_t>(4 * int64_t(d->pt), 1);
  if (int64_t(kStageFloats) * std::max<int64_t>(slots4, qp) >= lim) return CONV2D_ERR_OVERFLOW;
  if (int64_t(std::max(d->slots, 4096)) * roww >= lim) return CONV2D_ERR_OVERFLOW;
  if (qp * pt4 >= lim) return CONV2D_ERR_OVERFLOW;
  if ((wb + d->ntv + 1024) * wb >= lim) return CONV2D_ERR_OVERFLOW;
  if (int64_t(d->th) * d->tw * tw >= lim) return CONV2D_ERR_OVERFLOW;
  // copy-batch numerators: batches of a stage, weight pairs of a quad
  if (int64_t(kStageFloats) * std::max(copy_blocks(*d), 1) >= lim) return CONV2D_ERR_OVERFLOW;
  if ((qp + 256) * std::max(d->pt, 1) >= lim) return CONV2D_ERR_OVERFLOW;
  d->m_roww = fast_div_magic(uint32_t(roww));
  d->m_wb = fast_div_magic(uint32_t(wb));
  d->m_tw = fast_div_magic(uint32_t(tw));
  d->m_slots4 = fast_div_magic(uint32_t(slots4));
  d->m_qp = fast_div_magic(uint32_t(qp));
  d->m_pt4 = fast_div_magic(uint32_t(pt4));
  d->m_pt = fast_div_magic(uint32_t(std::max(d->pt, 1)));
  d->m_blocks = fast_div_magic(uint32_t(std::max(copy_blocks(*d), 1)));
  return CONV2D_OK;
}

// Split classes (already sorted heaviest first) into launches of at most
// kMaxPhasesPerLaunch classes.
static int emit_launches(const conv2d_params* p, int64_t ciblocks, int64_t cit, int64_t twm,
                         int variant, const std::vector<PhaseDesc>& phases,
                         std::vector<LaunchArgs>* launches, conv2d_plan_info* info, int op,
                         const MCClass* mcls) {
  for (size_t base = 0; base < phases.size(); base += kMaxPhasesPerLaunch) {
    LaunchArgs la = launch_header(p, ciblocks, cit, kVariants[variant].cm, twm, op);
    la.variant = variant;
    if (kVariants[variant].mc) {
      la.mc = 1;
      for (int k = 0; k < kMCClasses; ++k) la.mcls[k] = mcls[k];
    }
    int64_t total = 0, per_image = 0;
    const size_t end = std::min(phases.size(), base + kMaxPhasesPerLaunch);
    for (size_t i = base; i < end; ++i) {
      PhaseDesc d = phases[i];
      const int rc = finalize_divisors(&d);
      if (rc != CONV2D_OK) return rc;
      total += d.tiles;
      if (total >= kI31) return CONV2D_ERR_OVERFLOW;
      // a class's tiles run image by image (tile_class: N x bands x pixel
      // tiles x channel blocks)
      d.img_tiles = p->batch > 0 ? int32_t(d.tiles / p->batch) : 0;
      d.img_begin = int32_t(per_image);
      per_image += d.img_tiles;
      la.ph[la.nphases++] = d;
    }
    la.total_tiles = int32_t(total);
    la.img_total = int32_t(per_image);
    // Interleave the classes image by image when their tiles run the same
    // number of stages.  With unequal stage counts the heaviest-first class
    // order is kept: interleaved, a late image's heavy tiles would set the
    // launch's tail.
    bool same_stages = la.nphases > 1 && per_image > 0;
    for (int i = 1; i < la.nphases; ++i)
      same_stages = same_stages && la.ph[i].nchunks * la.ph[i].ngroups ==
                                       la.ph[0].nchunks * la.ph[0].ngroups;
    la.ilv = same_stages ? 1 : 0;
    if (launches) launches->push_back(la);
    if (info) {
      info->launches += 1;
      info->tiles += total;
    }
  }
  return CONV2D_OK;
}

namespace {

// Most grad_out rows a run of `ntv` consecutive pixels touches in a band
// `wb` wide, over all tiles p0 = k*ntv of a band of `bp` pixels.  The row
// phase p0 mod wb repeats with period wb / gcd(ntv, wb), so one period of
// full-length tiles covers every case (a shorter last tile spans no more
// rows than a full one at the same phase).
int64_t max_rows_spanned(int64_t wb, int64_t ntv, int64_t bp) {
  if (ntv % wb == 0) return ntv / wb;               // tiles start on row starts
  const int64_t tiles = ceil_div(bp, ntv);
  int64_t a = ntv, b = wb;
  while (b) {
    const int64_t t = a % b;
    a = b;
    b = t;
  }
  const int64_t period = wb / a;
  int64_t best = 0;
  for (int64_t t = 0; t < std::min(tiles, period); ++t) {
    const int64_t p0 = t * ntv, p1 = p0 + ntv - 1;
    best = std::max(best, p1 / wb - p0 / wb + 1);
  }
  return best;
}

// Band width and pixels per tile for a class whose window must fit
// `max_slots` slots per channel (slots rounded up to a multiple of 16).
// Fewest bands first; for each band width, equal tiles of at most ntl
// pixels, halving the tile until the window fits.
// `extra` > 0 asks for that many more tiles per band than the fewest that
// fit (smaller tiles, so that the tile count can match the CUs); false if
// the tiles would fall below one 16-pixel block.
bool choose_tiling(const PhaseDesc& d, int64_t ntl, int64_t max_slots, int64_t extra,
                   int64_t* wb_out, int64_t* ntv_out, int64_t* slots_out) {
  const int64_t th = d.th, tw = d.tw, hp = d.hp, wp = d.wp, ss = d.ss;
  int64_t last_wb = -1;
  for (int64_t nb = 1; nb <= wp; ++nb) {
    const int64_t wb = ceil_div(wp, nb);
    if (wb == last_wb) continue;
    last_wb = wb;
    const int64_t bp = hp * wb;
    const int64_t roww = (wb - 1) * ss + tw;
    for (int64_t cap = ntl;; cap = (cap + 1) / 2) {
      int64_t ntv = ceil_div(bp, ceil_div(bp, cap));
      if (extra > 0) {
        ntv = ceil_div(bp, ceil_div(bp, ntv) + extra);
        if (ntv < 16) return false;
      }
      const int64_t rows = (max_rows_spanned(wb, ntv, bp) - 1) * ss + th;
      const int64_t slots = ceil_div(rows * roww, 16) * 16;
      if (slots <= max_slots) {
        *wb_out = wb;
        *ntv_out = ntv;
        *slots_out = slots;
        return true;
      }
      if (cap <= 1 || ntv <= wb / 4) break;           // more tiles will not help
    }
    if (wb == 1) break;
  }
  return false;
}

// cm tiling: a tile is `rows` whole rows of a band `wb` wide; its lanes are
// the rows x (wb + tw - 1) window points (at most ntl), and its window of
// rows + th - 1 rows must fit `max_slots` slots per channel.  Fills the
// candidate for band count nb; false if nothing fits.
bool cm_tiling(const PhaseDesc& d, int64_t nb, int64_t ntl, int64_t max_slots, int64_t* wb_out,
               int64_t* rows_out, int64_t* slots_out) {
  const int64_t wb = ceil_div(d.wp, nb), roww = wb + d.tw - 1;
  int64_t rows = std::min<int64_t>({ntl / roww, int64_t(d.hp), max_slots / roww - d.th + 1});
  if (rows < 1) return false;
  rows = ceil_div(d.hp, ceil_div(d.hp, rows));       // equal row counts per tile
  *wb_out = wb;
  *rows_out = rows;
  *slots_out = ceil_div((rows + d.th - 1) * roww, 16) * 16;
  return *slots_out <= max_slots;
}

// Cost model of one tile, in CU cycles.  Its constants are a least-squares
// fit (log time) to forced-variant timings of every kernel variant on the
// four large workloads on MI355X, taken with an earlier copy path (loads that
// wrote LDS directly, overlapped with the stage's products); with the
// register-path copies it still ranks variants to within about 9%, and
// conv2d_tune chooses among the best-ranked ones by measurement:
//   matrix: per unit (16 k values) each wave issues MB x NBW blocks of four
//   fp32 instructions of 32 cycles (or half an f16 pair instruction of 16
//   cycles); the waves of a SIMD add up, at an efficiency set by how many
//   waves share the SIMD, plus the LDS latency the SIMD's waves cannot hide;
//   copies: a stage's buffer at kCopyBytesPerCycle, overlapped with the
//   stage's products;
//   fixed costs per stage (barrier, copy issue and wait) and per tile (set-up,
//   first copies, epilogue; cm variants add the column-tap sums).
// A two-per-CU variant that shares its CU (share = 2) gets half of every
// SIMD, and part of its stage overheads hides behind the other workgroup.
double simd_efficiency(int wps) { return wps >= 3 ? 1.0 : wps == 2 ? 0.9 : 0.4; }

constexpr double kUnitLatency = 500.0;        // exposed LDS latency per unit and SIMD
constexpr double kStageCycles = 2000.0;       // barrier, copy issue and wait per stage
constexpr double kTileCycles = 45000.0;       // set-up, first copies, epilogue
constexpr double kCopyBytesPerCycle = 12.0;   // stage copies, per CU
constexpr double kSharedStageVisible = 0.4;   // stage overhead left when sharing a CU
constexpr double kCmEpilogueCycles = 4000.0;   // cm: rows through LDS, column-tap sums
constexpr int64_t kMaxExtraTiles = 3;          // tiles per band beyond the fewest

// Blocks per wave the kernel multiplies for a tile of `pts` lanes in use,
// averaged over the waves along pixels: a wave whose last block holds no
// lane in use runs NBW - 1 blocks, any other NBW (mm_body).
double active_blocks(const Variant& v, int64_t pts) {
  double sum = 0.0;
  for (int ng = 0; ng < v.wn; ++ng) {
    int nact = 0;
    for (int b = 0; b < v.nbw; ++b)
      if ((int64_t(b) * v.wn + ng) * 16 < pts) nact = b + 1;
    sum += (v.nbw > 1 && nact == v.nbw - 1) ? v.nbw - 1 : v.nbw;
  }
  return sum / v.wn;
}

// Taps of a class's contraction: row taps (cm), every kernel tap (the
// multi-class union), or the class's taps.
int64_t stage_taps(const PhaseDesc& d, const Variant& v) {
  return v.cm ? int64_t(d.th) : d.mct > 0 ? int64_t(d.mct) : int64_t(d.th) * d.tw;
}

double tile_cost(const PhaseDesc& d, int64_t Co, const Variant& v, int share) {
  (void)Co;
  if (d.th == 0) return kTileCycles;
  const int64_t ntaps = stage_taps(d, v);
  const double wps = v.wm * v.wn / 4.0;
  const double nbw = v.cm ? double(v.nbw) : active_blocks(v, d.ntv);
  const double mfma = wps * v.mb * nbw * (v.f16 ? 8.0 : 128.0) * share;
  const double lds = 8.0 * v.wm * v.wn * (nbw + v.mb) * share;
  const double unit = std::max(mfma, lds) / simd_efficiency(int(wps * share)) +
                      kUnitLatency / std::max(1.0, wps * share);
  const double copy = double(stage_floats(v)) * 4.0 / kCopyBytesPerCycle * share;
  const double stage = kStageCycles * (share == 2 ? kSharedStageVisible : 1.0);
  double cycles = kTileCycles + (v.cm ? kCmEpilogueCycles : 0.0);
  for (int64_t g = 0; g < d.ngroups; ++g) {
    const int64_t ntg = std::min<int64_t>(d.tg, ntaps - g * d.tg);
    const int64_t u = int64_t(d.cg) * ntg;
    const double units = v.f16 ? 2.0 * double(ceil_div(u, 2)) : double(u);
    cycles += double(d.nchunks) * (std::max(units * unit, copy) + stage);
  }
  return cycles;
}

// Stage shape and tiling of one class for variant v: the (taps, channel
// groups) per stage and the band/tile sizes that fit the LDS stage buffer
// with the lowest cost per pixel.  False if nothing fits.
bool tile_class(PhaseDesc* d, const Variant& v, int64_t Co, int64_t OHOW, int64_t cstride,
                int64_t extra) {
  const int64_t ntl = 16 * int64_t(v.nbw) * v.wn, mt = 16 * int64_t(v.wm) * v.mb;
  if (d->th == 0) {                                   // zero class: stores only
    d->wb = d->wp;
    d->nbands = 1;
    d->ntv = int32_t(std::min<int64_t>(ntl, int64_t(d->hp) * d->wp));
    if (v.cm)   // whole rows
      d->ntv = int32_t(std::min<int64_t>(d->hp, std::max<int64_t>(1, ntl / d->wp)) * d->wp);
    d->ptiles = int32_t(ceil_div(int64_t(d->hp) * d->wp, d->ntv));
    d->cg = d->tg = d->ngroups = d->nchunks = d->slots = d->pt = d->qp = d->wfl = d->used = 0;
    return true;
  }
  const int64_t ntaps = stage_taps(*d, v);
  const int64_t cg_useful = std::max<int64_t>(1, ceil_div(Co, 16));
  bool found = false;
  double best = 0.0;
  PhaseDesc out = *d;
  int64_t last_tg = -1;
  // a multi-class stage holds every tap (one tap group)
  for (int64_t ng = ceil_div(ntaps, kMaxStageTaps); ng <= (d->mct > 0 ? 1 : ntaps); ++ng) {
    const int64_t tg = ceil_div(ntaps, ng);         // fewest taps for this group count
    if (tg == last_tg) continue;
    last_tg = tg;
    const int64_t pt = tg | 1;
    const int64_t qp = ceil_div(mt * pt * 4, 64) * 64;
    for (int64_t cg = 1; cg <= std::min<int64_t>(kMaxStageGroups, cg_useful); ++cg) {
      // byte ranges of a stage's buffer resources stay below 2^31
      if (16 * cg * OHOW * 4 >= kI31 || 16 * cg * cstride * 4 >= kI31) break;
      const int64_t wt = 4 * cg * qp;
      const int64_t max_slots = (stage_floats(v) - wt) / (16 * cg) / 16 * 16;
      if (max_slots < 16) break;
      // band candidates: the planner's own choice, or (cm) every band count
      // up to 8
      const int64_t ncand = v.cm ? std::min<int64_t>(8, d->wp) : 1;
      for (int64_t nb = 1; nb <= ncand; ++nb) {
      PhaseDesc c = *d;
      int64_t wb, ntv, slots;
      if (v.cm) {
        int64_t rows;
        if (!cm_tiling(c, nb, ntl, max_slots, &wb, &rows, &slots)) continue;
        ntv = rows * wb;
      } else if (!choose_tiling(c, ntl, max_slots, extra, &wb, &ntv, &slots)) {
        continue;
      }
      c.wb = int32_t(wb);
      c.nbands = int32_t(ceil_div(c.wp, wb));
      c.ntv = int32_t(ntv);
      c.ptiles = int32_t(ceil_div(int64_t(c.hp) * wb, ntv));
      c.cg = int32_t(cg);
      c.tg = int32_t(tg);
      c.ngroups = int32_t(ceil_div(ntaps, tg));
      c.nchunks = int32_t(ceil_div(Co, 16 * cg));
      c.slots = int32_t(slots);
      c.pt = int32_t(pt);
      c.qp = int32_t(qp);
      c.wfl = int32_t(16 * cg * slots);
      c.used = int32_t(16 * cg * slots + wt);
      if (stage_batches(c) > v.wm * v.wn * batches_per_wave(v)) continue;
      const double per_px = tile_cost(c, Co, v, v.half ? 2 : 1) / double(ntv);
      if (!found || per_px < best * 0.999) {
        found = true;
        best = per_px;
        out = c;
      }
      }
    }
  }
  if (found) *d = out;
  return found;
}

// Largest-first makespan of the tiles over `cus` compute units.
double lpt_makespan(const std::vector<PhaseDesc>& phases, int64_t per_class_mult,
                    const std::vector<double>& costs, int cus) {
  int64_t total_tiles = 0;
  double total_cost = 0.0, max_cost = 0.0;
  for (size_t i = 0; i < phases.size(); ++i) {
    const int64_t t = int64_t(phases[i].ptiles) * phases[i].nbands * per_class_mult;
    total_tiles += t;
    total_cost += t * costs[i];
    max_cost = std::max(max_cost, costs[i]);
  }
  if (total_tiles > (int64_t(1) << 16)) return total_cost / cus + max_cost;
  std::vector<double> load(size_t(cus), 0.0);   // min-heap of CU loads
  std::vector<size_t> order(phases.size());
  for (size_t i = 0; i < order.size(); ++i) order[i] = i;
  std::stable_sort(order.begin(), order.end(),
                   [&](size_t a, size_t b) { return costs[a] > costs[b]; });
  auto cmp = [](double a, double b) { return a > b; };
  for (size_t oi : order) {
    const int64_t t = int64_t(phases[oi].ptiles) * phases[oi].nbands * per_class_mult;
    for (int64_t k = 0; k < t; ++k) {
      std::pop_heap(load.begin(), load.end(), cmp);
      load.back() += costs[oi];
      std::push_heap(load.begin(), load.end(), cmp);
    }
  }
  return *std::max_element(load.begin(), load.end());
}

}  // namespace

int build_plan(const conv2d_params* p, int f16, int num_cus, std::vector<LaunchArgs>* launches,
               conv2d_plan_info* info, int force_variant, double* model_cost, int op) {
  int rc = validate_shape(p);
  if (rc != CONV2D_OK) return rc;
  if (op != kOpGradInput && op != kOpForward) return CONV2D_ERR_UNSUPPORTED;
  if (info) std::memset(info, 0, sizeof(*info));
  const bool fwd = op == kOpForward;
  const int64_t N = p->batch, Ci = p->in_channels, H = p->in_h, W = p->in_w;
  const int64_t Co = p->out_channels;
  const int64_t KHW = int64_t(p->kernel_h) * p->kernel_w;
  if (info) info->useful_macs = N * Co * p->out_h * p->out_w * Ci * KHW;
  if (force_variant >= kNumVariants || (force_variant >= 0 && kVariants[force_variant].f16 != (f16 ? 1 : 0)))
    return CONV2D_ERR_UNSUPPORTED;
  if (force_variant >= 0 && fwd && kVariants[force_variant].cm) return CONV2D_ERR_UNSUPPORTED;
  // nothing to write: an empty output (the forward output is empty only
  // with no image or no output channel; Ci = 0 or an empty input still
  // writes zeros)
  if (fwd ? (N == 0 || Co == 0) : (N == 0 || Ci == 0 || H == 0 || W == 0)) return CONV2D_OK;
  if (num_cus < 1) num_cus = kDefaultCUs;
  const int64_t OHOW = int64_t(p->out_h) * p->out_w;
  // roles (plan.hpp): matrix rows, contraction channels, source plane, and
  // weight elements between contraction channels
  const int64_t Mch = fwd ? Co : Ci;
  const int64_t Kch = fwd ? Ci : Co;
  const int64_t src_plane = fwd ? H * W : OHOW;
  const int64_t cstride = fwd ? KHW : Ci * KHW;
  // a forward stage's weight buffer reaches to the end of the tensor
  if (fwd && Co * Ci * KHW * 4 >= kI31) return CONV2D_ERR_OVERFLOW;

  std::vector<PhaseDesc> classes;
  if (fwd) make_forward_class(p, &classes);
  else make_classes(p, &classes);
  // cm variants: matrix rows per input channel (the widest class's column
  // taps) and input channels per tile
  const int64_t twm = ceil_div(p->kernel_w, p->stride);
  const int64_t cm_cit = twm <= 16 ? 16 / twm : 0;
  auto channels_per_tile = [&](const Variant& var) {
    return var.cm ? cm_cit : 16 * int64_t(var.wm) * var.mb;
  };
  // the four classes of a stride-2 input gradient as one multi-class tiling
  std::vector<PhaseDesc> mc_union(1);
  MCClass mcls[kMCClasses];
  std::memset(mcls, 0, sizeof(mcls));
  const bool mc_ok = !fwd && !f16 && make_mc_union(p, classes, &mc_union[0], mcls);

  int best_v = -1;
  double best_cost = 0.0;
  std::vector<PhaseDesc> best;
  for (int v = 0; v < kNumVariants; ++v) {
    const Variant& var = kVariants[v];
    if (force_variant >= 0 ? v != force_variant : var.f16 != (f16 ? 1 : 0)) continue;
    if (fwd && var.cm) continue;
    if (var.mc && !mc_ok) continue;
    const std::vector<PhaseDesc>& vclasses = var.mc ? mc_union : classes;
    const int64_t vmt = channels_per_tile(var);
    if (vmt < 1) continue;
    // Each class with the fewest tiles per band, or up to kMaxExtraTiles
    // more (cm variants tile whole rows: fewest only).  Shapes with up to
    // four classes try every combination of per-class choices (so that a
    // light class can take smaller tiles that fill the CUs the heavy classes
    // leave idle); others try the same choice for every class.
    const int64_t emax = var.cm ? 0 : kMaxExtraTiles;
    const size_t nc = vclasses.size();
    std::vector<PhaseDesc> cand(nc * size_t(emax + 1));
    std::vector<char> fits(nc * size_t(emax + 1), 0);
    for (size_t i = 0; i < nc; ++i)
      for (int64_t e = 0; e <= emax; ++e) {
        PhaseDesc d = vclasses[i];
        fits[i * size_t(emax + 1) + size_t(e)] =
            tile_class(&d, var, Kch, src_plane, cstride, e) ? 1 : 0;
        cand[i * size_t(emax + 1) + size_t(e)] = d;
      }
    const bool per_class = nc > 1 && nc <= 4;
    int64_t combos = emax + 1;
    if (per_class)
      for (size_t i = 1; i < nc; ++i) combos *= emax + 1;
    for (int64_t code = 0; code < combos; ++code) {
      std::vector<PhaseDesc> phases(nc);
      bool ok = true;
      int64_t rest = code;
      for (size_t i = 0; i < nc && ok; ++i) {
        int64_t e = code;
        if (per_class) {
          e = rest % (emax + 1);
          rest /= emax + 1;
        }
        ok = fits[i * size_t(emax + 1) + size_t(e)] != 0;
        phases[i] = cand[i * size_t(emax + 1) + size_t(e)];
      }
      if (!ok) continue;
      // a two-per-CU variant only shares its CU when there are more tiles
      // than CUs
      int64_t ntiles = 0;
      for (const PhaseDesc& d : phases)
        ntiles += N * d.nbands * int64_t(d.ptiles) * ceil_div(Mch, vmt);
      const int share = (var.half && ntiles > num_cus) ? 2 : 1;
      std::vector<double> costs;
      for (const PhaseDesc& d : phases) costs.push_back(tile_cost(d, Kch, var, share));
      const double cost = lpt_makespan(phases, N * ceil_div(Mch, vmt), costs, num_cus * share);
      if (best_v < 0 || cost < best_cost * 0.999) {
        best_v = v;
        best_cost = cost;
        best = phases;
      }
    }
  }
  if (best_v < 0) return CONV2D_ERR_UNSUPPORTED;
  if (model_cost) *model_cost = best_cost;

  const Variant& bv = kVariants[best_v];
  const int64_t bmt = 16 * int64_t(bv.wm) * bv.mb;   // matrix rows per tile
  const int64_t bcit = channels_per_tile(bv);
  const int64_t bci = ceil_div(Mch, bcit);
  for (PhaseDesc& d : best) {
    const int64_t tiles = N * d.nbands * int64_t(d.ptiles) * bci;
    if (tiles >= kI31) return CONV2D_ERR_OVERFLOW;
    d.tiles = int32_t(tiles);
    if (info) {
      info->phases += bv.mc ? kMCClasses : 1;
      if (d.th == 0) info->zero_phases += 1;
      if (d.th > 0) {
        // lanes the kernel multiplies: blocks past a short wave's last one
        // are skipped (mm_body); a multi-class tile multiplies each class's
        // blocks at that class's taps, kH x kW taps in all
        const double blocks = bv.cm ? double(bv.nbw) : active_blocks(bv, d.ntv);
        const int64_t lanes = int64_t(16.0 * blocks * bv.wn + 0.5);
        const int64_t kpad = int64_t(d.nchunks) * 16 * d.cg * stage_taps(d, bv);
        info->macs += tiles * lanes * bmt * kpad;
      }
    }
  }
  std::stable_sort(best.begin(), best.end(), [&](const PhaseDesc& a, const PhaseDesc& b) {
    return tile_cost(a, Kch, bv, 1) > tile_cost(b, Kch, bv, 1);
  });
  return emit_launches(p, bci, bcit, twm, best_v, best, launches, info, op, mcls);
}

}  // namespace c2b

namespace c2b {
// Plan summary of a shape on the 1x1 GEMM (one launch, one phase).
void describe_pw(const conv2d_params* p, int fwd, conv2d_plan_info* out) {
  std::memset(out, 0, sizeof(*out));
  out->launches = 1;
  out->phases = 1;
  pw::pw_describe(p, &out->tiles, &out->macs, fwd);
  out->useful_macs = int64_t(p->batch) * p->out_channels * p->out_h * p->out_w *
                     p->in_channels;
}
}  // namespace c2b

extern "C" int conv2d_check_params(const conv2d_params* p) {
  int rc = c2b::build_plan(p, 0, c2b::kDefaultCUs, nullptr, nullptr);
  if (rc != CONV2D_OK) return rc;
  return c2b::build_plan(p, 1, c2b::kDefaultCUs, nullptr, nullptr);
}

extern "C" int conv2d_describe_plan(const conv2d_params* p, int f16,
                                    conv2d_plan_info* out) {
  if (out == nullptr) return CONV2D_ERR_NULL_PTR;
  if (c2b::pw::pw_route(p, 0, f16 ? 1 : 0)) {   // the 1x1 GEMM over all images' pixels
    c2b::describe_pw(p, 0, out);
    return CONV2D_OK;
  }
  return c2b::build_plan(p, f16 ? 1 : 0, c2b::kDefaultCUs, nullptr, out);
}

extern "C" int conv2d_describe_plan_variant(const conv2d_params* p, int variant,
                                            conv2d_plan_info* out) {
  if (p == nullptr || out == nullptr) return CONV2D_ERR_NULL_PTR;
  if (variant < 0 || variant >= c2b::kNumVariants) return CONV2D_ERR_UNSUPPORTED;
  return c2b::build_plan(p, c2b::kVariants[variant].f16, c2b::kDefaultCUs, nullptr, out,
                         variant);
}

extern "C" int conv2d_describe_forward_plan(const conv2d_params* p, int f16,
                                            conv2d_plan_info* out) {
  if (out == nullptr) return CONV2D_ERR_NULL_PTR;
  if (c2b::pw::pw_route(p, 1, f16 ? 1 : 0)) {
    c2b::describe_pw(p, 1, out);
    return CONV2D_OK;
  }
  return c2b::build_plan(p, f16 ? 1 : 0, c2b::kDefaultCUs, nullptr, out, -1, nullptr,
                         c2b::kOpForward);
}

extern "C" int conv2d_describe_forward_plan_variant(const conv2d_params* p, int variant,
                                                    conv2d_plan_info* out) {
  if (p == nullptr || out == nullptr) return CONV2D_ERR_NULL_PTR;
  if (variant < 0 || variant >= c2b::kNumVariants) return CONV2D_ERR_UNSUPPORTED;
  return c2b::build_plan(p, c2b::kVariants[variant].f16, c2b::kDefaultCUs, nullptr, out,
                         variant, nullptr, c2b::kOpForward);
}

extern "C" int conv2d_num_variants(void) { return c2b::kNumVariants; }

extern "C" int conv2d_variant_is_f16(int variant) {
  if (variant < 0 || variant >= c2b::kNumVariants) return CONV2D_ERR_UNSUPPORTED;
  return c2b::kVariants[variant].f16;
}

extern "C" int conv2d_variant_uses_column_taps(int variant) {
  if (variant < 0 || variant >= c2b::kNumVariants) return CONV2D_ERR_UNSUPPORTED;
  return c2b::kVariants[variant].cm;
}

extern "C" int conv2d_variant_is_multi_class(int variant) {
  if (variant < 0 || variant >= c2b::kNumVariants) return CONV2D_ERR_UNSUPPORTED;
  return c2b::kVariants[variant].mc;
}

extern "C" const char* conv2d_status_string(int status) {
  switch (status) {
    case CONV2D_OK: return "ok";
    case CONV2D_ERR_NULL_PTR: return "null pointer";
    case CONV2D_ERR_BAD_SHAPE:
      return "bad shape: stride/kernel 0, padded input smaller than the kernel, "
             "or out_h/out_w not the forward-convolution extents";
    case CONV2D_ERR_ALIAS: return "grad_input overlaps grad_out or weight";
    case CONV2D_ERR_OVERFLOW: return "size exceeds 32-bit per-image indexing";
    case CONV2D_ERR_UNSUPPORTED:
      return "kernel window of one stride phase too large for the staging tile, "
             "or kernel variant not available for this path";
    case CONV2D_ERR_HIP: return "HIP runtime error at launch";
    case CONV2D_ERR_WORKSPACE: return "workspace smaller than conv2d_grad_weight_workspace_size";
    case CONV2D_ERR_SCRATCH:
      return "shape needs more scratch than the allocation-free entry point holds "
             "(CONV2D_GRAD_WEIGHT_NOALLOC_MAX_BYTES)";
    default: return "unknown status";
  }
}
