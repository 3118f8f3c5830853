// Host-side validation and launch planning (no HIP call in this file).
//
// Shape rules follow the `Params` struct of the shader this library
// re-designs (meganeura 0.2.0, conv2d_grad_input_gemm_coop.wgsl): one stride
// for both axes, separate paddings, out_h / out_w passed in.  Here out_h and
// out_w must equal the forward-convolution extents, so that grad_input is the
// exact adjoint of that forward convolution.
#include <algorithm>
#include <cstdint>
#include <cstring>

#include "plan.hpp"
#include "tile_index.hpp"

namespace c2b {

namespace {

constexpr int64_t kI31 = int64_t(1) << 31;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// First index i >= 0 with (i + pad) mod s == r.
int64_t first_of_class(int64_t r, int64_t pad, int64_t s) {
  return (((r - pad) % s) + s) % s;
}

// Choose band width and pixels per tile for a class whose halo window must
// fit `slab` elements per output channel.  Rows spanned by `ntv` consecutive
// pixels of a band `wb` wide are at most floor((wb + ntv - 2) / wb) + 1; the
// window adds th - 1 rows above and tw - 1 columns to the left.
bool choose_band(int64_t wp, int64_t th, int64_t tw, const TileShape& ts,
                 int64_t* wb_out, int64_t* ntv_out) {
  for (int64_t ntv = ts.nt; ntv >= 1; ntv /= 2) {
    // fewest bands first; ceil(wp / nb) keeps bands nearly equal
    int64_t last_wb = -1;
    for (int64_t nb = 1; nb <= wp; ++nb) {
      int64_t wb = ceil_div(wp, nb);
      if (wb == last_wb) continue;
      last_wb = wb;
      int64_t rows = (wb + ntv - 2) / wb + th;
      int64_t roww = wb + tw - 1;
      if (rows * roww <= ts.slab) {
        *wb_out = wb;
        *ntv_out = ntv;
        return true;
      }
      if (wb == 1) break;
    }
  }
  return false;
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
                   const conv2d_params* p) {
  if (p == nullptr) return CONV2D_ERR_NULL_PTR;
  const uint64_t n_gi = uint64_t(p->batch) * p->in_channels * p->in_h * p->in_w;
  const uint64_t n_go = uint64_t(p->batch) * p->out_channels * p->out_h * p->out_w;
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

static LaunchArgs launch_header(const conv2d_params* p, int64_t ciblocks) {
  LaunchArgs la;
  std::memset(&la, 0, sizeof(la));
  la.N = int32_t(p->batch);
  la.Ci = int32_t(p->in_channels);
  la.H = int32_t(p->in_h);
  la.W = int32_t(p->in_w);
  la.Co = int32_t(p->out_channels);
  la.KH = int32_t(p->kernel_h);
  la.KW = int32_t(p->kernel_w);
  la.S = int32_t(p->stride);
  la.PH = int32_t(p->padding_h);
  la.PW = int32_t(p->padding_w);
  la.OH = int32_t(p->out_h);
  la.OW = int32_t(p->out_w);
  la.ciblocks = int32_t(ciblocks);
  return la;
}

// Reciprocals of a class's per-lane divisors, and the bounds under which the
// kernels' fast_div is exact (numerator x divisor < 2^31): numerators are
// window cells (< 16 * slots or the tile window), taps, and positions inside
// a band row plus one tile of pixels.
static int finalize_divisors(PhaseDesc* d) {
  const int64_t roww = int64_t(d->wb) + d->tw - 1;
  const int64_t lim = int64_t(1) << 31;
  const int64_t wb = d->wb, tw = std::max(d->tw, 1);
  const int64_t slots4 = std::max<int64_t>(4 * int64_t(d->slabr), 1);
  const int64_t cp = std::max(d->cp, 1), tg = std::max(d->tg, 1);
  const int64_t win = std::max<int64_t>(int64_t(kF32StageCh) * d->slabr, 4096);
  if (roww >= 1 && win * roww >= lim) return CONV2D_ERR_OVERFLOW;
  if ((wb + d->ntv + 1024) * wb >= lim) return CONV2D_ERR_OVERFLOW;
  if (int64_t(d->th) * d->tw * tw >= lim) return CONV2D_ERR_OVERFLOW;
  d->m_roww = fast_div_magic(uint32_t(std::max<int64_t>(roww, 1)));
  d->m_wb = fast_div_magic(uint32_t(wb));
  d->m_tw = fast_div_magic(uint32_t(tw));
  d->m_slots4 = fast_div_magic(uint32_t(slots4));
  d->m_cp = fast_div_magic(uint32_t(cp));
  d->m_tg = fast_div_magic(uint32_t(tg));
  return CONV2D_OK;
}

// Split classes (already sorted heaviest first) into launches of at most
// kMaxPhasesPerLaunch classes.
static int emit_launches(const conv2d_params* p, int64_t ciblocks, int variant,
                         const std::vector<PhaseDesc>& phases,
                         std::vector<LaunchArgs>* launches, conv2d_plan_info* info) {
  for (size_t base = 0; base < phases.size(); base += kMaxPhasesPerLaunch) {
    LaunchArgs la = launch_header(p, ciblocks);
    la.variant = variant;
    int64_t total = 0;
    const size_t end = std::min(phases.size(), base + kMaxPhasesPerLaunch);
    for (size_t i = base; i < end; ++i) {
      PhaseDesc d = phases[i];
      const int rc = finalize_divisors(&d);
      if (rc != CONV2D_OK) return rc;
      d.tile_begin = int32_t(total);
      total += d.tiles;
      if (total >= kI31) return CONV2D_ERR_OVERFLOW;
      la.ph[la.nphases++] = d;
    }
    la.total_tiles = int32_t(total);
    if (launches) launches->push_back(la);
    if (info) {
      info->launches += 1;
      info->tiles += total;
    }
  }
  return CONV2D_OK;
}

int build_plan(const conv2d_params* p, const TileShape& ts,
               std::vector<LaunchArgs>* launches, conv2d_plan_info* info) {
  int rc = validate_shape(p);
  if (rc != CONV2D_OK) return rc;
  if (info) std::memset(info, 0, sizeof(*info));

  const int64_t N = p->batch, Ci = p->in_channels, H = p->in_h, W = p->in_w;
  const int64_t Co = p->out_channels;
  if (info) info->useful_macs = N * Co * p->out_h * p->out_w * Ci * p->kernel_h * p->kernel_w;
  if (N == 0 || Ci == 0 || H == 0 || W == 0) return CONV2D_OK;  // nothing to write

  const int64_t ciblocks = ceil_div(Ci, ts.mt);
  std::vector<PhaseDesc> phases;
  make_classes(p, &phases);
  for (PhaseDesc& d : phases) {
    const int64_t th = d.th, tw = d.tw, hp = d.hp, wp = d.wp;
    int64_t wb = wp, ntv = ts.nt;
    if (th > 0) {
      if (!choose_band(wp, th, tw, ts, &wb, &ntv)) return CONV2D_ERR_UNSUPPORTED;
      d.ngroups = int32_t(ceil_div(th * tw, ts.taps));
    }
    d.wb = int32_t(wb);
    d.nbands = int32_t(ceil_div(wp, wb));
    d.ntv = int32_t(ntv);
    const int64_t ptiles = ceil_div(hp * wb, ntv);
    const int64_t tiles = N * d.nbands * ptiles * ciblocks;
    if (ptiles >= kI31 || tiles >= kI31) return CONV2D_ERR_OVERFLOW;
    d.ptiles = int32_t(ptiles);
    d.tiles = int32_t(tiles);
    if (info) {
      info->phases += 1;
      if (d.th == 0) info->zero_phases += 1;
      // issued MACs: whole channel tiles, 32-pixel blocks, whole stages
      const int64_t band_px = hp * wb;
      const int64_t full = band_px / ntv, rem = band_px % ntv;
      const int64_t lanes = full * ceil_div(ntv, 32) * 32 + ceil_div(rem, 32) * 32;
      const int64_t kk = ceil_div(Co, ts.ck) * ts.ck * th * tw;
      info->macs += N * d.nbands * lanes * ciblocks * ts.mt * kk;
    }
  }
  // heaviest classes first: they start first and the light ones fill the tail
  std::stable_sort(phases.begin(), phases.end(), [](const PhaseDesc& a, const PhaseDesc& b) {
    return int64_t(a.th) * a.tw > int64_t(b.th) * b.tw;
  });
  return emit_launches(p, ciblocks, 0, phases, launches, info);
}

// ---------------------------------------------------------------------------
// fp32 kernel family planning.

namespace {

// Most grad_out rows a run of `ntv` consecutive pixels touches in a band
// `wb` wide, over all tiles p0 = k*ntv of a band of `bp` pixels.
int64_t max_rows_spanned(int64_t wb, int64_t ntv, int64_t bp) {
  if (ntv % wb == 0) return ntv / wb;               // tiles start on row starts
  const int64_t tiles = ceil_div(bp, ntv);
  int64_t best = 0;
  if (tiles <= 4096) {
    for (int64_t t = 0; t < tiles; ++t) {
      const int64_t p0 = t * ntv, p1 = std::min(p0 + ntv, bp) - 1;
      best = std::max(best, p1 / wb - p0 / wb + 1);
    }
    return best;
  }
  return (wb + ntv - 2) / wb + 1;                    // worst case over starts
}

struct F32Choice {
  std::vector<PhaseDesc> phases;
  double cost = 0.0;
};

// LDS floats per output channel of staged weights for mt channels x tg
// taps: at least mt*tg, = 4 mod 16.
int64_t weight_pitch(int64_t mt, int64_t tg) {
  int64_t x = mt * tg;
  return x + ((4 - x % 16) + 16) % 16;
}

// Tile one class for a variant; false if no band/tile size fits LDS.
bool tile_class_f32(PhaseDesc* d, int64_t ntl, int64_t mt) {
  const int64_t th = d->th, tw = d->tw, hp = d->hp, wp = d->wp;
  if (th == 0) {                                      // zero class: stores only
    d->wb = d->wp;
    d->nbands = 1;
    d->ntv = int32_t(std::min<int64_t>(ntl, hp * wp));
    d->ptiles = int32_t(ceil_div(hp * wp, d->ntv));
    d->ngroups = d->ckr = d->tg = d->slabr = d->cp = 0;
    return true;
  }
  const int64_t ntaps = th * tw;
  // taps per stage: as many as fit, the weights of a stage in LDS
  int64_t tg = std::min<int64_t>(ntaps, kF32StageTaps);
  while (tg > 1 && weight_pitch(mt, tg) > kF32MaxCP) --tg;
  const int64_t cp = weight_pitch(mt, tg);
  if (cp > kF32MaxCP) return false;
  const int64_t max_slots = kF32MaxSlots;
  int64_t last_wb = -1;
  for (int64_t nb = 1; nb <= wp; ++nb) {
    const int64_t wb = ceil_div(wp, nb);
    if (wb == last_wb) continue;
    last_wb = wb;
    const int64_t bp = hp * wb;
    const int64_t roww = wb + tw - 1;
    // equal tiles of at most ntl pixels first, then halve the tile
    for (int64_t cap = ntl;; cap = (cap + 1) / 2) {
      const int64_t ntv = ceil_div(bp, ceil_div(bp, cap));
      const int64_t rows = max_rows_spanned(wb, ntv, bp) + th - 1;
      // the four channel quads of a window start 16*slots floats apart; a
      // multiple of 256 bytes keeps 16-byte reads free of bank conflicts
      const int64_t slots = ceil_div(rows * roww, 16) * 16;
      if (slots <= max_slots) {
        d->wb = int32_t(wb);
        d->nbands = int32_t(ceil_div(wp, wb));
        d->ntv = int32_t(ntv);
        d->ptiles = int32_t(ceil_div(bp, ntv));
        d->slabr = int32_t(slots);
        d->cp = int32_t(cp);
        d->ckr = kF32StageCh;
        d->tg = int32_t(tg);
        d->ngroups = int32_t(ceil_div(ntaps, tg));
        return true;
      }
      if (cap <= 1 || ntv <= wb / 4) break;           // more tiles will not help
    }
    if (wb == 1) break;
  }
  return false;
}

// Matrix-unit efficiency reached with `wn` waves per SIMD (measured on the
// tap loop: more waves hide more of the LDS latency between taps).
double simd_efficiency(int wn) { return wn >= 4 ? 0.88 : wn == 3 ? 0.85 : wn == 2 ? 0.75 : 0.6; }

// Relative cost of one tile: matrix work of the waves sharing a SIMD (wn
// waves x NBW blocks x padded k values / efficiency) plus per-stage and
// per-tile overheads.
double tile_cost_f32(const PhaseDesc& d, int64_t Co, const F32Variant& v) {
  const double tile_overhead = 20000.0;               // cycles: set-up, epilogue
  if (d.th == 0) return tile_overhead;
  const int64_t ntaps = int64_t(d.th) * d.tw;
  const int64_t kpad = ceil_div(Co, d.ckr) * d.ckr * ntaps;
  const int64_t stages = ceil_div(Co, d.ckr) * d.ngroups;
  // 16x16x4 fp32 takes 32 cycles of a SIMD's matrix unit
  return double(v.wn) * v.nbw * (kpad / 4) * 32.0 / simd_efficiency(v.wn) + stages * 600.0 +
         tile_overhead;
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
  std::stable_sort(order.begin(), order.end(), [&](size_t a, size_t b) { return costs[a] > costs[b]; });
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

int build_plan_f32(const conv2d_params* p, int num_cus, std::vector<LaunchArgs>* launches,
                   conv2d_plan_info* info, int force_variant) {
  int rc = validate_shape(p);
  if (rc != CONV2D_OK) return rc;
  if (info) std::memset(info, 0, sizeof(*info));
  const int64_t N = p->batch, Ci = p->in_channels, H = p->in_h, W = p->in_w;
  const int64_t Co = p->out_channels;
  if (info) info->useful_macs = N * Co * p->out_h * p->out_w * Ci * p->kernel_h * p->kernel_w;
  if (N == 0 || Ci == 0 || H == 0 || W == 0) return CONV2D_OK;
  if (num_cus < 1) num_cus = kF32DefaultCUs;

  std::vector<PhaseDesc> classes;
  make_classes(p, &classes);
  const int wm = Ci > 64 ? 8 : 4;

  int best_v = -1;
  F32Choice best;
  for (int v = 0; v < kNumF32Variants; ++v) {
    if (force_variant >= 0 ? v != force_variant : kF32Variants[v].wm != wm) continue;
    const int64_t vmt = 16 * int64_t(kF32Variants[v].wm);
    const int64_t ntl = 16 * int64_t(kF32Variants[v].nbw) * kF32Variants[v].wn;
    F32Choice ch;
    ch.phases = classes;
    bool ok = true;
    std::vector<double> costs;
    for (PhaseDesc& d : ch.phases) {
      if (!tile_class_f32(&d, ntl, vmt)) {
        ok = false;
        break;
      }
      costs.push_back(tile_cost_f32(d, Co, kF32Variants[v]));
    }
    if (!ok) continue;
    ch.cost = lpt_makespan(ch.phases, N * ceil_div(Ci, vmt), costs, num_cus);
    if (best_v < 0 || ch.cost < best.cost * 0.999) {
      best_v = v;
      best = ch;
    }
  }
  if (best_v < 0) return CONV2D_ERR_UNSUPPORTED;

  const F32Variant bv = kF32Variants[best_v];
  const int64_t bmt = 16 * int64_t(bv.wm);
  const int64_t bci = ceil_div(Ci, bmt);
  for (PhaseDesc& d : best.phases) {
    const int64_t tiles = N * d.nbands * int64_t(d.ptiles) * bci;
    if (tiles >= kI31) return CONV2D_ERR_OVERFLOW;
    d.tiles = int32_t(tiles);
    if (info) {
      info->phases += 1;
      if (d.th == 0) info->zero_phases += 1;
      if (d.th > 0) {
        const int64_t lanes = 16 * int64_t(bv.nbw) * bv.wn;
        const int64_t kpad = ceil_div(Co, d.ckr) * d.ckr * int64_t(d.th) * d.tw;
        info->macs += tiles * lanes * bmt * kpad;
      }
    }
  }
  std::stable_sort(best.phases.begin(), best.phases.end(),
                   [&](const PhaseDesc& a, const PhaseDesc& b) {
                     return tile_cost_f32(a, Co, bv) > tile_cost_f32(b, Co, bv);
                   });
  return emit_launches(p, bci, best_v, best.phases, launches, info);
}

}  // namespace c2b

extern "C" int conv2d_check_params(const conv2d_params* p) {
  int rc = c2b::build_plan_f32(p, c2b::kF32DefaultCUs, nullptr, nullptr);
  if (rc != CONV2D_OK) return rc;
  return c2b::build_plan(p, c2b::kF16Tile, nullptr, nullptr);
}

extern "C" int conv2d_describe_plan(const conv2d_params* p, int f16,
                                    conv2d_plan_info* out) {
  if (out == nullptr) return CONV2D_ERR_NULL_PTR;
  if (f16) return c2b::build_plan(p, c2b::kF16Tile, nullptr, out);
  return c2b::build_plan_f32(p, c2b::kF32DefaultCUs, nullptr, out);
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
      return "kernel window of one stride phase too large for the staging tile";
    case CONV2D_ERR_HIP: return "HIP runtime error at launch";
    default: return "unknown status";
  }
}
