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

int build_plan(const conv2d_params* p, const TileShape& ts,
               std::vector<LaunchArgs>* launches, conv2d_plan_info* info) {
  int rc = validate_shape(p);
  if (rc != CONV2D_OK) return rc;
  if (info) std::memset(info, 0, sizeof(*info));

  const int64_t N = p->batch, Ci = p->in_channels, H = p->in_h, W = p->in_w;
  const int64_t Co = p->out_channels, KH = p->kernel_h, KW = p->kernel_w;
  const int64_t S = p->stride, PH = p->padding_h, PW = p->padding_w;
  const int64_t OH = p->out_h, OW = p->out_w;
  if (info) info->useful_macs = N * Co * OH * OW * Ci * KH * KW;
  if (N == 0 || Ci == 0 || H == 0 || W == 0) return CONV2D_OK;  // nothing to write

  const int64_t ciblocks = ceil_div(Ci, ts.mt);
  std::vector<PhaseDesc> phases;
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
      int64_t wb = wp, ntv = ts.nt;
      if (th > 0 && tw > 0) {
        d.th = int32_t(th);
        d.tw = int32_t(tw);
        d.ch = int32_t((ih0 + PH - rh) / S);
        d.cw = int32_t((iw0 + PW - rw) / S);
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
      phases.push_back(d);
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
  }
  // heaviest classes first: they start first and the light ones fill the tail
  std::stable_sort(phases.begin(), phases.end(),
                   [](const PhaseDesc& a, const PhaseDesc& b) {
                     return int64_t(a.th) * a.tw > int64_t(b.th) * b.tw;
                   });
  for (size_t base = 0; base < phases.size(); base += kMaxPhasesPerLaunch) {
    LaunchArgs la;
    std::memset(&la, 0, sizeof(la));
    la.N = int32_t(N);
    la.Ci = int32_t(Ci);
    la.H = int32_t(H);
    la.W = int32_t(W);
    la.Co = int32_t(Co);
    la.KH = int32_t(KH);
    la.KW = int32_t(KW);
    la.S = int32_t(S);
    la.PH = int32_t(PH);
    la.PW = int32_t(PW);
    la.OH = int32_t(OH);
    la.OW = int32_t(OW);
    la.ciblocks = int32_t(ciblocks);
    int64_t total = 0;
    const size_t end = std::min(phases.size(), base + kMaxPhasesPerLaunch);
    for (size_t i = base; i < end; ++i) {
      PhaseDesc d = phases[i];
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

}  // namespace c2b

extern "C" int conv2d_check_params(const conv2d_params* p) {
  return c2b::build_plan(p, c2b::kF32Tile, nullptr, nullptr);
}

extern "C" int conv2d_describe_plan(const conv2d_params* p, int f16,
                                    conv2d_plan_info* out) {
  if (out == nullptr) return CONV2D_ERR_NULL_PTR;
  return c2b::build_plan(p, f16 ? c2b::kF16Tile : c2b::kF32Tile, nullptr, out);
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
