// Host-side replay of the input-gradient kernels' addressing (no device code
// runs here).  For one shape it walks every workgroup and thread of every
// launch the plan makes and checks, with the same index functions the
// kernels use (tile_index.hpp):
//  * every global read of grad_out and weight lies inside its tensor, and the
//    element read is the one the gather rule asks for;
//  * every LDS index lies inside its array, and the window slot a pixel reads
//    for tap (j, l) holds grad_out[oh = i' + ch - j, ow = j' + cw - l];
//  * the weight cell a k-step reads belongs to the same tap as the window
//    offset it is multiplied with;
//  * every grad_input element is written by exactly one lane, and only by a
//    lane whose pixel block ran the contraction.
#include <cstdio>
#include <cstring>
#include <string>
#include <utility>
#include <vector>

#include "tile_index.hpp"

namespace c2b {
namespace {

struct Failure {
  std::string msg;
};

#define C2B_REQUIRE(cond, ...)                                  \
  do {                                                          \
    if (!(cond)) {                                              \
      char buf_[512];                                           \
      std::snprintf(buf_, sizeof buf_, __VA_ARGS__);            \
      throw Failure{std::string(#cond) + ": " + buf_};          \
    }                                                           \
  } while (0)

template <bool F16>
void check_launch(const LaunchArgs& a, std::vector<unsigned char>& written) {
  constexpr TileShape ts = F16 ? kF16Tile : kF32Tile;
  using G = KernelGeom<F16, ts.mt, ts.ck, ts.taps, ts.slab>;
  constexpr int MT = ts.mt, CK = ts.ck, TAPS = ts.taps, SLAB = ts.slab;
  const int64_t OHOW = int64_t(a.OH) * a.OW;
  const int64_t go_size = int64_t(a.N) * a.Co * OHOW;
  const int64_t cstride = int64_t(a.Ci) * a.KH * a.KW;
  const int64_t w_size = int64_t(a.Co) * cstride;
  const int64_t HW = int64_t(a.H) * a.W;

  for (int bid = 0; bid < a.total_tiles; ++bid) {
    const TileCtx c = decode_tile<MT>(a, bid, CK);
    const PhaseDesc& P = c.P;
    C2B_REQUIRE(c.n >= 0 && c.n < a.N, "bid %d n %d", bid, c.n);
    C2B_REQUIRE(c.band >= 0 && c.band < P.nbands, "bid %d band %d", bid, c.band);
    C2B_REQUIRE(c.ci0 >= 0 && c.ci0 < a.Ci, "bid %d ci0 %d", bid, c.ci0);
    C2B_REQUIRE(c.npx >= 1 && c.npx <= P.ntv && P.ntv <= ts.nt, "bid %d npx %d", bid, c.npx);
    if (c.ntaps > 0) C2B_REQUIRE(c.R * c.roww <= SLAB, "bid %d window %d", bid, c.R * c.roww);

    for (int tid = 0; tid < kThreads; ++tid) {
      const int lane = tid & 63, wave = tid >> 6, h = lane >> 5, l32 = lane & 31;
      // window copy: global reads and LDS writes
      int goff[G::kHS];
      for (int k = 0; k < G::kHS; ++k) {
        const int f = tid + kThreads * k;
        goff[k] = window_slot_offset(c, a, f);
        if (goff[k] >= 0) {
          C2B_REQUIRE(goff[k] < OHOW, "goff %d", goff[k]);
          const int oh = goff[k] / a.OW, ow = goff[k] % a.OW;
          C2B_REQUIRE(oh == c.oh_base + f / c.roww && ow == c.ow_base + f % c.roww,
                      "window slot %d", f);
        }
        if (f < SLAB)
          for (int cg = 0; cg < G::kNCG; ++cg)
            C2B_REQUIRE(cg * SLAB + f < G::kLdsH, "sH write %d", cg * SLAB + f);
      }
      // weight copy
      for (int st = 0; st < c.nstages; ++st) {
        int co0, g;
        stage_split(c, CK, st, &co0, &g);
        for (int co = 0; co < CK; ++co)
          for (int k = 0; k < G::kHS; ++k)
            if (co0 + co < a.Co && goff[k] >= 0) {
              const int64_t gi = int64_t(c.n) * a.Co * OHOW + int64_t(co0 + co) * OHOW + goff[k];
              C2B_REQUIRE(gi >= 0 && gi < go_size, "grad_out read %lld", (long long)gi);
            }
        for (int k = 0; k < G::kWS; ++k) {
          const int e = tid + kThreads * k;
          const int woff = weight_cell_offset<MT, G::kNCG, TAPS, G::kCPC>(c, a, e, g);
          const int lds_cell = weight_cell_lds<MT, G::kNCG, G::kPitch>(e);
          if (e < G::kAE) C2B_REQUIRE(lds_cell < G::kLdsA, "sA write %d", lds_cell);
          if (woff < 0) continue;
          const int cc = co0 + weight_cell_channel<MT, G::kNCG, G::kCPC>(e);
          const int t = e / (G::kNCG * MT), ci = e % MT;
          const int tap = g * TAPS + t;
          for (int v = 0; v < G::kCPC; ++v) {
            if (cc + v >= a.Co) continue;
            const int64_t wi = int64_t(co0) * cstride + woff + int64_t(v) * cstride;
            C2B_REQUIRE(wi >= 0 && wi < w_size, "weight read %lld", (long long)wi);
            const int64_t want = (int64_t(cc + v) * a.Ci + c.ci0 + ci) * a.KH * a.KW +
                                 tap_kidx(P, a, tap);
            C2B_REQUIRE(wi == want, "weight element %lld vs %lld", (long long)wi,
                        (long long)want);
          }
        }
      }
      // contraction reads
      const int first = wave * 64;
      const int nact = first >= c.npx ? 0 : (first + 32 >= c.npx ? 1 : 2);
      const int abase = h * G::kPitch + l32;
      int bbase[2], base[2];
      for (int nb = 0; nb < 2; ++nb) {
        base[nb] = window_base(c, first + nb * 32 + l32);
        bbase[nb] = h * SLAB + base[nb];
      }
      for (int st = 0; st < c.nstages; ++st) {
        int co0, g;
        stage_split(c, CK, st, &co0, &g);
        const int tap0 = g * TAPS;
        const int ntg = imin(TAPS, c.ntaps - tap0);
        int j = tap0 / P.tw, l = tap0 - (tap0 / P.tw) * P.tw;
        for (int tt = 0; tt < ntg; ++tt) {
          C2B_REQUIRE(j * P.tw + l == tap0 + tt, "tap order");
          const int boff = tap_window_offset(c, j, l);
          for (int ks = 0; ks < G::kKSteps; ++ks) {
            const int ai = abase + (tt * G::kNCG + 2 * ks) * G::kPitch;
            C2B_REQUIRE(ai >= 0 && ai + 32 < G::kLdsA, "sA read %d", ai);
            for (int nb = 0; nb < nact; ++nb) {
              const int bi = bbase[nb] + boff + 2 * ks * SLAB;
              C2B_REQUIRE(bi >= 0 && bi < G::kLdsH, "sH read %d", bi);
              const int slot = base[nb] + boff;
              C2B_REQUIRE(slot >= 0 && slot < SLAB, "slot %d", slot);
              const int local = first + nb * 32 + l32;
              if (local < c.npx) {
                C2B_REQUIRE(slot < c.R * c.roww, "slot %d beyond window", slot);
                const int q = c.p0 + local, ip = q / P.wb, jj = c.band * P.wb + q % P.wb;
                C2B_REQUIRE(c.oh_base + slot / c.roww == ip + P.ch - j &&
                                c.ow_base + slot % c.roww == jj + P.cw - l,
                            "tap (%d,%d) reads the wrong grad_out element", j, l);
              }
            }
          }
          if (++l == P.tw) {
            l = 0;
            ++j;
          }
        }
      }
      // epilogue
      for (int nb = 0; nb < 2; ++nb) {
        const int local = first + nb * 32 + l32;
        const int po = output_offset(c, a, local);
        if (po < 0) continue;
        C2B_REQUIRE(nb < nact || c.nstages == 0 || c.ntaps == 0,
                    "pixel stored from a block that did not run");
        const int ih = po / a.W, iw = po % a.W;
        C2B_REQUIRE(((ih + a.PH) % a.S) == P.rh && ((iw + a.PW) % a.S) == P.rw,
                    "pixel (%d,%d) outside class (%d,%d)", ih, iw, P.rh, P.rw);
        for (int mb = 0; mb < 2; ++mb)
          for (int r = 0; r < 16; ++r) {
            const int ci = c.ci0 + mb * 32 + acc_row(r, h);
            if (ci >= a.Ci) continue;
            const int64_t gi = int64_t(c.n) * a.Ci * HW + int64_t(ci) * HW + po;
            C2B_REQUIRE(gi >= 0 && gi < int64_t(written.size()), "grad_input write");
            C2B_REQUIRE(written[gi] == 0, "grad_input element %lld written twice",
                        (long long)gi);
            written[gi] = 1;
          }
      }
    }
  }
}

// fp32 family (grad_input_f32_kernel<WM, NBW>): window and weights are
// copied by buffer loads that write LDS directly (64 consecutive floats per
// wave-instruction), double-buffered.
template <int WM, int WN, int NBW>
void check_launch_f32(const LaunchArgs& a, std::vector<unsigned char>& written) {
  using G = F32Geom<WM, WN, NBW>;
  constexpr int MT = G::kMT, NT = G::kThreads, CH = kF32StageCh;
  const int64_t OHOW = int64_t(a.OH) * a.OW;
  const int64_t go_size = int64_t(a.N) * a.Co * OHOW;
  const int64_t KHW = int64_t(a.KH) * a.KW;
  const int64_t cstride = int64_t(a.Ci) * KHW;
  const int64_t w_size = int64_t(a.Co) * cstride;
  const int64_t HW = int64_t(a.H) * a.W;

  for (int bid = 0; bid < a.total_tiles; ++bid) {
    const TileCtx c = decode_tile<MT>(a, bid, 0);
    const PhaseDesc& P = c.P;
    C2B_REQUIRE(c.n >= 0 && c.n < a.N, "bid %d n %d", bid, c.n);
    C2B_REQUIRE(c.band >= 0 && c.band < P.nbands, "bid %d band %d", bid, c.band);
    C2B_REQUIRE(c.ci0 >= 0 && c.ci0 < a.Ci, "bid %d ci0 %d", bid, c.ci0);
    C2B_REQUIRE(c.npx >= 1 && c.npx <= P.ntv && P.ntv <= G::kNTL, "bid %d npx %d", bid, c.npx);
    const int SLOTS = P.slabr, CP = P.cp, TG = P.tg;
    const int fcount = CH * SLOTS, ecount = CH * CP;
    if (c.ntaps > 0) {
      C2B_REQUIRE(P.ckr == CH && TG >= 1 && TG <= kF32StageTaps, "stage shape");
      C2B_REQUIRE(c.R * c.roww <= SLOTS && SLOTS <= kF32MaxSlots && SLOTS % 16 == 0,
                  "bid %d window %d > %d", bid, c.R * c.roww, SLOTS);
      C2B_REQUIRE(CP >= MT * TG && CP % 16 == 4 && CP <= kF32MaxCP, "weight pitch %d", CP);
      C2B_REQUIRE(fcount <= kF32WinFloats && ecount <= kF32WtFloats, "stage exceeds buffers");
      C2B_REQUIRE(int64_t(CH) * OHOW * 4 < (int64_t(1) << 31) &&
                      int64_t(CH) * cstride * 4 < (int64_t(1) << 31),
                  "stage byte range");
    }
    for (int tid = 0; tid < NT; ++tid) {
      const int lane = tid & 63, wave = tid >> 6;
      const int mg = wave % WM, ng = wave / WM, g = lane >> 4, c16 = lane & 15;
      for (int st = 0; st < c.nstages; ++st) {
        int co0, grp;
        stage_split(c, CH, st, &co0, &grp);
        const int nco = imin(CH, a.Co - co0);
        C2B_REQUIRE(nco >= 1, "stage %d without channels", st);
        // window cells
        for (int k = 0; k < G::kHS; ++k) {
          const int f0 = wave * 64 + NT * k, f = tid + NT * k;
          if (f0 >= kF32WinFloats) continue;            // instruction not issued
          C2B_REQUIRE(f == f0 + lane && f < kF32WinFloats, "window lds %d", f);
          const int o = f32_window_cell(c, a, f);
          if (f >= fcount) C2B_REQUIRE(o < 0, "cell past the window reads memory");
          if (o < 0 || int64_t(o) >= int64_t(nco) * OHOW) continue;   // reads 0
          const int cq = f / (4 * SLOTS), r = f % (4 * SLOTS);
          const int slot = r / 4, ch = 4 * cq + r % 4;
          C2B_REQUIRE(ch < nco && slot < c.R * c.roww, "cell %d", f);
          const int oh = c.oh_base + slot / c.roww, ow = c.ow_base + slot % c.roww;
          C2B_REQUIRE(o == ch * OHOW + int64_t(oh) * a.OW + ow, "window element");
          const int64_t gi = int64_t(c.n) * a.Co * OHOW + int64_t(co0) * OHOW + o;
          C2B_REQUIRE(gi >= 0 && gi < go_size, "grad_out read %lld", (long long)gi);
        }
        const int tap0 = grp * TG;
        const int ntg = imin(TG, c.ntaps - tap0);
        C2B_REQUIRE(ntg >= 1, "stage without taps");
        // weight cells
        for (int k = 0; k < G::kWS; ++k) {
          const int e0 = wave * 64 + NT * k, e = tid + NT * k;
          if (e0 >= kF32WtFloats) continue;             // instruction not issued
          C2B_REQUIRE(e == e0 + lane && e < kF32WtFloats, "weight lds %d", e);
          const int o = f32_weight_cell<MT>(c, a, e, grp);
          if (e >= ecount) C2B_REQUIRE(o < 0, "cell past the weights reads memory");
          if (o < 0 || int64_t(o) >= int64_t(nco) * cstride) continue;  // reads 0
          const int co = e / CP, r = e % CP, ci = r / TG, t = r % TG;
          C2B_REQUIRE(co < nco && ci < MT && t < ntg, "weight cell %d", e);
          const int64_t want = (int64_t(co0 + co) * a.Ci + c.ci0 + ci) * KHW +
                               tap_kidx(P, a, tap0 + t);
          const int64_t wi = int64_t(co0) * cstride + o;
          C2B_REQUIRE(wi == want && wi >= 0 && wi < w_size, "weight element");
        }
        // contraction reads
        int j = tap0 / P.tw, l = tap0 % P.tw;
        for (int tt = 0; tt < ntg; ++tt) {
          C2B_REQUIRE(j * P.tw + l == tap0 + tt, "tap order");
          for (int q = 0; q < 4; ++q) {
            const int ai = 4 * g * CP + (mg * 16 + c16) * TG + q * CP + tt;
            C2B_REQUIRE(ai >= 0 && ai < ecount, "weight read %d", ai);
            C2B_REQUIRE(ai / CP == 4 * g + q && (ai % CP) / TG == mg * 16 + c16 &&
                            (ai % CP) % TG == tt,
                        "weight of k-step");
          }
          for (int b = 0; b < NBW; ++b) {
            const int local = f32_local(b, ng, c16, WN);
            const int base = window_base(c, local);
            const int slot = base + tap_window_offset(c, j, l);
            const int byte = (g * SLOTS + base) * 16 + tap_window_offset(c, j, l) * 16;
            C2B_REQUIRE(byte >= 0 && byte % 16 == 0 && byte + 16 <= fcount * 4, "window read %d",
                        byte);
            C2B_REQUIRE(slot >= 0 && slot < SLOTS && byte / 16 == g * SLOTS + slot,
                        "slot %d", slot);
            if (local < c.npx) {
              C2B_REQUIRE(slot < c.R * c.roww, "slot beyond window");
              const int qq = c.p0 + local, ip = qq / P.wb, jj = c.band * P.wb + qq % P.wb;
              C2B_REQUIRE(c.oh_base + slot / c.roww == ip + P.ch - j &&
                              c.ow_base + slot % c.roww == jj + P.cw - l,
                          "tap (%d,%d) reads the wrong grad_out element", j, l);
            }
          }
          if (++l == P.tw) {
            l = 0;
            ++j;
          }
        }
      }
      // epilogue
      for (int b = 0; b < NBW; ++b) {
        const int po = output_offset(c, a, f32_local(b, ng, c16, WN));
        if (po < 0) continue;
        const int ih = po / a.W, iw = po % a.W;
        C2B_REQUIRE(((ih + a.PH) % a.S) == P.rh && ((iw + a.PW) % a.S) == P.rw,
                    "pixel (%d,%d) outside class", ih, iw);
        for (int r = 0; r < 4; ++r) {
          const int cc = c.ci0 + mg * 16 + 4 * g + r;
          if (cc >= a.Ci) continue;
          const int64_t gi = int64_t(c.n) * a.Ci * HW + int64_t(cc) * HW + po;
          C2B_REQUIRE(gi >= 0 && gi < int64_t(written.size()), "grad_input write");
          C2B_REQUIRE(written[gi] == 0, "grad_input element %lld written twice", (long long)gi);
          written[gi] = 1;
        }
      }
    }
  }
}

template <int V>
void check_f32_variant(const LaunchArgs& la, std::vector<unsigned char>& written) {
  constexpr F32Variant v = kF32Variants[V];
  check_launch_f32<v.wm, v.wn, v.nbw>(la, written);
}

template <int... Vs>
void check_f32_dispatch(const LaunchArgs& la, std::vector<unsigned char>& written,
                        std::integer_sequence<int, Vs...>) {
  ((la.variant == Vs ? check_f32_variant<Vs>(la, written) : void()), ...);
}

template <bool F16>
int check_all(const conv2d_params* p, char* msg, size_t len, int variant) {
  std::vector<LaunchArgs> launches;
  int rc = F16 ? build_plan(p, kF16Tile, &launches, nullptr)
               : build_plan_f32(p, kF32DefaultCUs, &launches, nullptr, variant);
  if (rc != CONV2D_OK) return rc;
  const int64_t n_gi = int64_t(p->batch) * p->in_channels * p->in_h * p->in_w;
  std::vector<unsigned char> written(size_t(n_gi), 0);
  try {
    for (const LaunchArgs& la : launches) {
      if (F16)
        check_launch<true>(la, written);
      else
        check_f32_dispatch(la, written, std::make_integer_sequence<int, kNumF32Variants>());
    }
    for (int64_t i = 0; i < n_gi; ++i)
      C2B_REQUIRE(written[i] == 1, "grad_input element %lld never written", (long long)i);
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

}  // namespace
}  // namespace c2b

extern "C" int conv2d_check_indexing(const conv2d_params* p, int f16, char* msg,
                                     size_t msg_len) {
  return f16 ? c2b::check_all<true>(p, msg, msg_len, -1)
             : c2b::check_all<false>(p, msg, msg_len, -1);
}

extern "C" int conv2d_check_indexing_variant(const conv2d_params* p, int variant, char* msg,
                                             size_t msg_len) {
  if (variant < 0 || variant >= c2b::kNumF32Variants) return CONV2D_ERR_UNSUPPORTED;
  return c2b::check_all<false>(p, msg, msg_len, variant);
}

extern "C" int conv2d_num_f32_variants(void) { return c2b::kNumF32Variants; }
