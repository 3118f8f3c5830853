// Host-side replay of the input-gradient kernel's addressing (no device code
// runs here).  For one shape it walks every workgroup and thread of every
// launch the plan makes and checks, with the same index functions the kernel
// uses (tile_index.hpp):
//  * every copy instruction fills 64 consecutive floats inside one region
//    (window or weights) of its stage buffer, every global element it reads
//    lies inside its tensor and is the one the gather rule asks for, and
//    every padding cell's offset lies beyond its buffer's range (so it reads
//    0) without wrapping;
//  * every LDS read lies inside its region, and for a real pixel the window
//    cell a unit reads holds grad_out[oh = i' + ch - j, ow = j' + cw - l] of
//    the unit's output channels, while the weight cell it is multiplied with
//    holds the same output channels at the same tap;
//  * every grad_input element is written by exactly one lane.
#include <cstdio>
#include <cstring>
#include <string>
#include <utility>
#include <vector>

#include "pointwise.hpp"
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

template <int WM, int WN, int MB, int NBW, int SF, bool CM, bool MC>
void check_launch(const LaunchArgs& a, const conv2d_params& prm,
                  std::vector<unsigned char>& written) {
  using G = MMGeom<WM, WN, MB, NBW, SF>;
  constexpr int kStageFloats = SF;
  constexpr int MT = G::kMT, NT = G::kThreads, NW = G::kWaves, NJ = G::kBatches;
  const int64_t OHOW = int64_t(a.OH) * a.OW;
  const int64_t go_size = int64_t(a.N) * a.Co * OHOW;
  const int64_t KHW = int64_t(a.KH) * a.KW;
  const int64_t w_size = int64_t(a.Co) * a.Ci * KHW;   // the same product on both roles
  // forward launches (roles exchanged, plan.hpp): their geometry is checked
  // against the caller's stride and padding, not the launch's own fields
  const bool fwd = a.fwd != 0;
  C2B_REQUIRE(fwd ? (a.wsm == prm.in_channels * KHW && a.wsk == KHW && a.S == 1 && !CM)
                  : (a.wsm == KHW && a.wsk == prm.in_channels * KHW),
              "launch weight strides / roles");
  const int64_t HW = int64_t(a.H) * a.W;

  for (int bid = 0; bid < a.total_tiles; ++bid) {
    const TileCtx c = decode_tile(a, bid);
    const PhaseDesc& P = c.P;
    C2B_REQUIRE(c.n >= 0 && c.n < a.N, "bid %d n %d", bid, c.n);
    C2B_REQUIRE(c.band >= 0 && c.band < P.nbands, "bid %d band %d", bid, c.band);
    C2B_REQUIRE(c.ci0 >= 0 && c.ci0 < a.Ci, "bid %d ci0 %d", bid, c.ci0);
    C2B_REQUIRE(c.npx >= 1 && c.npx <= P.ntv && (CM || P.ntv <= G::kNTL), "bid %d npx %d", bid,
                c.npx);
    C2B_REQUIRE(a.cm == (CM ? 1 : 0) && (CM ? a.cit * a.twm <= MT : a.cit == MT),
                "launch matrix rows: cm %d cit %d twm %d", a.cm, a.cit, a.twm);
    C2B_REQUIRE(a.mc == (MC ? 1 : 0) && (MC ? a.nphases == 1 && P.mct == KHW && a.S == 2 &&
                                                  !fwd && P.ngroups == 1 && P.tg == KHW
                                            : P.mct == 0),
                "multi-class launch fields");
    if (CM) {
      // whole rows of the band per tile, and one lane per window point
      C2B_REQUIRE(c.p0 % P.wb == 0 && c.npx % P.wb == 0, "bid %d: cm tile not whole rows", bid);
      C2B_REQUIRE(c.R - P.th + 1 == c.npx / P.wb, "bid %d: cm window rows", bid);
      C2B_REQUIRE(c.ntaps == 0 || (cm_points(c) <= G::kNTL && P.tw <= a.twm),
                  "bid %d: cm points %d", bid, cm_points(c));
    }
    const int SLOTS = P.slots, QP = P.qp, PT = P.pt, TG = P.tg, CG = P.cg;
    const int CH = 16 * CG;
    if (c.ntaps > 0) {
      C2B_REQUIRE(CG >= 1 && CG <= kMaxStageGroups && TG >= 1 && TG <= kMaxStageTaps,
                  "stage shape cg %d tg %d", CG, TG);
      C2B_REQUIRE(P.ngroups == (c.ntaps + TG - 1) / TG && P.nchunks == (a.Co + CH - 1) / CH,
                  "stage counts");
      C2B_REQUIRE(c.R * c.roww <= SLOTS && SLOTS % 16 == 0, "bid %d window %d > %d", bid,
                  c.R * c.roww, SLOTS);
      C2B_REQUIRE(PT >= TG && PT % 2 == 1 && QP >= MT * PT * 4 && QP % 64 == 0,
                  "weight pitch pt %d qp %d", PT, QP);
      C2B_REQUIRE(P.wfl == CH * SLOTS && P.used == P.wfl + 4 * CG * QP &&
                      P.used <= kStageFloats && P.wfl % 64 == 0 && P.used % 64 == 0,
                  "stage buffer wfl %d used %d", P.wfl, P.used);
      C2B_REQUIRE(int64_t(CH) * OHOW * 4 < (int64_t(1) << 31) &&
                      int64_t(CH) * a.wsk * 4 < (int64_t(1) << 31) &&
                      w_size * 4 < (int64_t(1) << 31),
                  "stage byte range");
    }
    std::vector<unsigned char> covered(size_t(c.nstages) * size_t(c.ntaps > 0 ? P.used : 0), 0);
    std::vector<unsigned char> qrows(CM ? size_t(16) * (16 * NBW * WN + 4) : 0, 0);
    for (int tid = 0; tid < NT; ++tid) {
      const int lane = tid & 63, wave = tid >> 6;
      const int mg = wave % WM, ng = wave / WM, g = lane >> 4, c16 = lane & 15;
      int bb[NBW], aq[MB];
      for (int b = 0; b < NBW; ++b)
        bb[b] = (g * SLOTS + (MC   ? window_pixel(c, mm_local(b, ng, c16, WN))
                              : CM ? window_base_cm(c, mm_local(b, ng, c16, WN))
                                   : window_base(c, mm_local(b, ng, c16, WN)))) * 16;
      for (int m = 0; m < MB; ++m) aq[m] = (g * QP + mm_channel(m, mg, c16, MB) * 4 * PT) * 4;
      for (int st = 0; st < c.nstages; ++st) {
        int co0, grp;
        stage_split(c, st, &co0, &grp);
        const int nco = imin(CH, a.Co - co0);
        C2B_REQUIRE(nco >= 1 && co0 % CH == 0, "stage %d channels", st);
        const int tap0 = grp * TG;
        const int ntg = imin(TG, c.ntaps - tap0);
        C2B_REQUIRE(ntg >= 1 && grp < P.ngroups, "stage %d without taps", st);
        // copies: batch wave + NW*j of this wave (tile_index.hpp); every
        // stage-buffer cell below `used` must be written by exactly one lane
        // of one wave per stage (checked after the last thread below)
        const int NB = stage_batches(P), WB = window_blocks(P);
        C2B_REQUIRE(NB <= NW * NJ, "bid %d: %d copy batches for %d waves", bid, NB, NW);
        for (int j = 0; j < NJ; ++j) {
          const int k = wave + NW * j;
          if (k >= NB) break;
          int block, quad;
          batch_split(P, k, &block, &quad);
          C2B_REQUIRE(block >= 0 && block < copy_blocks(P) && quad >= 0 && quad < 4 * CG,
                      "batch %d split", k);
          const bool win = block < WB;
          const uint32_t off = win ? window_lane_offset(c, a, block, lane)
                                   : weight_lane_offset<MT, CM>(c, a, block - WB, lane, grp);
          const uint32_t ch = win ? window_channel_bytes(a) : weight_channel_bytes(a);
          // the buffer ranges of stage_src: a forward stage's weights run to
          // the end of w, and its channels past nco are cut per load instead
          const int64_t range = win ? int64_t(nco) * OHOW * 4
                                    : fwd ? (w_size - int64_t(co0) * a.wsk) * 4
                                          : int64_t(nco) * a.wsk * 4;
          C2B_REQUIRE(off == kPadOffset || off % 4 == 0, "unaligned copy offset");
          const int f = batch_lds_float(P, block, quad, lane);
          if (f < 0) continue;                               // lane writes nothing
          C2B_REQUIRE(f % 4 == 0 && f + 4 <= (win ? P.wfl : P.used) && (win || f >= P.wfl),
                      "batch %d lane %d writes float %d outside its region", k, lane, f);
          for (int q = 0; q < 4; ++q) {
            const int cell = f + q;
            unsigned char& cov = covered[size_t(st) * size_t(P.used) + size_t(cell)];
            C2B_REQUIRE(cov == 0, "stage %d cell %d written twice", st, cell);
            cov = 1;
            const bool cut = fwd && !win && 4 * quad + q >= nco;   // forward channel guard
            const uint64_t o64 = cut ? uint64_t(kPadOffset) : uint64_t(off) + uint64_t(4 * quad + q) * ch;
            C2B_REQUIRE(o64 < (uint64_t(1) << 32), "copy offset wraps");
            const bool pad = off == kPadOffset || cut;
            C2B_REQUIRE(!pad || int64_t(o64) >= range, "padding cell inside the range");
            const bool reads = !pad && int64_t(o64) < range;
            if (win) {
              const int o = mm_window_cell(c, a, cell);
              if (o < 0 || int64_t(o) >= int64_t(nco) * OHOW) {
                C2B_REQUIRE(!reads, "window cell %d should read 0", cell);
                continue;
              }
              C2B_REQUIRE(reads && int64_t(o64) == int64_t(o) * 4, "window cell %d offset", cell);
              const int cq2 = cell / (4 * SLOTS), r = cell % (4 * SLOTS);
              const int slot = r / 4, chn = 4 * cq2 + r % 4;
              C2B_REQUIRE(chn < nco && slot < c.R * c.roww, "window cell %d", cell);
              const int oh = c.oh_base + slot / c.roww, ow = c.ow_base + slot % c.roww;
              C2B_REQUIRE(oh >= 0 && oh < a.OH && ow >= 0 && ow < a.OW, "window pixel");
              C2B_REQUIRE(o == chn * OHOW + int64_t(oh) * a.OW + ow, "window element");
              const int64_t gi = int64_t(c.n) * a.Co * OHOW + int64_t(co0) * OHOW + o;
              C2B_REQUIRE(gi >= 0 && gi < go_size, "grad_out read %lld", (long long)gi);
            } else {
              const int e = cell - P.wfl;
              const int o = mm_weight_cell<MT, CM>(c, a, e, grp);
              const int cch = 4 * (e / QP) + (e % QP) % 4;   // the cell's contraction channel
              if (o < 0 || cch >= nco) {
                C2B_REQUIRE(!reads, "weight cell %d should read 0", e);
                continue;
              }
              C2B_REQUIRE(reads && int64_t(o64) == int64_t(o) * 4, "weight cell %d offset", e);
              const int cq2 = e / QP, r = e % QP, m = r / (4 * PT), t = (r % (4 * PT)) / 4;
              const int co = 4 * cq2 + r % 4;
              C2B_REQUIRE(co < nco && m < MT && t < ntg, "weight cell %d", e);
              // matrix row m: input channel ci0 + m at tap tap0 + t of the
              // class, or (cm) channel ci0 + m / twm at row tap tap0 + t and
              // column tap m mod twm
              int64_t want;
              if (fwd) {
                // w[co, ci, kh, kw] with co = matrix row, ci = contraction
                // channel, and the flipped tap kh = KH-1-j, kw = KW-1-l
                const int tap = tap0 + t, jt = tap / P.tw, lt = tap % P.tw;
                want = ((int64_t(c.ci0 + m) * prm.in_channels + co0 + co) * a.KH +
                        (a.KH - 1 - jt)) * a.KW + (a.KW - 1 - lt);
              } else if (CM) {
                const int cl = m / a.twm, l = m % a.twm, jt = tap0 + t;
                C2B_REQUIRE(l < P.tw && cl < a.cit && jt < P.th, "cm weight cell %d", e);
                want = (int64_t(co0 + co) * a.Ci + c.ci0 + cl) * KHW +
                       (P.rh + a.S * jt) * a.KW + (P.rw + a.S * l);
              } else if (MC) {
                // every kernel tap in the weight's own order
                want = (int64_t(co0 + co) * a.Ci + c.ci0 + m) * KHW + tap0 + t;
              } else {
                want = (int64_t(co0 + co) * a.Ci + c.ci0 + m) * KHW + tap_kidx(P, a, tap0 + t);
              }
              const int64_t wi = int64_t(co0) * a.wsk + o;
              C2B_REQUIRE(wi == want && wi >= 0 && wi < w_size, "weight element");
            }
          }
        }
        if (MC) {
          // multi-class unit reads, in the kernel's order: for each channel
          // group, class and class tap, the class's blocks at its window
          // offset and the weights of kernel tap (rh + 2j, rw + 2l); the
          // classes' taps must cover every kernel tap once
          std::vector<int> tap_seen(size_t(KHW), 0);
          for (int cgi = 0; cgi < CG; ++cgi)
            for (int k = 0; k < kMCClasses; ++k) {
              const MCClass& K = a.mcls[k];
              for (int j = 0; j < K.th; ++j)
                for (int l = 0; l < K.tw; ++l) {
                  const int kh = K.rh + 2 * j, kw = K.rw + 2 * l, kidx = kh * a.KW + kw;
                  C2B_REQUIRE(kh < a.KH && kw < a.KW, "class %d tap (%d,%d)", k, j, l);
                  if (cgi == 0) ++tap_seen[size_t(kidx)];
                  const int ao = cgi * QP * 16 + kidx * 16;
                  for (int m = 0; m < MB; ++m) {
                    const int byte = aq[m] + ao;
                    C2B_REQUIRE(byte >= 0 && byte % 16 == 0 && byte + 16 <= 4 * CG * QP * 4,
                                "weight read %d", byte);
                    const int e = byte / 4, cq = e / QP, r = e % QP;
                    C2B_REQUIRE(cq == 4 * cgi + g && r / (4 * PT) == mm_channel(m, mg, c16, MB) &&
                                    (r % (4 * PT)) / 4 == kidx && r % 4 == 0,
                                "weight of unit");
                  }
                  const int wo = cgi * SLOTS * 64 + (K.e * c.roww + K.f) * 16 +
                                 tap_window_offset(c, j, l) * 16;
                  for (int b = 0; b < NBW; ++b) {
                    const int byte = bb[b] + wo;
                    C2B_REQUIRE(byte >= 0 && byte % 16 == 0 && byte + 16 <= P.wfl * 4,
                                "window read %d", byte);
                    const int cell = byte / 16, cq = cell / SLOTS, slot = cell % SLOTS;
                    C2B_REQUIRE(cq == 4 * cgi + g && slot < c.R * c.roww,
                                "window read of class %d outside the window", k);
                    const int local = mm_local(b, ng, c16, WN);
                    const int po = mc_output_offset(c, a, K, local);
                    if (po < 0) continue;
                    // the gather rule: grad_out row (ih + padding_h - kh) / 2
                    const int ih = po / a.W, iw = po % a.W;
                    const int row = c.oh_base + slot / c.roww, col = c.ow_base + slot % c.roww;
                    C2B_REQUIRE(2 * row == ih + a.PH - kh && 2 * col == iw + a.PW - kw,
                                "class %d tap (%d,%d) reads the wrong grad_out element", k, j,
                                l);
                  }
                }
            }
          for (int64_t t = 0; t < KHW; ++t)
            C2B_REQUIRE(tap_seen[size_t(t)] == 1, "kernel tap %d taken %d times", int(t),
                        tap_seen[size_t(t)]);
          continue;
        }
        // unit reads, in the kernel's order (cm: row taps only)
        const int twl = CM ? 1 : P.tw;
        const int j0 = tap0 / twl, l0 = tap0 % twl;
        int cgi = 0, t = 0, j = j0, l = l0;
        for (int u = 0; u < CG * ntg; ++u) {
          C2B_REQUIRE(cgi < CG && j * twl + l == tap0 + t, "unit order");
          const int wo = cgi * SLOTS * 64 + tap_window_offset(c, j, l) * 16;
          const int ao = cgi * QP * 16 + t * 16;
          for (int m = 0; m < MB; ++m) {
            const int byte = aq[m] + ao;
            C2B_REQUIRE(byte >= 0 && byte % 16 == 0 && byte + 16 <= 4 * CG * QP * 4,
                        "weight read %d", byte);
            const int e = byte / 4, cq = e / QP, r = e % QP;
            C2B_REQUIRE(cq == 4 * cgi + g && r / (4 * PT) == mm_channel(m, mg, c16, MB) &&
                            (r % (4 * PT)) / 4 == t && r % 4 == 0,
                        "weight of unit");
          }
          for (int b = 0; b < NBW; ++b) {
            const int byte = bb[b] + wo;
            C2B_REQUIRE(byte >= 0 && byte % 16 == 0 && byte + 16 <= P.wfl * 4, "window read %d",
                        byte);
            const int cell = byte / 16, cq = cell / SLOTS, slot = cell % SLOTS;
            C2B_REQUIRE(cq == 4 * cgi + g, "window quad of unit");
            const int local = mm_local(b, ng, c16, WN);
            if (CM) {
              if (local < cm_points(c)) {
                // point (r, u) at row tap j: grad_out row i' + ch - j, window column u
                const int r = local / c.roww, uu = local % c.roww;
                C2B_REQUIRE(slot < c.R * c.roww && l == 0, "slot beyond window");
                C2B_REQUIRE(c.oh_base + slot / c.roww == c.i_start + r + P.ch - j &&
                                slot % c.roww == uu,
                            "row tap %d reads the wrong grad_out element", j);
              }
            } else if (local < c.npx) {
              C2B_REQUIRE(slot < c.R * c.roww, "slot beyond window");
              const int qq = c.p0 + local, ip = qq / P.wb, jj = c.band * P.wb + qq % P.wb;
              const int row = c.oh_base + slot / c.roww, col = c.ow_base + slot % c.roww;
              if (fwd) {
                // forward definition: output pixel (ip, jj) at kernel tap
                // (KH-1-j, KW-1-l) reads x[s*ip - padding_h + kh, ...]
                C2B_REQUIRE(row == int(prm.stride) * ip - int(prm.padding_h) + (a.KH - 1 - j) &&
                                col == int(prm.stride) * jj - int(prm.padding_w) + (a.KW - 1 - l),
                            "forward tap (%d,%d) reads the wrong x element", j, l);
              } else {
                C2B_REQUIRE(row == ip + P.ch - j && col == jj + P.cw - l,
                            "tap (%d,%d) reads the wrong grad_out element", j, l);
              }
            }
          }
          if (++t == ntg) {
            t = 0;
            ++cgi;
            j = j0;
            l = l0;
          } else if (++l == twl) {
            l = 0;
            ++j;
          }
        }
      }
      if (CM) {
        // cm epilogue, part 1: matrix row 4g + r of block b goes to LDS float
        // (4g + r) * QR + point
        constexpr int QR = 16 * NBW * WN + 4;
        C2B_REQUIRE(16 * QR <= 2 * SF, "cm rows exceed the stage buffers");
        if (c.ntaps > 0)
          for (int b = 0; b < NBW; ++b) {
            const int local = mm_local(b, ng, c16, WN);
            for (int r = 0; r < 4; ++r) {
              const int f = (4 * g + r) * QR + local;
              C2B_REQUIRE(f >= 0 && f < 16 * QR && local < QR - 4, "cm row write %d", f);
              C2B_REQUIRE(qrows[size_t(f)] == 0, "cm row cell %d written twice", f);
              qrows[size_t(f)] = 1;
            }
          }
        continue;   // part 2 (the column-tap sums) runs per tile below
      }
      if (MC) {
        // the kernel's paired stores: row class hk's two classes at a grid
        // point write the even and odd column of one input row; each must be
        // the pixel its class holds there (mc_output_offset) and inside it
        for (int hk = 0; hk < 2; ++hk)
          for (int b = 0; b < NBW; ++b) {
            const int local = mm_local(b, ng, c16, WN);
            int ih, col0;
            bool even_ok, odd_ok;
            const bool any = mc_pair_pixel(c, a, hk, local, &ih, &col0, &even_ok, &odd_ok);
            for (int kk = 0; kk < 2; ++kk) {
              const int k = 2 * hk + kk;
              const int po_k = mc_output_offset(c, a, a.mcls[k], local);
              const bool even_k = a.mcls[k].iw0 == 0;
              const bool ok_k = any && (even_k ? even_ok : odd_ok);
              C2B_REQUIRE(ok_k == (po_k >= 0), "class %d store mask", k);
              if (ok_k)
                C2B_REQUIRE(po_k == ih * a.W + col0 + (even_k ? 0 : 1) && col0 % 2 == 0,
                            "class %d store position", k);
            }
          }
        // every class's pixels at the tile's grid points
        for (int k = 0; k < kMCClasses; ++k) {
          const MCClass& K = a.mcls[k];
          for (int b = 0; b < NBW; ++b) {
            const int po = mc_output_offset(c, a, K, mm_local(b, ng, c16, WN));
            if (po < 0) continue;
            const int ih = po / a.W, iw = po % a.W;
            C2B_REQUIRE(((ih + a.PH) % 2) == K.rh && ((iw + a.PW) % 2) == K.rw && ih < a.H &&
                            iw < a.W,
                        "pixel (%d,%d) outside class %d", ih, iw, k);
            for (int m = 0; m < MB; ++m)
              for (int r = 0; r < 4; ++r) {
                const int cc = c.ci0 + (mg * MB + m) * 16 + 4 * g + r;
                if (cc >= a.Ci) continue;
                const int64_t gi = int64_t(c.n) * a.Ci * HW + int64_t(cc) * HW + po;
                C2B_REQUIRE(gi >= 0 && gi < int64_t(written.size()), "grad_input write");
                C2B_REQUIRE(written[gi] == 0, "grad_input element %lld written twice",
                            (long long)gi);
                written[gi] = 1;
              }
          }
        }
        continue;
      }
      // epilogue
      for (int b = 0; b < NBW; ++b) {
        const int po = output_offset(c, a, mm_local(b, ng, c16, WN));
        if (po < 0) continue;
        const int ih = po / a.W, iw = po % a.W;
        C2B_REQUIRE(fwd || (((ih + a.PH) % a.S) == P.rh && ((iw + a.PW) % a.S) == P.rw),
                    "pixel (%d,%d) outside class", ih, iw);
        for (int m = 0; m < MB; ++m)
          for (int r = 0; r < 4; ++r) {
            const int cc = c.ci0 + (mg * MB + m) * 16 + 4 * g + r;
            if (cc >= a.Ci) continue;
            const int64_t gi = int64_t(c.n) * a.Ci * HW + int64_t(cc) * HW + po;
            C2B_REQUIRE(gi >= 0 && gi < int64_t(written.size()), "grad_input write");
            C2B_REQUIRE(written[gi] == 0, "grad_input element %lld written twice",
                        (long long)gi);
            written[gi] = 1;
          }
      }
    }
    for (size_t i = 0; i < covered.size(); ++i)
      C2B_REQUIRE(covered[i] == 1, "bid %d: stage %d cell %d never copied", bid,
                  int(i / size_t(P.used)), int(i % size_t(P.used)));
    if (CM) {
      // cm epilogue, part 2: every class pixel (i', j') of the tile, for every
      // channel of the tile, adds matrix row cl*twm + l at point
      // (r, j'' + tw - 1 - l) over its tw column taps l; that point's window
      // column must be the grad_out column j' + cw - l of the gather rule,
      // and the row must hold channel ci0 + cl at column tap l
      constexpr int QR = 16 * NBW * WN + 4;
      const int rows = c.R - P.th + 1;
      for (int cl = 0; cl < a.cit && c.ci0 + cl < a.Ci; ++cl)
        for (int q = 0; q < rows * P.wb; ++q) {
          const int r = q / P.wb, jj = q % P.wb, col = c.band * P.wb + jj;
          if (col >= P.wp) continue;
          for (int l = 0; c.ntaps > 0 && l < P.tw; ++l) {
            const int pt = r * c.roww + jj + P.tw - 1 - l, m = cl * a.twm + l;
            C2B_REQUIRE(pt >= 0 && pt < cm_points(c) && m < MT, "cm sum point %d", pt);
            C2B_REQUIRE(qrows[size_t(m) * QR + pt] == 1, "cm sum reads an unwritten row cell");
            C2B_REQUIRE(c.ow_base + pt % c.roww == col + P.cw - l, "cm column tap %d", l);
            // weight_source of row m at any row tap is channel ci0 + cl, column l
            const int src = weight_source<MT, CM>(c, a, m, 0, 0);
            C2B_REQUIRE(src >= 0 && src / (a.KH * a.KW) == c.ci0 + cl &&
                            (src % (a.KH * a.KW)) % a.KW == P.rw + a.S * l,
                        "cm row %d is not channel %d column tap %d", m, c.ci0 + cl, l);
          }
          const int ih = P.ih0 + a.S * (c.i_start + r), iw = P.iw0 + a.S * col;
          C2B_REQUIRE(ih < a.H && iw < a.W, "cm pixel (%d,%d) outside the image", ih, iw);
          const int64_t gi = int64_t(c.n) * a.Ci * HW + int64_t(c.ci0 + cl) * HW +
                             int64_t(ih) * a.W + iw;
          C2B_REQUIRE(written[gi] == 0, "grad_input element %lld written twice", (long long)gi);
          written[gi] = 1;
        }
    }
  }
}

template <int V>
void check_variant(const LaunchArgs& la, const conv2d_params& prm,
                   std::vector<unsigned char>& written) {
  constexpr Variant v = kVariants[V];
  check_launch<v.wm, v.wn, v.mb, v.nbw, stage_floats(v), v.cm != 0, v.mc != 0>(la, prm, written);
}

template <int... Vs>
void check_dispatch(const LaunchArgs& la, const conv2d_params& prm,
                    std::vector<unsigned char>& written, std::integer_sequence<int, Vs...>) {
  ((la.variant == Vs ? check_variant<Vs>(la, prm, written) : void()), ...);
}

int check_all(const conv2d_params* p, int f16, int variant, char* msg, size_t len,
              int op = kOpGradInput) {
  std::vector<LaunchArgs> launches;
  const int rc = build_plan(p, f16, kDefaultCUs, &launches, nullptr, variant, nullptr, op);
  if (rc != CONV2D_OK) return rc;
  // elements of the output: grad_input, or y on a forward launch
  const int64_t n_gi = op == kOpForward
                           ? int64_t(p->batch) * p->out_channels * p->out_h * p->out_w
                           : int64_t(p->batch) * p->in_channels * p->in_h * p->in_w;
  std::vector<unsigned char> written(size_t(n_gi), 0);
  try {
    for (const LaunchArgs& la : launches) {
      C2B_REQUIRE(la.fwd == (op == kOpForward ? 1 : 0), "launch operation");
      check_dispatch(la, *p, written, std::make_integer_sequence<int, kNumVariants>());
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
  // the path conv2d_grad_input / _f16 take for this shape (aligned tensors)
  if (c2b::pw::pw_shape(p)) return c2b::pw::pw_check(p, msg, msg_len);
  return c2b::check_all(p, f16 ? 1 : 0, -1, msg, msg_len);
}

extern "C" int conv2d_check_indexing_variant(const conv2d_params* p, int variant, char* msg,
                                             size_t msg_len) {
  if (variant < 0 || variant >= c2b::kNumVariants) return CONV2D_ERR_UNSUPPORTED;
  return c2b::check_all(p, c2b::kVariants[variant].f16, variant, msg, msg_len);
}

namespace c2b {
namespace fg {   // forward_gemm.hip
bool fg_applies(const conv2d_params* p, int f16);
int fg_check(const conv2d_params* p, char* msg, size_t len);
}  // namespace fg
}  // namespace c2b

extern "C" int conv2d_check_indexing_forward(const conv2d_params* p, int f16, char* msg,
                                             size_t msg_len) {
  // the path conv2d_forward / conv2d_forward_f16 take for this shape
  if (c2b::fg::fg_applies(p, f16 ? 1 : 0)) return c2b::fg::fg_check(p, msg, msg_len);
  if (c2b::pw::pw_shape(p)) return c2b::pw::pw_check(p, msg, msg_len, 1);
  return c2b::check_all(p, f16 ? 1 : 0, -1, msg, msg_len, c2b::kOpForward);
}

extern "C" int conv2d_check_indexing_forward_variant(const conv2d_params* p, int variant,
                                                     char* msg, size_t msg_len) {
  if (variant < 0 || variant >= c2b::kNumVariants) return CONV2D_ERR_UNSUPPORTED;
  return c2b::check_all(p, c2b::kVariants[variant].f16, variant, msg, msg_len, c2b::kOpForward);
}
