// Convolution input-gradient as an implicit GEMM on CDNA4 (gfx950) matrix
// cores, and the C-ABI entry points that launch it.
//
// What is computed (meganeura 0.2.0, conv2d_grad_input_gemm_coop.wgsl, header
// comment): per batch item, C[Ci, H*W] = A[Ci, K] x B[K, H*W] with
// K = Co*kH*kW, A[ci, (co,kh,kw)] = weight[co, ci, kh, kw] (weight_T staging)
// and B the im2col of grad_out under the stride > 1 gather rule.
//
// How it is computed here (a re-design for gfx950, not the shader's scheme):
//  * Stride-residue classes (plan.hpp): every class is a dense stride-1
//    problem on a sub-image, so no structural zero is staged or multiplied.
//    Batch, class, pixel band and channel block are folded into one
//    one-dimensional grid.  Workgroups are dealt to the 8 XCDs round robin,
//    so the tile index is remapped (decode_tile) to give each XCD one
//    contiguous run of tiles: neighbours that share halo rows and weights
//    then meet in the same L2.
//  * B is never materialised: per stage a workgroup copies the grad_out
//    window its pixels read (band rows plus the kernel halo, zero outside the
//    image) into LDS once, then every tap reads that window at a fixed
//    offset, so each grad_out element crosses from L2/HBM once per stage
//    instead of once per tap.
//  * fp32 path (grad_input_f32_kernel): WM x WN waves, v_mfma_f32_16x16x4_f32.
//    Window and weights go straight from global memory into LDS with buffer
//    loads that write LDS (no register round trip); reads past a tensor's
//    extent return 0, which supplies the padding halo.  Two LDS buffers per
//    operand: the copies of stage s+1 are issued during the first tap of
//    stage s, one barrier per stage.  The planner picks the wave shape
//    (channel blocks x pixel blocks) per problem from a cost model of the
//    schedule over all CUs.
//  * f16-staged path (grad_input_kernel<true, ...>): 4 waves own a
//    64-channel x 256-pixel tile, operands are staged through registers and
//    rounded to f16 (round to nearest even) on their way into LDS, products
//    on v_mfma_f32_32x32x16_f16 with fp32 accumulators.
//  * Epilogue: masked stores straight to NCHW grad_input; every pixel of a
//    class is owned by exactly one tile, so grad_input is overwritten once,
//    with no race between workgroups.
#include <hip/hip_runtime.h>

#include <utility>

#include "tile_index.hpp"

namespace c2b {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

struct alignas(16) Half8 {
  _Float16 v[8];
};

// f32 -> f16 with round-to-nearest-even (the hardware conversion in the
// default rounding mode), 8 values into one 16-byte LDS cell.
__device__ __forceinline__ Half8 pack8(const float (&x)[8]) {
  Half8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r.v[i] = (_Float16)x[i];
  return r;
}

template <bool F16>
struct Cell;
template <>
struct Cell<false> {
  using type = float;
  static constexpr int kChannels = 1;   // output channels per LDS cell
  static constexpr int kKPerStep = 2;   // k values per matrix instruction
};
template <>
struct Cell<true> {
  using type = Half8;
  static constexpr int kChannels = 8;
  static constexpr int kKPerStep = 16;
};

// A/B operands of one k-step for both 32-pixel blocks, then the 2 x 2 block
// products.  NB = number of pixel blocks of this wave that hold a pixel.
template <bool F16, int NB>
__device__ __forceinline__ void mma_step(const typename Cell<F16>::type* sA,
                                         const typename Cell<F16>::type* sH, int ai,
                                         const int (&bi)[2], f32x16 (&acc)[2][2]) {
  if constexpr (!F16) {
    const float a0 = sA[ai], a1 = sA[ai + 32];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const float b = sH[bi[nb]];
      acc[0][nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b, acc[0][nb], 0, 0, 0);
      acc[1][nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b, acc[1][nb], 0, 0, 0);
    }
  } else {
    const f16x8 a0 = __builtin_bit_cast(f16x8, sA[ai]);
    const f16x8 a1 = __builtin_bit_cast(f16x8, sA[ai + 32]);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const f16x8 b = __builtin_bit_cast(f16x8, sH[bi[nb]]);
      acc[0][nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, b, acc[0][nb], 0, 0, 0);
      acc[1][nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, b, acc[1][nb], 0, 0, 0);
    }
  }
}

template <bool F16, int MT, int NT, int CK, int TAPS, int SLAB>
__global__ __launch_bounds__(kThreads) void grad_input_kernel(const LaunchArgs a) {
  using T = typename Cell<F16>::type;
  using G = KernelGeom<F16, MT, CK, TAPS, SLAB>;
  static_assert(MT == 64 && NT == 256, "4 waves x 2x2 blocks of 32x32");
  static_assert(G::kCPC == Cell<F16>::kChannels && G::kKPerStep == Cell<F16>::kKPerStep,
                "cell geometry");
  constexpr int CPC = G::kCPC;
  constexpr int NCG = G::kNCG;
  constexpr int KSTEPS = G::kKSteps;
  constexpr int PITCH = G::kPitch;
  constexpr int HS = G::kHS;
  constexpr int AE = G::kAE;
  constexpr int WS = G::kWS;
  static_assert(SLAB % 64 == 32 || F16, "fp32 window pitch keeps half-waves 32 banks apart");
  __shared__ T sA[G::kLdsA];
  __shared__ T sH[G::kLdsH];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, h = lane >> 5, l32 = lane & 31;
  const TileCtx c = decode_tile<MT>(a, blockIdx.x, CK);
  const PhaseDesc& P = c.P;
  const int OHOW = a.OH * a.OW;
  const int cstride = a.Ci * a.KH * a.KW;   // weight distance between channels
  const float* go_n = a.go + (size_t)c.n * a.Co * OHOW;

  int goff[HS];
#pragma unroll
  for (int k = 0; k < HS; ++k) goff[k] = window_slot_offset(c, a, tid + kThreads * k);

  // pixel blocks of this wave holding at least one pixel (wave-uniform)
  const int first = wave * 64;
  const int nact = first >= c.npx ? 0 : (first + 32 >= c.npx ? 1 : 2);
  int bbase[2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) bbase[nb] = h * SLAB + window_base(c, first + nb * 32 + l32);
  const int abase = h * PITCH + l32;

  int woff[WS];
  int wgroup = -1;
  float hreg[CK][HS];
  float wreg[WS][CPC];
  auto load_stage = [&](int st) {
    int co0, g;
    stage_split(c, CK, st, &co0, &g);
    if (g != wgroup) {
#pragma unroll
      for (int k = 0; k < WS; ++k)
        woff[k] = weight_cell_offset<MT, NCG, TAPS, CPC>(c, a, tid + kThreads * k, g);
      wgroup = g;
    }
#pragma unroll
    for (int co = 0; co < CK; ++co) {
      const bool cv = co0 + co < a.Co;
      const float* src = go_n + (size_t)(co0 + co) * OHOW;
#pragma unroll
      for (int k = 0; k < HS; ++k) hreg[co][k] = (cv && goff[k] >= 0) ? src[goff[k]] : 0.0f;
    }
    const float* wsrc = a.w + (size_t)co0 * cstride;
#pragma unroll
    for (int k = 0; k < WS; ++k) {
      const int cc = co0 + weight_cell_channel<MT, NCG, CPC>(tid + kThreads * k);
#pragma unroll
      for (int v = 0; v < CPC; ++v)
        wreg[k][v] = (woff[k] >= 0 && cc + v < a.Co) ? wsrc[woff[k] + v * cstride] : 0.0f;
    }
  };
  auto store_stage = [&]() {
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg)
#pragma unroll
      for (int k = 0; k < HS; ++k) {
        const int f = tid + kThreads * k;
        if (f < SLAB) {
          if constexpr (F16) {
            float x[8];
#pragma unroll
            for (int v = 0; v < 8; ++v) x[v] = hreg[cg * 8 + v][k];
            sH[cg * SLAB + f] = pack8(x);
          } else {
            sH[cg * SLAB + f] = hreg[cg][k];
          }
        }
      }
#pragma unroll
    for (int k = 0; k < WS; ++k) {
      const int e = tid + kThreads * k;
      if (e < AE) {
        if constexpr (F16)
          sA[weight_cell_lds<MT, NCG, PITCH>(e)] = pack8(wreg[k]);
        else
          sA[weight_cell_lds<MT, NCG, PITCH>(e)] = wreg[k][0];
      }
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // taps of stage st: k-step ks of tap tt uses cell group 2*ks + h
  auto compute_stage = [&](auto nb_tag, int st) {
    constexpr int NB = decltype(nb_tag)::value;
    int co0, g;
    stage_split(c, CK, st, &co0, &g);
    const int tap0 = g * TAPS;
    const int ntg = imin(TAPS, c.ntaps - tap0);
    int j = tap0 / P.tw;
    int l = tap0 - j * P.tw;
    for (int tt = 0; tt < ntg; ++tt) {
      const int boff = tap_window_offset(c, j, l);
      const int bi0[2] = {bbase[0] + boff, bbase[1] + boff};
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        const int ai = abase + (tt * NCG + 2 * ks) * PITCH;
        const int bi[2] = {bi0[0] + 2 * ks * SLAB, bi0[1] + 2 * ks * SLAB};
        mma_step<F16, NB>(sA, sH, ai, bi, acc);
      }
      if (++l == P.tw) {
        l = 0;
        ++j;
      }
    }
  };

  if (c.nstages > 0) load_stage(0);
  for (int st = 0; st < c.nstages; ++st) {
    __syncthreads();
    store_stage();
    __syncthreads();
    if (st + 1 < c.nstages) load_stage(st + 1);
    if (nact == 2)
      compute_stage(std::integral_constant<int, 2>(), st);
    else if (nact == 1)
      compute_stage(std::integral_constant<int, 1>(), st);
  }

  float* gi_n = a.gi + (size_t)c.n * a.Ci * (a.H * a.W);
  const size_t HW = (size_t)a.H * a.W;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int po = output_offset(c, a, first + nb * 32 + l32);
    if (po < 0) continue;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ci = c.ci0 + mb * 32 + acc_row(r, h);
        if (ci < a.Ci) gi_n[ci * HW + po] = acc[mb][nb][r];
      }
  }
}

// Word 3 of a raw (untyped, unswizzled) buffer resource: 32-bit data format.
constexpr int kRawBufferFlags = 0x00020000;
// A byte offset past every buffer's range: such loads return 0.
constexpr unsigned kOutOfRange = 0xFFFFFFFFu;

__device__ __forceinline__ __attribute__((address_space(3))) void* lds_ptr(float* p) {
  return (__attribute__((address_space(3))) void*)p;
}

// Wait until this wave's outstanding vector-memory operations (including
// loads that write LDS directly) have completed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// ---------------------------------------------------------------------------
// fp32 family: 8 waves, v_mfma_f32_16x16x4_f32 (layouts: see F32Geom).
// Stage s+1 (window and weights) is copied into the second LDS buffers while
// stage s is multiplied; one barrier per stage.  Per tap, a wave reads one
// 16-byte window cell per 16-pixel block and 4 weights, then issues
// 4 x NBW matrix instructions.
template <int WM, int WN, int NBW>
__global__ __launch_bounds__(64 * WM * WN) void grad_input_f32_kernel(const LaunchArgs a) {
  using G = F32Geom<WM, WN, NBW>;
  constexpr int MT = G::kMT, HS = G::kHS, WS = G::kWS, NT = G::kThreads;
  constexpr int TGM = kF32StageTaps, CH = kF32StageCh;
  // fixed LDS regions (floats): two window buffers, then two weight buffers
  constexpr int kWin0 = 0, kWin1 = kF32WinFloats, kWt0 = 2 * kF32WinFloats,
                kWt1 = 2 * kF32WinFloats + kF32WtFloats;
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  __shared__ f32x4 lds4[kF32LdsFloats / 4];
  float* lds = reinterpret_cast<float*>(lds4);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int mg = wave % WM, ng = wave / WM;
  const int g = lane >> 4, c16 = lane & 15;
  const TileCtx c = decode_tile<MT>(a, blockIdx.x, 0);
  const PhaseDesc& P = c.P;
  const int OHOW = a.OH * a.OW;
  const int cstride = a.Ci * a.KH * a.KW;
  const float* go_n = a.go + (size_t)c.n * a.Co * OHOW;
  const int SLOTS = P.slabr, CP = P.cp, TG = P.tg;

  // copy cells: thread tid holds cells tid + NT*k of the window and of the
  // weights; every wave-instruction writes 64 consecutive floats inside its
  // fixed buffer, cells past the stage's data read 0
  unsigned gbyte[HS];
#pragma unroll
  for (int k = 0; k < HS; ++k) {
    const int f = tid + NT * k;
    const int o = f < kF32WinFloats ? f32_window_cell(c, a, f) : -1;
    gbyte[k] = o >= 0 ? unsigned(o) * 4u : kOutOfRange;
  }
  unsigned wbyte[WS];
  int wgroup = -1;
  struct StageCopy {
    __amdgpu_buffer_rsrc_t rg, rw;
    int buf;
  };
  auto begin_stage_copy = [&](int st, int buf) {
    int co0, grp;
    stage_split(c, CH, st, &co0, &grp);
    if (grp != wgroup) {
#pragma unroll
      for (int k = 0; k < WS; ++k) {
        const int e = tid + NT * k;
        const int o = e < kF32WtFloats ? f32_weight_cell<MT>(c, a, e, grp) : -1;
        wbyte[k] = o >= 0 ? unsigned(o) * 4u : kOutOfRange;
      }
      wgroup = grp;
    }
    const int nco = imin(CH, a.Co - co0);
    StageCopy sc;
    sc.rg = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(go_n + (size_t)co0 * OHOW), 0,
                                              nco * OHOW * 4, kRawBufferFlags);
    sc.rw = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(a.w + (size_t)co0 * cstride), 0,
                                              nco * cstride * 4, kRawBufferFlags);
    sc.buf = buf;
    return sc;
  };
  // copy instructions [lo, hi) of a stage (window ones first); lo and hi are
  // compile-time constants here, so the range test folds away
  auto copy_chunk = [&](const StageCopy& sc, int lo, int hi) {
#pragma unroll
    for (int i = 0; i < HS + WS; ++i) {
      if (i < lo || i >= hi) continue;
      if (i < HS) {
        const int f0 = wave * 64 + NT * i;
        if (HS * NT == kF32WinFloats || f0 < kF32WinFloats)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              sc.rg, lds_ptr(lds + (sc.buf ? kWin1 : kWin0) + f0), 4, gbyte[i], 0, 0, 0);
      } else {
        const int k = i - HS;
        const int e0 = wave * 64 + NT * k;
        if (WS * NT == kF32WtFloats || e0 < kF32WtFloats)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              sc.rw, lds_ptr(lds + (sc.buf ? kWt1 : kWt0) + e0), 4, wbyte[k], 0, 0, 0);
      }
    }
  };
  constexpr int kCopies = HS + WS;

  const int nst = c.nstages;
  if (nst > 0) {
    const StageCopy sc0 = begin_stage_copy(0, 0);
    copy_chunk(sc0, 0, kCopies);
  }

  // byte offsets within a window buffer of each block's cell for the class's
  // first tap, and within a weight buffer of this lane's weights
  int bb[NBW];
#pragma unroll
  for (int b = 0; b < NBW; ++b)
    bb[b] = (g * SLOTS + window_base(c, f32_local(b, ng, c16, WN))) * 16;
  // byte offsets of this lane's weights of channel 4g + q, tap 0
  int aq[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) aq[q] = ((4 * g + q) * CP + (mg * 16 + c16) * TG) * 4;

  f32x4 acc[NBW];
#pragma unroll
  for (int b = 0; b < NBW; ++b) acc[b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  // multiply stage st out of buffer st&1; the copies of stage st+1 (if any)
  // go out into the other buffer during the first tap.  Tap tt reads the
  // window at a fixed slot offset and weight t = tt of channel 4g + q.
  auto tap_mma = [&](const char* Hb, const char* Ab, int boff) {
    // all addresses, then all reads, then (in the caller) the products: the
    // scheduling barriers keep the compiler from recycling a read's target
    // register as the next address, which would serialise the reads
    const f32x4* ba[NBW];
#pragma unroll
    for (int b = 0; b < NBW; ++b) ba[b] = reinterpret_cast<const f32x4*>(Hb + bb[b] + boff);
    const float* aa[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) aa[q] = reinterpret_cast<const float*>(Ab + aq[q]);
    __builtin_amdgcn_sched_barrier(0);
    float aw[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) aw[q] = *aa[q];
    f32x4 bv[NBW];
#pragma unroll
    for (int b = 0; b < NBW; ++b) bv[b] = *ba[b];
    __builtin_amdgcn_sched_barrier(0);
    return [&, bv, aw]() mutable {
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int b = 0; b < NBW; ++b)
          acc[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(aw[q], bv[b][q], acc[b], 0, 0, 0);
    };
  };
  auto compute = [&](int st) {
    const int buf = st & 1;
    int co0, grp;
    stage_split(c, CH, st, &co0, &grp);
    const int tap0 = grp * TG;
    const int ntg = imin(TG, c.ntaps - tap0);
    const char* Hb = reinterpret_cast<const char*>(lds + (buf ? kWin1 : kWin0));
    const char* Ab = reinterpret_cast<const char*>(lds + (buf ? kWt1 : kWt0));
    int j = tap0 / P.tw, l = tap0 - (tap0 / P.tw) * P.tw;
    // first tap, with the copies of the next stage
    {
      auto mma = tap_mma(Hb, Ab, tap_window_offset(c, j, l) * 16);
      if (st + 1 < nst) {
        const StageCopy sc = begin_stage_copy(st + 1, buf ^ 1);
        copy_chunk(sc, 0, kCopies);
      }
      mma();
      if (++l == P.tw) {
        l = 0;
        ++j;
      }
    }
    for (int tt = 1; tt < ntg; ++tt) {
      Ab += 4;   // weight t = tt
      auto mma = tap_mma(Hb, Ab, tap_window_offset(c, j, l) * 16);
      mma();
      if (++l == P.tw) {
        l = 0;
        ++j;
      }
    }
  };

  wait_vmem();
  __syncthreads();
  for (int st = 0; st < nst; ++st) {
    compute(st);
    wait_vmem();          // this wave's copies of stage st+1 have landed
    __syncthreads();      // ... everyone's, and buffer st&1 may be refilled
  }

  // epilogue: register r of block b holds channel mg*16 + 4g + r, pixel
  // (b*WN + ng)*16 + c16
  float* gi_n = a.gi + (size_t)c.n * a.Ci * (a.H * a.W);
  const size_t HW = (size_t)a.H * a.W;
#pragma unroll
  for (int b = 0; b < NBW; ++b) {
    const int po = output_offset(c, a, f32_local(b, ng, c16, WN));
    if (po < 0) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int cc = c.ci0 + mg * 16 + 4 * g + r;
      if (cc < a.Ci) gi_n[cc * HW + po] = acc[b][r];
    }
  }
}

template <int V>
void launch_f32_variant(const LaunchArgs& la, hipStream_t st) {
  constexpr F32Variant v = kF32Variants[V];
  hipLaunchKernelGGL((grad_input_f32_kernel<v.wm, v.wn, v.nbw>), dim3(la.total_tiles),
                     dim3(64 * v.wm * v.wn), 0, st, la);
}

template <int... Vs>
void launch_f32_dispatch(const LaunchArgs& la, hipStream_t st,
                         std::integer_sequence<int, Vs...>) {
  ((la.variant == Vs ? launch_f32_variant<Vs>(la, st) : void()), ...);
}

int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return kF32DefaultCUs;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < 1)
    return kF32DefaultCUs;
  return cus;
}

int launch_f32(const float* go, const float* w, float* gi, const conv2d_params* p,
               void* stream) {
  int rc = validate_shape(p);
  if (rc != CONV2D_OK) return rc;
  rc = check_pointers(go, w, gi, p);
  if (rc != CONV2D_OK) return rc;
  std::vector<LaunchArgs> launches;
  rc = build_plan_f32(p, device_cus(), &launches, nullptr);
  if (rc != CONV2D_OK) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  for (LaunchArgs& la : launches) {
    la.go = go;
    la.w = w;
    la.gi = gi;
    if (la.total_tiles == 0) continue;
    launch_f32_dispatch(la, st, std::make_integer_sequence<int, kNumF32Variants>());
  }
  if (hipGetLastError() != hipSuccess) return CONV2D_ERR_HIP;
  return CONV2D_OK;
}

template <bool F16>
constexpr TileShape tile_of() {
  return F16 ? kF16Tile : kF32Tile;
}

template <bool F16>
int launch(const float* go, const float* w, float* gi, const conv2d_params* p, void* stream) {
  constexpr TileShape ts = tile_of<F16>();
  int rc = validate_shape(p);
  if (rc != CONV2D_OK) return rc;
  rc = check_pointers(go, w, gi, p);
  if (rc != CONV2D_OK) return rc;
  std::vector<LaunchArgs> launches;
  rc = build_plan(p, ts, &launches, nullptr);
  if (rc != CONV2D_OK) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  for (LaunchArgs& la : launches) {
    la.go = go;
    la.w = w;
    la.gi = gi;
    if (la.total_tiles == 0) continue;
    hipLaunchKernelGGL((grad_input_kernel<F16, ts.mt, ts.nt, ts.ck, ts.taps, ts.slab>),
                       dim3(la.total_tiles), dim3(kThreads), 0, st, la);
  }
  if (hipGetLastError() != hipSuccess) return CONV2D_ERR_HIP;
  return CONV2D_OK;
}

}  // namespace c2b

extern "C" int conv2d_grad_input(const float* grad_out, const float* weight, float* grad_input,
                                 const conv2d_params* p, void* stream) {
  return c2b::launch_f32(grad_out, weight, grad_input, p, stream);
}

extern "C" int conv2d_grad_input_f16(const float* grad_out, const float* weight,
                                     float* grad_input, const conv2d_params* p, void* stream) {
  return c2b::launch<true>(grad_out, weight, grad_input, p, stream);
}
