// Gradient of multi-head attention with respect to V on CDNA4 (gfx950)
// matrix cores, its host replay, and its C-ABI entry point.
//
// What is computed (meganeura 0.2.0, src/shaders/mha_grad_v.wgsl: Params,
// the bounds of the position loop, the score recomputation, P * dO): for key
// t of kv head g, dv[t, g] = sum over pos in [causal ? t : 0, window ?
// min(q_seq, t + window) : q_seq) and the heads h of g's group of
// P(pos, h, t) * dout[pos, h], with P = exp(min(s - max, 0) - log_sum) from
// the forward's row statistics and s = q[pos, h] . k[t, g] / sqrt(64).
//
// The page runs one 64-lane workgroup per (key, kv head), reducing each
// score across the workgroup.  Here a workgroup (four waves) takes 64 keys of
// one kv head and, for each head of the group and each 64-position query
// block that reaches those keys:
//  * stages Q [pos][d], dO transposed [d][pos] and the row statistics in LDS
//    (the K block stays there for the whole workgroup), rows 68 floats
//    apart so that 16-byte reads of 16 rows hit distinct banks;
//  * computes S = Q K^T for the wave's 16 keys: 4 x 4 v_mfma_f32_16x16x4_f32
//    k steps per 16-position block, both operands read 16 bytes along d;
//  * turns the accumulators into P in registers (mask, scale, clamped
//    exponent);
//  * accumulates dV^T[d, t] += dO^T[d, pos] P[pos, t]: register r of the S
//    block of positions 16b + 4 g' + r is exactly the B operand MFMA r needs
//    (lane group g' supplies position 4 g' + r), so P never leaves registers.
// The last stores write dV rows as 16-byte pieces.  When the causal pairing
// below leaves fewer workgroups than two per CU, each unit is split over two
// workgroups by the heads of the group; each adds its partial dV onto a
// zeroed dv, and since exactly two terms meet on zero (0 + a + b equals
// 0 + b + a in fp32), the result does not depend on their order.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "mha_grad_v.h"

#if defined(__HIPCC__)
#define MHA_HD __host__ __device__ __forceinline__
#else
#define MHA_HD inline
#endif

namespace mhv {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kD = 64;               // head dimension
constexpr int kBK = 64;              // keys per workgroup
constexpr int kBQ = 64;              // positions per query block
constexpr int kPitch = 68;           // LDS floats between rows
constexpr int kThreads = 256;
constexpr uint32_t kPad = 0x80000000u;   // byte offset past every buffer range
constexpr int64_t kI31 = int64_t(1) << 31;

MHA_HD int imin(int a, int b) { return a < b ? a : b; }
MHA_HD int imax(int a, int b) { return a > b ? a : b; }

struct Args {
  const float* dout;
  const float* q;
  const float* k;
  const float* lse;
  float* dv;
  int32_t q_seq, kv_seq, H, HKV, group, window, causal;
  int32_t nkb;     // key blocks
  int32_t paired;  // 1: a workgroup takes key blocks u and nkb - 1 - u
  int32_t units;   // units (1 or 2 key blocks) per kv head
  int32_t hsplit;  // workgroups per unit, each taking group / hsplit heads
  float scale;
};

// Workgroup bid -> kv head and its key blocks (1 or 2), returned count.
// Under a causal mask without a short window, key block u reaches nkb - u
// query blocks, so blocks u and nkb - 1 - u share a workgroup and every
// workgroup gets about the same work.
// Workgroups [part * units * HKV, (part + 1) * units * HKV) take heads
// [part * group / hsplit, (part + 1) * group / hsplit) of their group.
MHA_HD int unit_of(const Args& a, int bid, int kb[2], int* kvh, int* part) {
  const int per = a.units * a.HKV;
  *part = bid / per;
  bid -= *part * per;
  *kvh = bid % a.HKV;
  const int u = bid / a.HKV;
  kb[0] = u;
  if (!a.paired) return 1;
  kb[1] = a.nkb - 1 - u;
  return kb[1] != u ? 2 : 1;
}

// Query positions [lo, hi) that reach some key of key block kb: the union of
// the keys' ranges [causal ? t : 0, window ? min(q_seq, t + window) : q_seq).
MHA_HD void pos_range(const Args& a, int kb, int* lo, int* hi) {
  const int t0 = kb * kBK, t1 = imin(t0 + kBK, a.kv_seq) - 1;
  *lo = a.causal ? t0 : 0;
  *hi = a.window > 0 ? imin(a.q_seq, t1 + a.window) : a.q_seq;
}

// Query pos sees key t (the page's position loop read from the key side).
MHA_HD bool visible(const Args& a, int pos, int t) {
  return pos < a.q_seq && t < a.kv_seq && (!a.causal || pos >= t) &&
         (a.window <= 0 || pos < t + a.window);
}

// Copy roles of thread tid.  Row tiles (K, Q): rows tid / 16 + 16 p, d quad
// tid % 16 (one 16-byte load each).  dO^T: d = tid % 64, position quads
// tid / 64 + 4 p (four 4-byte loads, one 16-byte LDS write).
MHA_HD int row_of(int tid, int p) { return tid / 16 + 16 * p; }
MHA_HD int dq_of(int tid) { return tid % 16; }
MHA_HD int gd_of(int tid) { return tid % 64; }
MHA_HD int gpq_of(int tid, int p) { return tid / 64 + 4 * p; }

// Byte offsets (kPad past the sequence): the 16-byte d quad of row `row`
// of Q (head h) or K (kv head kvh), one dout element, one lse pair.
MHA_HD uint32_t q_offset(const Args& a, int pos, int h, int dq) {
  return pos < a.q_seq ? (uint32_t(pos * a.H + h) * kD + 4 * dq) * 4u : kPad;
}
MHA_HD uint32_t k_offset(const Args& a, int t, int kvh, int dq) {
  return t < a.kv_seq ? (uint32_t(t * a.HKV + kvh) * kD + 4 * dq) * 4u : kPad;
}
MHA_HD uint32_t g_offset(const Args& a, int pos, int h, int d) {
  return pos < a.q_seq ? (uint32_t(pos * a.H + h) * kD + d) * 4u : kPad;
}
MHA_HD uint32_t l_offset(const Args& a, int pos, int h, int e) {
  return pos < a.q_seq ? (uint32_t(pos * a.H + h) * 2 + e) * 4u : kPad;
}

__device__ __forceinline__ float load_f32(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
}
__device__ __forceinline__ f32x4 load_f32x4(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
}

__global__ __launch_bounds__(kThreads, 2) void mha_grad_v_kernel(const Args a) {
  __shared__ f32x4 kt4[kBK * kPitch / 4];   // K block [t][d]
  __shared__ f32x4 qs4[kBQ * kPitch / 4];   // Q block [pos][d]
  __shared__ f32x4 gt4[kD * kPitch / 4];    // dO^T block [d][pos]
  __shared__ float ls[kBQ * 2];             // (max, log_sum) per position
  float* Kt = reinterpret_cast<float*>(kt4);
  float* Qs = reinterpret_cast<float*>(qs4);
  float* Gt = reinterpret_cast<float*>(gt4);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c16 = lane & 15;
  int kbs[2], kvh, part;
  const int nblocks = unit_of(a, blockIdx.x, kbs, &kvh, &part);
  const int hper = a.group / a.hsplit;

  const __amdgpu_buffer_rsrc_t rsQ = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(a.q), 0, a.q_seq * a.H * kD * 4, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsK = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(a.k), 0, a.kv_seq * a.HKV * kD * 4, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsG = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(a.dout), 0, a.q_seq * a.H * kD * 4, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsL = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(a.lse), 0, a.q_seq * a.H * 2 * 4, 0x00020000);

  for (int ib = 0; ib < nblocks; ++ib) {
  const int kb = kbs[ib];
  const int t0 = kb * kBK;
  int lo, hi;
  pos_range(a, kb, &lo, &hi);
  __syncthreads();   // the previous key block's reads of Kt are done
  // the K block, once per key block
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const f32x4 v = load_f32x4(rsK, k_offset(a, t0 + row_of(tid, p), kvh, dq_of(tid)));
    *reinterpret_cast<f32x4*>(Kt + row_of(tid, p) * kPitch + 4 * dq_of(tid)) = v;
  }

  f32x4 acc[4];   // dV^T[d = 16 b + 4 g + r][t = wave's key c16], b = 0..3
#pragma unroll
  for (int b = 0; b < 4; ++b) acc[b] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  const int tk = 16 * wave + c16;   // this lane's key within the block

  // Query blocks run from the last down: under a causal mask every key
  // block's range ends at the sequence's end, so the workgroups resident
  // together start on the same blocks and share them in L2.
  const int qb0 = lo / kBQ * kBQ, qlast = (hi - 1) / kBQ * kBQ;
  for (int r = part * hper; r < (part + 1) * hper; ++r) {
    const int h = kvh * a.group + r;
    for (int pos0 = qlast; pos0 >= qb0 && hi > lo; pos0 -= kBQ) {
      __syncthreads();   // the previous block's reads are done
      f32x4 qv[4];
      float gv[4][4], lv = 0.0f;
#pragma unroll
      for (int p = 0; p < 4; ++p)
        qv[p] = load_f32x4(rsQ, q_offset(a, pos0 + row_of(tid, p), h, dq_of(tid)));
#pragma unroll
      for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          gv[p][e] = load_f32(rsG, g_offset(a, pos0 + 4 * gpq_of(tid, p) + e, h, gd_of(tid)));
      if (tid < 2 * kBQ) lv = load_f32(rsL, l_offset(a, pos0 + tid / 2, h, tid % 2));
#pragma unroll
      for (int p = 0; p < 4; ++p)
        *reinterpret_cast<f32x4*>(Qs + row_of(tid, p) * kPitch + 4 * dq_of(tid)) = qv[p];
#pragma unroll
      for (int p = 0; p < 4; ++p)
        *reinterpret_cast<f32x4*>(Gt + gd_of(tid) * kPitch + 4 * gpq_of(tid, p)) =
            f32x4{gv[p][0], gv[p][1], gv[p][2], gv[p][3]};
      if (tid < 2 * kBQ) ls[tid] = lv;
      __syncthreads();

      // S[pos][t] for the wave's 16 keys, 4 blocks of 16 positions
      f32x4 s[4];
#pragma unroll
      for (int pb = 0; pb < 4; ++pb) s[pb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int u = 0; u < kD / 16; ++u) {
        const f32x4 kv = *reinterpret_cast<const f32x4*>(Kt + tk * kPitch + 16 * u + 4 * g);
#pragma unroll
        for (int pb = 0; pb < 4; ++pb) {
          const f32x4 qa = *reinterpret_cast<const f32x4*>(
              Qs + (16 * pb + c16) * kPitch + 16 * u + 4 * g);
#pragma unroll
          for (int q = 0; q < 4; ++q)
            s[pb] = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[q], kv[q], s[pb], 0, 0, 0);
        }
      }
      // P in place: register j of block pb is position pos0 + 16 pb + 4 g + j
#pragma unroll
      for (int pb = 0; pb < 4; ++pb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int lp = 16 * pb + 4 * g + j;
          const float e = fminf(s[pb][j] * a.scale - ls[2 * lp], 0.0f) - ls[2 * lp + 1];
          s[pb][j] = visible(a, pos0 + lp, t0 + tk) ? __expf(e) : 0.0f;
        }
      // dV^T[d][t] += dO^T[d][pos] P[pos][t]
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int pb = 0; pb < 4; ++pb) {
          const f32x4 ga = *reinterpret_cast<const f32x4*>(
              Gt + (16 * b + c16) * kPitch + 16 * pb + 4 * g);
#pragma unroll
          for (int q = 0; q < 4; ++q)
            acc[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(ga[q], s[pb][q], acc[b], 0, 0, 0);
        }
    }
  }

  const int t = t0 + tk;
  if (t < a.kv_seq) {
    float* out = a.dv + (size_t(t) * a.HKV + kvh) * kD;
    if (a.hsplit == 1) {
#pragma unroll
      for (int b = 0; b < 4; ++b) *reinterpret_cast<f32x4*>(out + 16 * b + 4 * g) = acc[b];
    } else {
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int j = 0; j < 4; ++j) unsafeAtomicAdd(out + 16 * b + 4 * g + j, acc[b][j]);
    }
  }
  }
}

// dv = 0 ahead of a split launch's two partial sums.
__global__ __launch_bounds__(256) void mha_zero_kernel(f32x4* dv, uint32_t n4) {
  for (uint32_t i = blockIdx.x * 256u + threadIdx.x; i < n4; i += gridDim.x * 256u)
    dv[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
}

// ---------------------------------------------------------------------------
// Host side.

int plan(const mha_grad_v_params* p, Args* a) {
  if (p == nullptr) return CONV2D_ERR_NULL_PTR;
  if (p->head_dim != kD || (p->heads > 0 && p->kv_heads == 0) ||
      (p->kv_heads > 0 && p->heads % p->kv_heads) || p->causal > 1 ||
      (p->causal && p->q_seq != p->kv_seq))
    return CONV2D_ERR_BAD_SHAPE;
  const int64_t QB = int64_t(p->q_seq) * p->heads * kD * 4, KB = int64_t(p->kv_seq) * p->kv_heads * kD * 4;
  if (QB >= kI31 || KB >= kI31 || int64_t(p->q_seq) + kBQ + p->window >= kI31 ||
      int64_t(p->kv_seq) + kBK >= kI31 || p->window >= kI31)
    return CONV2D_ERR_OVERFLOW;
  std::memset(a, 0, sizeof(*a));
  a->q_seq = int32_t(p->q_seq);
  a->kv_seq = int32_t(p->kv_seq);
  a->H = int32_t(p->heads);
  a->HKV = int32_t(p->kv_heads);
  a->group = p->kv_heads ? int32_t(p->heads / p->kv_heads) : 0;
  a->window = int32_t(p->window);
  a->causal = int32_t(p->causal);
  a->nkb = int32_t((int64_t(p->kv_seq) + kBK - 1) / kBK);
  a->paired = p->causal && (p->window == 0 || p->window >= p->q_seq / 2) ? 1 : 0;
  a->units = a->paired ? (a->nkb + 1) / 2 : a->nkb;
  // fewer units than two per CU of the largest MI355X part: split each over
  // two workgroups by heads (an even group of at least two)
  a->hsplit =
      a->paired && a->group >= 2 && a->group % 2 == 0 && int64_t(a->units) * a->HKV < 2 * 256 ? 2 : 1;
  a->scale = 1.0f / std::sqrt(float(kD));
  if (int64_t(a->nkb) * a->HKV >= kI31) return CONV2D_ERR_OVERFLOW;
  return CONV2D_OK;
}

namespace {
struct Failure {
  std::string msg;
};
#define MHA_REQUIRE(cond, ...)                                  \
  do {                                                          \
    if (!(cond)) {                                              \
      char buf_[512];                                           \
      std::snprintf(buf_, sizeof buf_, __VA_ARGS__);            \
      throw Failure{std::string(#cond) + ": " + buf_};          \
    }                                                           \
  } while (0)
}  // namespace

// Host replay of the launch, through the kernel's own index functions.
int check(const mha_grad_v_params* p, char* msg, size_t len) {
  Args a;
  const int rc = plan(p, &a);
  if (rc != CONV2D_OK) return rc;
  try {
    const int64_t q_bytes = int64_t(a.q_seq) * a.H * kD * 4;
    const int64_t k_bytes = int64_t(a.kv_seq) * a.HKV * kD * 4;
    const int64_t l_bytes = int64_t(a.q_seq) * a.H * 2 * 4;
    MHA_REQUIRE(a.hsplit >= 1 && a.group % a.hsplit == 0, "head split %d of %d", a.hsplit,
                a.group);
    MHA_REQUIRE(a.hsplit == 1 || a.paired, "only paired units are split");
    // (key block, kv head, head of the group) -> times covered
    std::vector<unsigned char> seen(size_t(int64_t(a.nkb) * a.HKV * (a.group ? a.group : 1)), 0);
    for (int ub = 0; ub < 2 * a.units * a.HKV * a.hsplit; ++ub) {
      const int bid = ub / 2;
      int kbs[2], kvh, part;
      const int nb = unit_of(a, bid, kbs, &kvh, &part);
      if (ub % 2 >= nb) continue;
      const int kb = kbs[ub % 2];
      MHA_REQUIRE(kb >= 0 && kb < a.nkb && kvh >= 0 && kvh < a.HKV && part >= 0 &&
                      part < a.hsplit,
                  "workgroup %d unit", bid);
      const int hper = a.group / a.hsplit;
      for (int r = part * hper; r < (part + 1) * hper; ++r) {
        const size_t e = (size_t(kb) * a.HKV + kvh) * a.group + r;
        MHA_REQUIRE(!seen[e], "key block %d, kv head %d, head %d taken twice", kb, kvh, r);
        seen[e] = 1;
      }
      if (a.group == 0) seen[size_t(kb) * a.HKV + kvh] = 1;
      int lo, hi;
      pos_range(a, kb, &lo, &hi);
      const int qb0 = lo / kBQ * kBQ;
      // every position of every key's range lies in a visited query block,
      // and `visible` is exactly the range
      for (int tk = 0; tk < kBK; ++tk) {
        const int t = kb * kBK + tk;
        if (t >= a.kv_seq) break;
        const int start = a.causal ? t : 0;
        const int end = a.window > 0 ? imin(a.q_seq, t + a.window) : a.q_seq;
        for (int pos = 0; pos < a.q_seq + kBQ; ++pos) {
          const bool in = pos >= start && pos < end;
          MHA_REQUIRE(visible(a, pos, t) == in, "visible(%d, %d)", pos, t);
          if (in) MHA_REQUIRE(pos >= qb0 && pos < hi, "position %d of key %d not visited", pos, t);
        }
      }
      // staged elements of one query block at each visited block start
      // (position roles, 0 past the sequence), and the K block; with no
      // heads the head loop stages nothing
      for (int pos0 = qb0; pos0 < hi && a.group > 0; pos0 += kBQ) {
        for (int tid = 0; tid < kThreads; ++tid)
          for (int pq = 0; pq < 4; ++pq) {
            const int pos = pos0 + row_of(tid, pq), dq = dq_of(tid);
            MHA_REQUIRE(row_of(tid, pq) < kBQ && dq < kD / 4, "Q roles");
            const uint32_t o = q_offset(a, pos, 0, dq);
            MHA_REQUIRE(pos < a.q_seq ? int64_t(o) + 16 <= q_bytes &&
                                            o == uint32_t((int64_t(pos) * a.H * kD + 4 * dq) * 4)
                                      : int64_t(o) >= q_bytes,
                        "Q element (%d, %d)", pos, dq);
            for (int e = 0; e < 4; ++e) {
              const int gp = pos0 + 4 * gpq_of(tid, pq) + e, d = gd_of(tid);
              MHA_REQUIRE(4 * gpq_of(tid, pq) + e < kBQ && d < kD, "dO roles");
              const uint32_t og = g_offset(a, gp, a.H - 1, d);
              MHA_REQUIRE(gp < a.q_seq ? int64_t(og) < q_bytes : int64_t(og) >= q_bytes,
                          "dO element (%d, %d)", gp, d);
            }
          }
        for (int tid = 0; tid < 2 * kBQ; ++tid) {
          const int pos = pos0 + tid / 2;
          const uint32_t ol = l_offset(a, pos, a.H - 1, tid % 2);
          MHA_REQUIRE(pos < a.q_seq ? int64_t(ol) < l_bytes : int64_t(ol) >= l_bytes, "lse");
        }
      }
      for (int tid = 0; tid < kThreads; ++tid)
        for (int pq = 0; pq < 4; ++pq) {
          const int t = kb * kBK + row_of(tid, pq);
          const uint32_t o = k_offset(a, t, kvh, dq_of(tid));
          MHA_REQUIRE(t < a.kv_seq ? int64_t(o) + 16 <= k_bytes : int64_t(o) >= k_bytes,
                      "K element %d", t);
        }
    }
    for (size_t i = 0; i < seen.size(); ++i)
      MHA_REQUIRE(seen[i] == 1, "(key block, kv head, head) %zu never taken", i);
    // every LDS row cell of a stage is written once: rows x quads
    std::vector<int> cnt(size_t(kBQ) * 16, 0), gcnt(size_t(kD) * 16, 0);
    for (int tid = 0; tid < kThreads; ++tid)
      for (int pq = 0; pq < 4; ++pq) {
        cnt[size_t(row_of(tid, pq)) * 16 + dq_of(tid)] += 1;
        gcnt[size_t(gd_of(tid)) * 16 + gpq_of(tid, pq)] += 1;
      }
    for (size_t i = 0; i < cnt.size(); ++i)
      MHA_REQUIRE(cnt[i] == 1 && gcnt[i] == 1, "LDS cell %zu written %d / %d times", i, cnt[i],
                  gcnt[i]);
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

}  // namespace mhv

extern "C" int mha_grad_v(const float* dout, const float* q, const float* k, const float* lse,
                          float* dv, const mha_grad_v_params* p, void* stream) {
  mhv::Args a;
  const int rc = mhv::plan(p, &a);
  if (rc != CONV2D_OK) return rc;
  const uint64_t nq = uint64_t(a.q_seq) * a.H * mhv::kD, nk = uint64_t(a.kv_seq) * a.HKV * mhv::kD;
  const uint64_t nl = uint64_t(a.q_seq) * a.H * 2;
  if ((nq && (dout == nullptr || q == nullptr || lse == nullptr)) ||
      (nk && (k == nullptr || dv == nullptr)))
    return CONV2D_ERR_NULL_PTR;
  auto overlap = [](const void* a0, uint64_t na, const void* b0, uint64_t nb) {
    if (na == 0 || nb == 0) return false;
    const uintptr_t u = reinterpret_cast<uintptr_t>(a0), v = reinterpret_cast<uintptr_t>(b0);
    return u < v + nb && v < u + na;
  };
  if (overlap(dv, nk * 4, dout, nq * 4) || overlap(dv, nk * 4, q, nq * 4) ||
      overlap(dv, nk * 4, k, nk * 4) || overlap(dv, nk * 4, lse, nl * 4))
    return CONV2D_ERR_ALIAS;
  if (nk == 0) return CONV2D_OK;
  if (reinterpret_cast<uintptr_t>(q) % 16 || reinterpret_cast<uintptr_t>(k) % 16 ||
      reinterpret_cast<uintptr_t>(dv) % 16)
    return CONV2D_ERR_BAD_SHAPE;
  a.dout = dout;
  a.q = q;
  a.k = k;
  a.lse = lse;
  a.dv = dv;
  // (heads == 0: the kernel's head loop is empty and it stores zeros)
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (a.hsplit > 1) {
    const uint32_t n4 = uint32_t(nk / 4);   // nk = kv_seq * kv_heads * 64
    hipLaunchKernelGGL(mhv::mha_zero_kernel, dim3((n4 + 255) / 256 < 1024 ? (n4 + 255) / 256 : 1024),
                       dim3(256), 0, st, reinterpret_cast<mhv::f32x4*>(dv), n4);
  }
  hipLaunchKernelGGL(mhv::mha_grad_v_kernel, dim3(a.units * a.HKV * a.hsplit),
                     dim3(mhv::kThreads), 0, st, a);
  return hipGetLastError() == hipSuccess ? CONV2D_OK : CONV2D_ERR_HIP;
}

extern "C" int mha_grad_v_check_indexing(const mha_grad_v_params* p, char* msg, size_t msg_len) {
  return mhv::check(p, msg, msg_len);
}
