// Wavefront-round attention over 8-bit-key pages (the 8-bit QK^T tier), one
// layer, every active query group in one launch.
//
// "Wave Forcing: Towards Speed-of-Light Streaming Video Generation" §3.1
// Eq. 4-5 define the context (anchor, history, store, cleaner denoising
// chunks).  App. B.1 and App. C.2 Tab. 4 name an approximate compute mode
// that replaces self-attention by SageAttention: Q K^T in 8 bits, P V in
// higher precision.  Pages hold E4M3 codes of K/2^eK (one power-of-two scale
// per 64-token tile of a head) and the values in bf16; pages are padded to
// 64 T tokens, so a key tile never straddles two pages and only the last
// tile of each page is partial.
//
// CDNA4, two matrix-core instructions per tile:
//   * S^T = K Q^T on v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3 x E4M3): the
//     matrix core applies the tile's K exponent and each query row's
//     exponent (the bf16 q_rot row times scale * log2(e), quantised here), so
//     S comes out in base-2 exponent units.  A lane holds 32 bytes of an
//     operand: dims 64 s + 32 half + j of its row, the same for K and Q.
//   * O^T = Vt P^T on v_mfma_f32_32x32x16_bf16: A = 32 value dims x 16 keys
//     of the bf16 Vt tile, B = the softmax weights rounded to bf16.
//   * K rows enter the QK A operand permuted: accumulator row r = 8 a + 4 h
//     + b of QK MFMA t2 is key 32 t2 + 16 (a >> 1) + 8 h + 4 (a & 1) + b.
//     The 16 values a lane of lane half h holds per t2 are then keys
//     16 kk + 8 h + j (kk = 2 t2 + (a >> 1), j = 0..7): the B operand layout
//     of the four PV k-steps, so P^T goes from the QK accumulator to the PV
//     MFMA without any lane exchange.
// Schedule as the bf16 instance: 8 waves x 32 queries in two ping-pong
// groups of 4 (waves i and i+4 share a SIMD), one group in its MFMA cluster
// (PV of tile t-1, QK of tile t, at raised issue priority) while the other
// runs its softmax; a 4-stage LDS ring of K and Vt tiles (rows padded by one
// 16-byte chunk), tile t+3 fetched into registers while tile t is
// multiplied.  Online softmax in base 2; the QK accumulators start from
// minus the running max; lazy rescale (2^8) detected from the rounded
// weights' exponent bits; the row sum of the rounded weights is taken in the
// MFMA cluster.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "wf_kernels.h"
#include "wf_items.h"
#include "wf_partial.h"

namespace wf {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kD = 128;
constexpr int kBN = 64;                   // keys per tile
constexpr int kNT = 512;                  // threads: 8 waves in two groups of 4
constexpr int kStages = 4;
constexpr int kVPitch = kBN + 8;          // Vt row pitch in LDS (bf16 elements)
constexpr int kKPitch = kD + 16;          // K row pitch in LDS (bytes)
constexpr int kKTile = kBN * kKPitch;     // bytes of a padded K tile
constexpr int kVTile = kD * kVPitch * 2;  // bytes of a padded Vt tile
constexpr int kStage = kKTile + kVTile;
constexpr int kVLoads = kD * (kBN / 8) / kNT;   // 16-byte Vt chunks per thread
constexpr int kE8M0One = 127;             // scale code of 2^0
static_assert(kVLoads * kNT == kD * (kBN / 8) && kBN * kD == 16 * kNT, "shape");

__device__ inline int find_group(const AttnArgs& a, int item) {
  int g = 0;
  while (g + 1 < a.n_groups && item >= a.grp[g + 1].item0) ++g;
  return g;
}

// Byte offset of 16-byte chunk c of K row r inside a stage.  Rows are padded
// by one chunk: a QK operand read by 16 lanes covers 16 consecutive keys at
// one chunk index, 9 r + c mod 16 differs for all of them.
__device__ inline int k_off(int r, int c) { return r * kKPitch + (c << 4); }

// Key of A-operand row r of QK MFMA t2 (see the header).
__device__ inline int qk_key(int t2, int r) {
  return 32 * t2 + 16 * (r >> 4) + 8 * ((r >> 2) & 1) + 4 * ((r >> 3) & 1) + (r & 3);
}

__device__ inline float pair_max32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float pair_sum32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Smallest e with amax <= 448 * 2^e (0 for amax == 0), clamped to E8M0.
__device__ inline int fp8_exponent(float amax) {
  if (!(amax > 0.f)) return 0;
  int x;
  const float m = frexpf(amax, &x);
  const int e = m <= 0.875f ? x - 9 : x - 8;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

__device__ inline uint32_t pack4(float a, float b, float c, float d) {
  uint32_t r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
}

__global__ __launch_bounds__(kNT, 1) void wf_attention_fp8k_kernel(const AttnArgs a) {
  constexpr int BM = kAttnBM_fp8k;
  constexpr int NPV = 16;                 // PV MFMAs per tile (4 k-steps x 4 dim tiles)
  constexpr int NQK = 4;                  // QK MFMAs per tile (2 k-steps x 2 key halves)
  __shared__ __attribute__((aligned(16))) uint8_t lds[kStages * kStage];
  __shared__ uint8_t tcode[kFp8MaxCtxTiles];   // eK + 127 of every context tile

  if (static_cast<int>(blockIdx.x) >= a.n_items) return;
  const int item = xcd_item(blockIdx.x, a.n_items, a.q_tiles);   // whole units per XCD
  const int g = find_group(a, item);
  const AttnGroup& G = a.grp[g];
  const int li = item - G.item0;
  const int h = li / a.q_tiles;
  const int qt = li - h * a.q_tiles;
  const int N = a.N, H = a.H, Np = a.Npad, T = a.T;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int col = lane & 31, half = lane >> 5;
  const int pgroup = wave >> 2;           // ping-pong group
  const int n_pages = G.n_pages;
  const int n_tiles = n_pages * T;
  const int last_valid = N - kBN * (T - 1);   // keys in the last tile of a page

  // Byte offsets inside this layer's pool fit in 32 bits (checked on the
  // host): every load is "uniform base + 32-bit lane offset".
  const char* pool = static_cast<const char*>(a.pool);
  const uint32_t page_bytes = static_cast<uint32_t>(a.page_bytes);
  const uint32_t k_part = static_cast<uint32_t>(H) * Np * kD;     // K8 bytes
  const uint32_t k_head = static_cast<uint32_t>(h) * Np * kD;
  const uint32_t v_head = k_part + static_cast<uint32_t>(h) * kD * Np * 2u;
  const uint32_t code_head = 3u * k_part + static_cast<uint32_t>(h) * T * 2u;

  // ---- K scale codes of every tile of the context ----
  for (int i = tid; i < n_tiles; i += kNT) {
    const int p = i / T, tp = i - p * T;
    const uint32_t off = static_cast<uint32_t>(G.slot[p]) * page_bytes + code_head + 2u * tp;
    tcode[i] = *reinterpret_cast<const uint8_t*>(pool + off);
  }

  // ---- query row: B operand of S^T = K Q^T, quantised per row ----
  // Lane (col, half) holds dims 64 s + 32 half + j (j = 0..31) for k-steps
  // s = 0, 1; the row's other 64 dims sit in lane col + 32 (1 - half).  The
  // row is multiplied by c = scale * log2(e) (fp32) before quantisation.
  // Rows past N are clamped (never stored).
  const int q = qt * BM + wave * 32 + col;
  const int qc = q < N ? q : N - 1;
  const __bf16* qrow = static_cast<const __bf16*>(a.q_rot) +
                       ((static_cast<int64_t>(G.stage) * N + qc) * H + h) * kD;
  const float c = a.scale_log2e;
  i32x8 qf[2];
  int qscale;
  {
    float qv[2][32];
    float qmax = 0.f;
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        const bf16x8 x = *reinterpret_cast<const bf16x8*>(qrow + 64 * s + 32 * half + 8 * cc);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          qv[s][8 * cc + e] = static_cast<float>(x[e]) * c;
          qmax = fmaxf(qmax, fabsf(qv[s][8 * cc + e]));
        }
      }
    const int eq = fp8_exponent(pair_max32(qmax));
    qscale = eq + kE8M0One;
    const float qs = ldexpf(1.f, -eq);
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int w = 0; w < 8; ++w)
        qf[s][w] = static_cast<int>(pack4(qv[s][4 * w] * qs, qv[s][4 * w + 1] * qs,
                                          qv[s][4 * w + 2] * qs, qv[s][4 * w + 3] * qs));
  }

  // ---- tile staging: one 16-byte K chunk and kVLoads Vt chunks per thread ----
  const int kr = tid >> 3, kc = tid & 7;          // K row (key), chunk
  const int vc = tid & 7, vd0 = tid >> 3;         // Vt rows vd0 + 64 i, keys 8 vc ..
  const uint32_t tk = static_cast<uint32_t>(kr * kD + kc * 16);
  uint32_t tv[kVLoads];
#pragma unroll
  for (int i = 0; i < kVLoads; ++i) tv[i] = static_cast<uint32_t>(((vd0 + 64 * i) * Np + 8 * vc) * 2);
  const int ks_off = k_off(kr, kc);
  const uint32_t lane_slot = lane < n_pages ? static_cast<uint32_t>(G.slot[lane]) * page_bytes : 0u;
  int lp = 0, ltp = 0;                            // page and tile of the next load
  u32x4 kreg, vreg[kVLoads];
  auto load_next = [&]() {
    const uint32_t s0 = __builtin_amdgcn_readlane(lane_slot, lp);
    const uint32_t row0 = static_cast<uint32_t>(ltp * kBN);
    kreg = *reinterpret_cast<const u32x4*>(pool + (s0 + k_head + row0 * kD + tk));
#pragma unroll
    for (int i = 0; i < kVLoads; ++i)
      vreg[i] = *reinterpret_cast<const u32x4*>(pool + (s0 + v_head + row0 * 2u + tv[i]));
    if (++ltp == T) {
      ltp = 0;
      ++lp;
    }
  };
  auto store_tile = [&](int stage) {
    uint8_t* st = lds + stage * kStage;
    *reinterpret_cast<u32x4*>(st + ks_off) = kreg;
#pragma unroll
    for (int i = 0; i < kVLoads; ++i)
      *reinterpret_cast<u32x4*>(st + kKTile + ((vd0 + 64 * i) * kVPitch + 8 * vc) * 2) = vreg[i];
  };

  // LDS operand offsets of this lane: QK MFMA (t2, s) reads K row
  // qk_key(t2, col), chunks 4 s + 2 half + {0, 1}; PV MFMA (kk, dt) reads Vt
  // row 32 dt + col, keys 16 kk + 8 half ...
  // (qk_key(1, r) = qk_key(0, r) + 32: one base plus immediates)
  const int ka = k_off(qk_key(0, col), 2 * half);
  const int va = kKTile + (col * kVPitch + 8 * half) * 2;

  f32x16 oacc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) oacc[i] = f32x16{};
  f32x16 sacc[2];
  bf16x8 pf[2][2];
  // The QK accumulators start from moff = -m - kBias (m = this lane's
  // running max), so they hold S - m - kBias and P' = exp2(S) needs no
  // per-score arithmetic.
  f32x16 moff = f32x16{};
  bool first_tile = true;
  float l_run = 0.f;
  const bf16x2 ones = {static_cast<__bf16>(1.f), static_cast<__bf16>(1.f)};
  int kcode = kE8M0One;                           // K scale of the next QK tile

  // ---- MFMA cluster: O^T += Vt(t-1) P(t-1)^T, then S^T(t) = K(t) Q^T.
  // Fragments are read from LDS kAhead MFMAs ahead; the scheduling barriers
  // pin that order.  PV fragments are one 16-byte read, QK fragments two.
  constexpr int kAhead = 4;
  auto mfma_cluster = [&](int pv_stage, int qk_stage) {
    const uint8_t* vb = lds + pv_stage * kStage;
    const uint8_t* kb = lds + qk_stage * kStage;
    struct Frag {
      u32x4 lo, hi;
    };
    auto frag = [&](int i) -> Frag {
      Frag f;
      if (i < NPV) {
        const int kk = i >> 2, dt = i & 3;
        f.lo = *reinterpret_cast<const u32x4*>(vb + va + (dt * 32 * kVPitch + kk * 16) * 2);
        f.hi = f.lo;
      } else {
        const int j = i - NPV, s = j >> 1, t2 = j & 1;
        f.lo = *reinterpret_cast<const u32x4*>(kb + ka + t2 * 32 * kKPitch + 64 * s);
        f.hi = *reinterpret_cast<const u32x4*>(kb + ka + t2 * 32 * kKPitch + 64 * s + 16);
      }
      return f;
    };
    constexpr int NI = NPV + NQK;
    Frag fr[kAhead + 1];
#pragma unroll
    for (int i = 0; i < kAhead; ++i) fr[i] = frag(i);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      if (i + kAhead < NI) fr[(i + kAhead) % (kAhead + 1)] = frag(i + kAhead);
      const Frag f = fr[i % (kAhead + 1)];
      if (i < NPV) {
        const int kk = i >> 2, dt = i & 3;
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, f.lo),
                                                           pf[kk >> 1][kk & 1], oacc[dt], 0, 0, 0);
      } else {
        const int j = i - NPV, s = j >> 1, t2 = j & 1;
        i32x8 kf;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kf[e] = static_cast<int>(f.lo[e]);
          kf[4 + e] = static_cast<int>(f.hi[e]);
        }
        sacc[t2] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kf, qf[s], s == 0 ? moff : sacc[t2], 0, 0,
                                                                   0, kcode, 0, qscale);
      }
    }
    // Row sum of P(t-1), the rounded weights the PV product uses, in the
    // VALU slots between this wave's MFMAs.
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int a2 = 0; a2 < 2; ++a2)
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const bf16x2 pp = {pf[t2][a2][e], pf[t2][a2][e + 1]};
          l_run = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, l_run, false);
        }
    // order: the first kAhead fragments' reads, then (MFMA, reads of the
    // fragment kAhead further) pairs, then the last MFMAs
    __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i + kAhead < NPV) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      else if (i + kAhead < NI) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
  };

  // ---- VALU cluster: online softmax of S(t) (base 2, lazy rescale) ----
  // The accumulators hold S - m - kBias (m = the lane's running max), so the
  // weights come out as P' = 2^(S - m - kBias); numerator and denominator
  // share the factor 2^-kBias.  A weight reaches 2 (bf16 exponent field
  // >= 128: bit 14 of its half-word) exactly when S - m >= kBias + 1 = 8, so
  // one OR over the rounded weights tells whether m must move (lazy rescale
  // at 2^8) without a row max.  Then -- rarely -- the tile's scores are
  // multiplied again from LDS (the stage is intact until two clusters
  // later, and kcode still holds this tile's K scale), the row max is taken
  // and O, l and the weights are redone with the new m.  The first tile
  // takes the row max to start m.
  constexpr float kBias = 7.f;
  auto qk_again = [&](int qk_stage) {
    const uint8_t* kb = lds + qk_stage * kStage;
#pragma unroll
    for (int j = 0; j < NQK; ++j) {
      const int s = j >> 1, t2 = j & 1;
      const u32x4 lo = *reinterpret_cast<const u32x4*>(kb + ka + t2 * 32 * kKPitch + 64 * s);
      const u32x4 hi = *reinterpret_cast<const u32x4*>(kb + ka + t2 * 32 * kKPitch + 64 * s + 16);
      i32x8 kf;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kf[e] = static_cast<int>(lo[e]);
        kf[4 + e] = static_cast<int>(hi[e]);
      }
      sacc[t2] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kf, qf[s], s == 0 ? moff : sacc[t2], 0, 0, 0,
                                                                 kcode, 0, qscale);
    }
  };
  auto mask = [&](int valid) {
    // value v of sacc[t2] in lane half h is key 32 t2 + 16 (v / 8) + 8 h + (v % 8)
    if (valid < kBN) {
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if (32 * t2 + 16 * (v >> 3) + 8 * half + (v & 7) >= valid) sacc[t2][v] = -__builtin_inff();
    }
  };
  // m += up with up = the row max's growth (first tile: the row max itself)
  auto move_max = [&](bool first) {
    // max of the lane's 32 values as a tree of 3-input maxima, both halves
    float r[11];
#pragma unroll
    for (int i = 0; i < 10; ++i) {
      const int a0 = 3 * i, a1 = 3 * i + 1, a2 = 3 * i + 2;
      r[i] = fmaxf(fmaxf(sacc[a0 >> 4][a0 & 15], sacc[a1 >> 4][a1 & 15]), sacc[a2 >> 4][a2 & 15]);
    }
    r[10] = fmaxf(sacc[1][14], sacc[1][15]);
    const float r0 = fmaxf(fmaxf(r[0], r[1]), r[2]), r1 = fmaxf(fmaxf(r[3], r[4]), r[5]);
    const float r2 = fmaxf(fmaxf(r[6], r[7]), r[8]), r3 = fmaxf(r[9], r[10]);
    const float mx = pair_max32(fmaxf(fmaxf(r0, r1), fmaxf(r2, r3))) + kBias;
    const float up = first ? mx : fmaxf(mx, 0.f);
    if (!first) {
      const float alpha = __builtin_amdgcn_exp2f(-up);
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < 4; ++i) oacc[i] *= alpha;
    }
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      sacc[0][v] -= up;
      sacc[1][v] -= up;
      moff[v] -= up;
    }
  };
  auto weights = [&]() {
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        pf[t2][v >> 3][v & 7] = static_cast<__bf16>(__builtin_amdgcn_exp2f(sacc[t2][v]));
  };
  auto softmax = [&](int valid, int qk_stage) {
    mask(valid);
    if (first_tile) {
      first_tile = false;
      move_max(true);
    }
    weights();
    u32x4 w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = __builtin_bit_cast(u32x4, pf[i >> 1][i & 1]);
    const uint32_t o0 = w[0][0] | w[0][1] | w[0][2], o1 = w[0][3] | w[1][0] | w[1][1];
    const uint32_t o2 = w[1][2] | w[1][3] | w[2][0], o3 = w[2][1] | w[2][2] | w[2][3];
    const uint32_t o4 = w[3][0] | w[3][1] | w[3][2];
    const uint32_t any_big = (o0 | o1 | o2) | (o3 | o4 | w[3][3]);
    if (__any((any_big & 0x40004000u) != 0u)) {
      qk_again(qk_stage);
      mask(valid);
      move_max(false);
      weights();
    }
  };

  // ---- prologue: tiles 0..2 into stages 0..2.  The first MFMA cluster
  // multiplies P = 0 with the Vt region of the last stage, which is zeroed
  // so that stale LDS contents cannot turn 0 * x into NaN. ----
  const int pre = n_tiles < kStages - 1 ? n_tiles : kStages - 1;
  for (int t = 0; t < pre; ++t) {
    load_next();
    store_tile(t);
  }
  {
    const u32x4 z = {0u, 0u, 0u, 0u};
    uint8_t* vz = lds + (kStages - 1) * kStage + kKTile;
    for (int i = tid; i < kVTile / 16; i += kNT) *reinterpret_cast<u32x4*>(vz + 16 * i) = z;
  }
#pragma unroll
  for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
    for (int a2 = 0; a2 < 2; ++a2)
#pragma unroll
      for (int e = 0; e < 8; ++e) pf[t2][a2][e] = static_cast<__bf16>(0.f);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  kcode = tcode[0];

  // Ping-pong: the two wave groups run the same sequence of clusters one
  // cluster apart (group 1 first passes one extra barrier), so on every SIMD
  // one wave issues MFMAs while the other runs the softmax.  Every cluster
  // ends at a work-group barrier; both groups pass the same number.  A tile
  // stored after the barrier that closes cluster t is first read in cluster
  // t+2, and its stage was last read in cluster t-1.  The last MFMA
  // cluster's S^T is not used.
  if (pgroup == 1) __syncthreads();
  bool staged = false;
  int ptp = 0;                                    // tile-in-page of the softmax's tile
  // A wave whose 32 query rows all lie past N (the last query tile of a
  // chunk) has no products to compute: it only stages its share of every
  // tile and passes the same barriers, so its SIMD partner has the matrix
  // core to itself.
  if (__builtin_amdgcn_readfirstlane(qt * BM + wave * 32) >= N) {
    for (int t = 0; t <= n_tiles; ++t) {
      __syncthreads();
      if (t < n_tiles) {
        if (staged) store_tile((t + 2) & (kStages - 1));
        staged = false;
        if (t + 3 < n_tiles) {
          load_next();
          staged = true;
        }
      }
      __syncthreads();
    }
    if (pgroup == 0) __syncthreads();
    return;
  }
  for (int t = 0; t <= n_tiles; ++t) {
    __builtin_amdgcn_s_setprio(1);
    mfma_cluster((t - 1) & (kStages - 1), t & (kStages - 1));
    // The scores and the row sum are needed only after the barrier; this
    // empty statement keeps their MFMAs and additions in the cluster (the
    // compiler would otherwise sink them past the barrier into the softmax,
    // out of the raised-priority window).
    asm volatile("" : "+v"(sacc[0]), "+v"(sacc[1]), "+v"(l_run));
    __builtin_amdgcn_s_setprio(0);
    __syncthreads();
    if (t < n_tiles) {
      if (staged) store_tile((t + 2) & (kStages - 1));
      staged = false;
      if (t + 3 < n_tiles) {
        load_next();
        staged = true;
      }
      softmax(ptp == T - 1 ? last_valid : kBN, t & (kStages - 1));
      if (++ptp == T) ptp = 0;
      kcode = tcode[t + 1 < n_tiles ? t + 1 : t];
    }
    __syncthreads();
  }
  if (pgroup == 0) __syncthreads();

  // ---- epilogue: O = (O^T)^T / l, or the half's partial result ----
  const float l_sum = pair_sum32(l_run);
  if (G.part >= 0) {
    if (q < N) store_partial(a, G.part, q, h, -moff[0], l_sum, oacc, half);
    return;
  }
  const float inv = 1.f / l_sum;
  if (q < N) {
    __bf16* orow = static_cast<__bf16*>(a.out) + ((static_cast<int64_t>(G.stage) * N + q) * H + h) * kD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        bf16x4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] = static_cast<__bf16>(oacc[dt][4 * i4 + j] * inv);
        *reinterpret_cast<bf16x4*>(orow + 32 * dt + 8 * i4 + 4 * half) = o;
      }
  }
}

}  // namespace

hipError_t launch_attention_fp8k(const AttnArgs& a, hipStream_t stream) {
  if (a.n_items <= 0) return hipSuccess;
  if (a.D != kD) return hipErrorInvalidValue;
  hipLaunchKernelGGL(wf_attention_fp8k_kernel, dim3(a.n_items), dim3(kNT), 0, stream, a);
  return hipGetLastError();
}

}  // namespace wf
