// Wavefront-round attention over FP8 pages, one layer, every active query
// group in one launch.
//
// "Wave Forcing: Towards Speed-of-Light Streaming Video Generation" §3.1
// Eq. 4-5 define the context (anchor, history, store, cleaner denoising
// chunks); App. C.6 (Eq. 20-21) is the 8-bit K/V variant.  Pages hold E4M3
// codes of K/2^eK and V/2^eV with one power-of-two scale per 64-token tile
// of a head; pages are padded to 64 T tokens, so a key tile never straddles
// two pages and only the last tile of each page is partial.
//
// CDNA4 v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3 x E4M3, fp32 accumulate):
//   * the matrix core applies the scales: per query column the row exponent
//     of Q (quantised here from the bf16 q_rot row times scale * log2(e)),
//     per tile the K or V exponent, so S comes out in base-2 exponent units
//     and O in true units;
//   * a lane holds 32 bytes of an operand; the product pairs byte j of lane
//     half h of A with byte j of lane half h of B, so any k order works as
//     long as both operands use the same one;
//   * S^T = K Q^T: K rows enter the A operand permuted so that the 16
//     accumulator values a lane holds of each 32-key half are keys
//     32 h + 16 t2 + v of the tile: the lane's 32 values are then exactly
//     the B operand bytes of the PV product (P^T, k = key), no lane exchange;
//   * O^T = Vt P^T, A = Vt rows (value dims), keys contiguous.
// Schedule: the 8 waves (32 query rows each) run in lockstep, one
// work-group barrier per 64-key tile.  The QK product runs one tile ahead
// of the softmax: in step t a wave issues PV of tile t-1 and the row sums
// (5 FP8 MFMAs) among the row max of S(t), issues QK of tile t+1 (4 MFMAs)
// among the exponentials of tile t, then stages tile t+2, so the matrix core
// works while the wave's VALU runs the softmax, and the softmax never waits
// for the scores it uses.  The scores of two consecutive tiles live in two
// register sets that swap roles every step.  K and Vt tiles live in a
// 4-stage LDS ring with 16-byte chunks XOR-swizzled per row (conflict-free
// operand reads and stores).  Softmax in base 2 with lazy rescale; the QK
// accumulators start from 2^7 divided by the running max (in exponent
// units), so the weights come out of one exp2 per score already biased by
// 2^7 and are rounded to E4M3 (at most 2^8 < 448).  The row
// sum is one more FP8 MFMA of an all-ones operand against the same rounded
// weights, so numerator and denominator use identical weights (and the
// VALU, the bottleneck here, does no per-weight addition).
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

constexpr int kD = 128;
constexpr int kBN = 64;             // keys per tile
constexpr int kNT = 512;            // threads: 8 waves
constexpr int kStages = 4;
constexpr int kKTile = kBN * kD;    // bytes of a K tile (64 rows x 128)
constexpr int kVTile = kD * kBN;    // bytes of a Vt tile (128 rows x 64)
constexpr int kStage = kKTile + kVTile;
constexpr int kE8M0One = 127;       // scale code of 2^0

__device__ inline int find_group(const AttnArgs& a, int item) {
  int g = 0;
  while (g + 1 < a.n_groups && item >= a.grp[g + 1].item0) ++g;
  return g;
}

// Byte offset of 16-byte chunk c of K row r / Vt row d inside a stage.
__device__ inline int k_off(int r, int c) {
  const int f = ((r >> 1) & 3) | (((r >> 5) & 1) << 2);
  return r * kD + ((c ^ f) << 4);
}
__device__ inline int v_off(int d, int c) { return kKTile + d * kBN + ((c ^ ((d >> 2) & 3)) << 4); }

// Key of A-operand row r of QK MFMA t2 (0/1): 32 h + 16 t2 + 4 a + b for
// r = 8 a + 4 h + b.
__device__ inline int qk_key(int t2, int r) { return 32 * ((r >> 2) & 1) + 16 * t2 + 4 * (r >> 3) + (r & 3); }

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

__global__ __launch_bounds__(kNT, 1) void wf_attention_fp8_kernel(const AttnArgs a) {
  constexpr int BM = kAttnBM_fp8;
  // Lazy rescale threshold and weight bias (log2 units): P' = 2^kBias P with
  // P <= 2^kRescale keeps P' <= 2^8 < 448, and weights down to 2^-13 stay in
  // E4M3's normal range.  The row sum uses the same P', so O is unchanged.
  constexpr float kRescale = 1.f;
  constexpr float kBias = 7.f;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kStages * kStage];
  __shared__ uint16_t tcode[kFp8MaxCtxTiles];   // (eK + 127) | (eV + 127) << 8

  if (static_cast<int>(blockIdx.x) >= a.n_items) return;
  const int item = xcd_item(blockIdx.x, a.n_items, a.q_tiles);   // whole units per XCD
  const int g = find_group(a, item);
  const AttnGroup& G = a.grp[g];
  const int li = item - G.item0;
  const int h = li / a.q_tiles;
  const int qt = li - h * a.q_tiles;
  const int N = a.N, H = a.H, Np = a.Npad, T = a.T;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int col = lane & 31, half = lane >> 5;
  const int n_pages = G.n_pages;
  const int n_tiles = n_pages * T;
  const int last_valid = N - kBN * (T - 1);       // keys in the last tile of a page

  const char* pool = static_cast<const char*>(a.pool);
  const uint32_t page_bytes = static_cast<uint32_t>(a.page_bytes);
  const uint32_t v_part = static_cast<uint32_t>(H) * Np * kD;
  const uint32_t k_head = static_cast<uint32_t>(h) * Np * kD;
  const uint32_t v_head = v_part + static_cast<uint32_t>(h) * kD * Np;
  const uint32_t code_head = 2 * v_part + static_cast<uint32_t>(h) * T * 2;

  // ---- scale codes of every tile of the context ----
  for (int i = tid; i < n_tiles; i += kNT) {
    const int p = i / T, tp = i - p * T;
    const uint32_t off = static_cast<uint32_t>(G.slot[p]) * page_bytes + code_head + 2u * tp;
    tcode[i] = *reinterpret_cast<const uint16_t*>(pool + off);
  }

  // ---- query row: B operand of S^T = K Q^T, quantised per row ----
  // Lane (col, half) holds dims 64 s + 32 half + j (j = 0..31) for k-steps
  // s = 0, 1; the other 64 dims of the row sit in lane col + 32 (1 - half).
  const int q = qt * BM + wave * 32 + col;
  const int qc = q < N ? q : N - 1;
  const __bf16* qrow = static_cast<const __bf16*>(a.q_rot) +
                       ((static_cast<int64_t>(G.stage) * N + qc) * H + h) * kD;
  // The row is multiplied by c = scale * log2(e) (fp32) before it is
  // quantised, so S comes out in base-2 exponent units.
  const float c = a.scale_log2e;
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
  const int qscale = eq + kE8M0One;
  const float qs = ldexpf(1.f, -eq);
  i32x8 qf[2];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int w = 0; w < 8; ++w)
      qf[s][w] = static_cast<int>(pack4(qv[s][4 * w] * qs, qv[s][4 * w + 1] * qs,
                                        qv[s][4 * w + 2] * qs, qv[s][4 * w + 3] * qs));

  // ---- tile staging: one 16-byte K chunk and one Vt chunk per thread ----
  const int kr = tid >> 3, kc = tid & 7;          // K row (key), chunk
  const int vd = tid >> 2, vc = tid & 3;          // Vt row (dim), chunk
  const uint32_t tk = static_cast<uint32_t>(kr * kD + kc * 16);
  const uint32_t tv = static_cast<uint32_t>(vd * Np + vc * 16);
  const int ks_off = k_off(kr, kc), vs_off = v_off(vd, vc);
  const uint32_t lane_slot = lane < n_pages ? static_cast<uint32_t>(G.slot[lane]) * page_bytes : 0u;
  int lp = 0, ltp = 0;                            // page and tile of the next load
  u32x4 kreg, vreg;
  auto load_next = [&]() {
    const uint32_t s0 = __builtin_amdgcn_readlane(lane_slot, lp);
    const uint32_t row0 = static_cast<uint32_t>(ltp * kBN);
    kreg = *reinterpret_cast<const u32x4*>(pool + (s0 + k_head + row0 * kD + tk));
    vreg = *reinterpret_cast<const u32x4*>(pool + (s0 + v_head + row0 + tv));
    if (++ltp == T) {
      ltp = 0;
      ++lp;
    }
  };
  auto store_tile = [&](int stage) {
    uint8_t* st = lds + stage * kStage;
    *reinterpret_cast<u32x4*>(st + ks_off) = kreg;
    *reinterpret_cast<u32x4*>(st + vs_off) = vreg;
  };

  // LDS operand offsets of this lane: QK MFMA (t2, s) reads K row
  // qk_key(t2, col) chunks 4 s + 2 half + {0, 1}; PV MFMA dt reads Vt row
  // 32 dt + col chunks 2 half + {0, 1}.
  int ka[2][2][2], va[4][2];
#pragma unroll
  for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int u = 0; u < 2; ++u) ka[t2][s][u] = k_off(qk_key(t2, col), 4 * s + 2 * half + u);
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int u = 0; u < 2; ++u) va[dt][u] = v_off(32 * dt + col, 2 * half + u);

  f32x16 oacc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) oacc[i] = f32x16{};
  f32x16 sA[2], sB[2];                            // S^T of two consecutive tiles
  f32x16 lacc = f32x16{};                         // row sums: ones x P^T
  i32x8 pf = {};
  i32x8 ones;
#pragma unroll
  for (int w = 0; w < 8; ++w) ones[w] = 0x38383838;   // E4M3 1.0
  // The QK accumulators start from moff = kBias - m (m = this lane's running
  // max), so they hold S - m + kBias and P' = exp2(S) needs no per-score op.
  f32x16 moff = f32x16{};
  bool first_tile = true;
  int kcode = kE8M0One, vcode = kE8M0One;         // scales of the tiles in use

  // one 32-byte operand fragment from two 16-byte LDS chunks
  auto frag = [&](const uint8_t* p0, const uint8_t* p1) -> i32x8 {
    const u32x4 lo = *reinterpret_cast<const u32x4*>(p0);
    const u32x4 hi = *reinterpret_cast<const u32x4*>(p1);
    i32x8 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      r[e] = static_cast<int>(lo[e]);
      r[4 + e] = static_cast<int>(hi[e]);
    }
    return r;
  };
  // ---- O^T += Vt(t-1) P(t-1)^T and the row sums (ones x P^T) ----
  auto pv_cluster = [&](int pv_stage) {
    const uint8_t* vb = lds + pv_stage * kStage;
    i32x8 fr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) fr[i] = frag(vb + va[i][0], vb + va[i][1]);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      oacc[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fr[i], pf, oacc[i], 0, 0, 0, vcode, 0, kE8M0One);
    lacc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ones, pf, lacc, 0, 0, 0, kE8M0One, 0, kE8M0One);
  };
  // ---- S^T = K Q^T of one tile into sn, from the current moff ----
  auto qk_issue = [&](int qk_stage, f32x16 (&sn)[2]) {
    const uint8_t* kb = lds + qk_stage * kStage;
    i32x8 fr[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int s2 = j >> 1, t2 = j & 1;
      fr[j] = frag(kb + ka[t2][s2][0], kb + ka[t2][s2][1]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int s2 = j >> 1, t2 = j & 1;
      sn[t2] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fr[j], qf[s2], s2 == 0 ? moff : sn[t2], 0, 0, 0,
                                                              kcode, 0, qscale);
    }
  };
  // ---- online softmax of sc = S(t) (base 2, lazy rescale), with PV of
  // tile t-1 among its row max and QK of tile t+1 into sn among its
  // exponentials.  QK is issued after the rescale decision, so it starts
  // from the moved m.  Value v of sc[t2] in lane (col, half) is key
  // 32 half + 16 t2 + v. ----
  auto softmax = [&](int valid, f32x16 (&sc)[2], f32x16 (&sn)[2], int qk_stage, int pv_stage) {
    if (valid < kBN) {
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if (32 * half + 16 * t2 + v >= valid) sc[t2][v] = -__builtin_inff();
    }
    pv_cluster(pv_stage);
    // max of the lane's 32 values (S - m + kBias) as a tree of 3-input maxima
    float r[11];
#pragma unroll
    for (int i = 0; i < 10; ++i) {
      const int a0 = 3 * i, a1 = 3 * i + 1, a2 = 3 * i + 2;
      r[i] = fmaxf(fmaxf(sc[a0 >> 4][a0 & 15], sc[a1 >> 4][a1 & 15]), sc[a2 >> 4][a2 & 15]);
    }
    r[10] = fmaxf(sc[1][14], sc[1][15]);
    const float r0 = fmaxf(fmaxf(r[0], r[1]), r[2]), r1 = fmaxf(fmaxf(r[3], r[4]), r[5]);
    const float r2 = fmaxf(fmaxf(r[6], r[7]), r[8]), r3 = fmaxf(r[9], r[10]);
    const float mx = pair_max32(fmaxf(fmaxf(r0, r1), fmaxf(r2, r3))) - kBias;   // max S - m
    // order: the 8 Vt operand reads, then each PV MFMA with 3 VALU ops of
    // the row max
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 1);
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
      __builtin_amdgcn_sched_group_barrier(0x002, 3, 1);
    }
    // Lazy rescale: m moves only when some lane's max exceeds it by more
    // than 2^kRescale (always on the first tile).  (The vote and the flag
    // are combined without a branch, which keeps the PV MFMAs in the row
    // max's block.)
    const bool grow = __any(mx > kRescale);
    float alpha = 1.f;
    bool rescale = false;                         // wave-uniform
    if (grow | first_tile) {
      const float up = first_tile ? mx : fmaxf(mx, 0.f);
      if (!first_tile) {
        alpha = __builtin_amdgcn_exp2f(-up);
        rescale = true;
      }
      // (before the first tile the accumulators start from 0, i.e. m = kBias)
      first_tile = false;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        sc[0][v] -= up;
        sc[1][v] -= up;
        moff[v] -= up;
      }
    }
    qk_issue(qk_stage, sn);
    float p[2][16];
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int v = 0; v < 16; ++v) p[t2][v] = __builtin_amdgcn_exp2f(sc[t2][v]);
    // byte j = 16 t2 + v of the PV B operand
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const int t2 = w >> 2, v0 = 4 * (w & 3);
      pf[w] = static_cast<int>(pack4(p[t2][v0], p[t2][v0 + 1], p[t2][v0 + 2], p[t2][v0 + 3]));
    }
    // order: the 8 K operand reads, then each QK MFMA with 10 VALU ops of
    // the exponentials and the E4M3 packing
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 10, 0);
    }
    // O and l take the new m at the end of the softmax: PV of tile t-1,
    // issued among the row max, has finished by then
    if (rescale) {
      lacc *= alpha;
#pragma unroll
      for (int i = 0; i < 4; ++i) oacc[i] *= alpha;
    }
  };

  // ---- prologue: tiles 0..2 into stages 0..2; stage 3's Vt zeroed (the
  // first step multiplies P = 0 with it); QK of tile 0 ----
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
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  kcode = tcode[0] & 0xff;
  qk_issue(0, sA);

  // One barrier per tile orders the LDS ring: at its end, step t stores
  // tile t+2 (fetched at the end of step t-1, so its loads had a whole step
  // to land) into the stage that held tile t-2, whose last reader (PV in
  // step t-1) every wave finished (LDS reads drained) before the barrier
  // closing step t-1; tile t+1's K (read in step t) was stored at the end
  // of step t-1, and tile t-1's Vt (read in step t) at the end of step t-3.
  // The QK of step n_tiles - 1 reads a stale stage; its scores are never
  // used.
  bool staged = false;
  int ptp = 0;                                    // tile-in-page of the softmax's tile
  auto step = [&](int t, f32x16 (&sc)[2], f32x16 (&sn)[2]) {
    // scales: QK of tile t+1 now, PV of tile t in the next step
    const int nxt = t + 1 < n_tiles ? t + 1 : t;
    kcode = tcode[nxt] & 0xff;
    softmax(ptp == T - 1 ? last_valid : kBN, sc, sn, (t + 1) & (kStages - 1), (t - 1) & (kStages - 1));
    if (++ptp == T) ptp = 0;
    vcode = tcode[t] >> 8;
    // staging after the softmax: the LDS stores stay out of the operand
    // reads' way, and a late load stalls the wave while its QK MFMAs run
    if (staged) store_tile((t + 2) & (kStages - 1));
    staged = false;
    if (t + 3 < n_tiles) {
      load_next();
      staged = true;
    }
    // keep the QK MFMAs and the weights before the barrier (their results
    // are used only after it; the compiler would sink them past it)
    asm volatile("" : "+v"(sn[0]), "+v"(sn[1]), "+v"(pf));
    __builtin_amdgcn_sched_barrier(0); __syncthreads(); __builtin_amdgcn_sched_barrier(0);
  };
  for (int t = 0; t < n_tiles; t += 2) {         // the score sets swap roles every step
    step(t, sA, sB);
    if (t + 1 < n_tiles) step(t + 1, sB, sA);
  }
  pv_cluster((n_tiles - 1) & (kStages - 1));      // PV of the last tile

  // ---- epilogue: O = (O^T)^T / l, or the half's partial result ----
  // The lane's query row is derived again from the lane id (read by an asm
  // statement the compiler cannot merge with the first read), so no
  // register carries it through the tile loop.
  uint32_t lane_e;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane_e));
  const int half_e = static_cast<int>(lane_e >> 5);
  const int q_e = qt * BM + wave * 32 + static_cast<int>(lane_e & 31);
  if (G.part >= 0) {
    if (q_e < N) store_partial(a, G.part, q_e, h, -moff[0], lacc[0], oacc, half_e);
    return;
  }
  const float inv = 1.f / lacc[0];
  if (q_e < N) {
    __bf16* orow = static_cast<__bf16*>(a.out) + ((static_cast<int64_t>(G.stage) * N + q_e) * H + h) * kD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        bf16x4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] = static_cast<__bf16>(oacc[dt][4 * i4 + j] * inv);
        *reinterpret_cast<bf16x4*>(orow + 32 * dt + 8 * i4 + 4 * half_e) = o;
      }
  }
}

}  // namespace

hipError_t launch_attention_fp8(const AttnArgs& a, hipStream_t stream) {
  if (a.n_items <= 0) return hipSuccess;
  if (a.D != kD) return hipErrorInvalidValue;
  hipLaunchKernelGGL(wf_attention_fp8_kernel, dim3(a.n_items), dim3(kNT), 0, stream, a);
  return hipGetLastError();
}

}  // namespace wf
