// Wavefront-round attention for one layer: every active query group of the
// round in one launch.
//
// "Wave Forcing: Towards Speed-of-Light Streaming Video Generation" §3.1:
// Eq. 4 lets query stage s read active stage j iff j >= s, and Eq. 5 orders
// the context as anchor, clean history, live store, denoising chunks by
// increasing stage.  The mask is chunk-granular, so the host plan lists only
// readable pages: the kernel walks a group's pages as one virtual key range
// (key t -> page t / N, row t mod N) and never loads a masked tile.  Only
// the last tile of a range can be partial.  §4.2 Eq. 10 gives the per-stage
// key counts; groups are ordered longest first.
//
// bf16 instance (D = 64 or 128), CDNA4 MFMA v_mfma_f32_32x32x16_bf16:
//   * work item = (group, head, 256 query rows); 8 waves x 32 queries, in two
//     groups of 4 (waves i and i+4 share a SIMD).
//   * S^T = K Q^T: A = 32 keys x 16 dims of K from LDS, B = Q fragments held
//     in registers for the whole item.  Each lane ends up owning one query
//     (its column), so the row max is an in-lane reduction plus one
//     permlane32 swap; the row sum stays per lane until the epilogue.
//   * K rows enter the A operand in the order pi(r) (bits 2 and 3 of r
//     swapped).  Then the 8 accumulator values a lane holds for one 16-key
//     step are keys 8*half .. 8*half+7 of that step, which is exactly the B
//     operand layout of the PV product: P^T goes from the QK accumulator to
//     the PV MFMA without any lane exchange.
//   * O^T = Vt P^T: A = 32 value dims x 16 keys read from the Vt tile (keys
//     contiguous in the page layout), fp32 accumulation in registers.
//   * K and Vt tiles (64 keys) pass through a 4-stage LDS ring (140 KB, one
//     work-group per CU).  Rows are padded by one 16-byte chunk, which makes
//     the operand reads conflict-free.  Tile t+3 is fetched into registers
//     while tile t is multiplied and written to LDS one tile later, so no
//     load latency is waited on.
//   * Ping-pong: both wave groups run the same sequence of MFMA and softmax
//     clusters, one cluster apart, so on every SIMD one wave issues MFMAs
//     while the other runs the softmax; the MFMA wave runs at raised issue
//     priority (s_setprio).
//   * Online softmax in base 2.  The Q fragments carry the scale and the QK
//     accumulators start from minus the running max (and a bias of 2^-7), so
//     the product is already the exponent of P.  Whether a row max grew by
//     2^8 or more is read off the rounded weights' exponent bits (one OR per
//     tile, no row max); only then are the tile's scores recomputed and O, l
//     rescaled.  The row sum of P(t-1) is taken in the MFMA cluster of tile
//     t, where the wave's VALU slots are otherwise idle.
//
// fp32 instance (head_dim <= 128, % 4): a plain tiled kernel (4 lanes per
// query, 32-key LDS tiles, fp32 FMA), used for fp32 rounds.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "wf_kernels.h"
#include "wf_items.h"
#include "wf_partial.h"

namespace wf {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Group of a work item (groups are few; linear scan over kernel args).
__device__ inline int find_group(const AttnArgs& a, int item) {
  int g = 0;
  while (g + 1 < a.n_groups && item >= a.grp[g + 1].item0) ++g;
  return g;
}

// A-operand row order for the QK MFMA: swaps bits 2 and 3.
__device__ inline int perm_row(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

// v_permlane32_swap exchanges the upper half of its first operand with the
// lower half of its second.  With both operands = x the two results hold, in
// every lane, x of this lane and x of lane ^ 32 (in an order that depends on
// the half), so max and sum of the pair are the same in both halves.
__device__ inline float pair_max32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float pair_sum32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D>
__global__ __launch_bounds__(512, 1) void wf_attention_bf16_kernel(const AttnArgs a) {
  constexpr int BM = kAttnBM_bf16;  // 256 query rows per work-group
  constexpr int BN = 64;            // keys per tile
  constexpr int NT = 512;           // threads: 8 waves in two groups of 4
  constexpr int KSTEPS = D / 16;    // MFMA k-steps of QK^T
  constexpr int DT = D / 32;        // 32-row output tiles of O^T
  constexpr int KCH = D / 8;        // 16-byte chunks per K row
  constexpr int VCH = BN / 8;       // 16-byte chunks per Vt row
  // LDS rows are padded by one 16-byte chunk: K row r at r * KPITCH, Vt row
  // d at d * VPITCH (elements).  Lanes 0..15 of an operand read hit 16
  // different 16-byte bank groups, and a fragment's address is one base
  // register plus an immediate per k-step.
  constexpr int KPITCH = D + 8;
  constexpr int VPITCH = BN + 8;
  constexpr int KTILE = BN * KPITCH;  // elements of one padded K tile
  constexpr int VTILE = D * VPITCH;   // elements of one padded Vt tile
  constexpr int STAGES = 4;         // LDS ring of K+Vt tiles
  constexpr int KLOADS = BN * KCH / NT;
  constexpr int VLOADS = D * VCH / NT;
  constexpr int KROWS = NT / KCH;   // K rows covered by one load round
  constexpr int VROWS = NT / VCH;   // Vt rows covered by one load round
  constexpr int NPV = 4 * DT;       // PV MFMAs per tile
  constexpr int NQK = 2 * KSTEPS;   // QK MFMAs per tile
  static_assert(KCH >= 8 && KLOADS * NT == BN * KCH && VLOADS * NT == D * VCH, "shape");

  __shared__ __attribute__((aligned(16))) __bf16 lds[STAGES][KTILE + VTILE];

  if (static_cast<int>(blockIdx.x) >= a.n_items) return;
  const int item = xcd_item(blockIdx.x, a.n_items, a.q_tiles);   // whole units per XCD
  const int g = find_group(a, item);
  const AttnGroup& G = a.grp[g];
  const int li = item - G.item0;
  const int h = li / a.q_tiles;
  const int qt = li - h * a.q_tiles;
  const int N = a.N, H = a.H;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int col = lane & 31, half = lane >> 5;
  const int pgroup = wave >> 2;     // ping-pong group
  const int n_pages = G.n_pages;

  // Byte offsets inside this layer's pool fit in 32 bits (checked on the
  // host), so every load is "uniform base + 32-bit lane offset".
  const char* pool = static_cast<const char*>(a.pool);
  const uint32_t page_bytes = static_cast<uint32_t>(a.page_elems) * 2u;
  const uint32_t v_part = static_cast<uint32_t>(H) * N * D * 2u;   // Vt after K
  const uint32_t k_head = static_cast<uint32_t>(h) * N * D * 2u;
  const uint32_t v_head = v_part + static_cast<uint32_t>(h) * D * N * 2u;
  const int total = n_pages * N;
  const int n_full = total / BN;
  const int tail = total - n_full * BN;
  const int n_tiles = n_full + (tail > 0 ? 1 : 0);

  // Query fragments (B operand of S^T = K Q^T): lane holds query `col`,
  // dims 16 s + 8 half .. +7.  Rows past N are clamped (never stored).
  const int q = qt * BM + wave * 32 + col;
  const int qc = q < N ? q : N - 1;
  const __bf16* qrow = static_cast<const __bf16*>(a.q_rot) +
                       ((static_cast<int64_t>(G.stage) * N + qc) * H + h) * D;
  // The fragments are pre-multiplied by c = scale * log2(e) (and rounded to
  // bf16 again), so S^T comes out in base-2 exponent units.
  const float c = a.scale_log2e;
  bf16x8 qf[KSTEPS];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) {
    const bf16x8 x = *reinterpret_cast<const bf16x8*>(qrow + 16 * s + 8 * half);
#pragma unroll
    for (int e = 0; e < 8; ++e) qf[s][e] = static_cast<__bf16>(static_cast<float>(x[e]) * c);
  }

  // Per-thread load assignment: K rows kr0 + i*KROWS, chunk kc; Vt rows
  // (value dims) vd0 + i*VROWS, keys 8*vc .. 8*vc+7 of the tile.
  const int kc = tid % KCH, kr0 = tid / KCH;
  const int vc = tid % VCH, vd0 = tid / VCH;
  uint32_t tk[KLOADS], tv[VLOADS];
#pragma unroll
  for (int i = 0; i < KLOADS; ++i) tk[i] = static_cast<uint32_t>(((kr0 + i * KROWS) * D + kc * 8) * 2);
#pragma unroll
  for (int i = 0; i < VLOADS; ++i) tv[i] = static_cast<uint32_t>(((vd0 + i * VROWS) * N + vc * 8) * 2);

  // LDS byte addresses (within a stage) of this lane's MFMA operands: K row
  // pi(col), dims 8 half ..; Vt row col, keys 8 half ..
  const uint32_t ka = static_cast<uint32_t>((perm_row(col) * KPITCH + 8 * half) * 2);
  const uint32_t va = static_cast<uint32_t>((KTILE + col * VPITCH + 8 * half) * 2);
  const char* lds_bytes = reinterpret_cast<const char*>(&lds[0][0]);
  constexpr uint32_t kStageBytes = (KTILE + VTILE) * 2;

  u32x4 kreg[KLOADS], vreg[VLOADS];
  // Byte offset of every context page's slot, one page per lane; tile loads
  // read the two they need with v_readlane (uniform page index).
  const uint32_t lane_slot = lane < n_pages ? static_cast<uint32_t>(G.slot[lane]) * page_bytes : 0u;
  // Page and row of the next tile to load (a 64-key tile straddles at most
  // one page boundary, so the position advances without division).
  int lp = 0, lrow = 0, lnext = 0;

  // Global -> registers for tile `lnext`.  The partial last tile clamps its
  // keys past the end of the context to the tile's first key (finite data;
  // their scores are masked).
  auto load_tile = [&](auto last_c) {
    constexpr bool last = decltype(last_c)::value;
    const int p1 = lp + 1 < n_pages ? lp + 1 : lp;
    const uint32_t s0 = __builtin_amdgcn_readlane(lane_slot, lp);
    const uint32_t s1 = __builtin_amdgcn_readlane(lane_slot, p1);
    const int left = N - lrow;            // keys of the tile still in page lp
    const uint32_t kb0 = s0 + k_head + static_cast<uint32_t>(lrow * D * 2);
    const uint32_t kb1 = s1 + k_head + static_cast<uint32_t>((lrow - N) * D * 2);
#pragma unroll
    for (int i = 0; i < KLOADS; ++i) {
      const int r = kr0 + i * KROWS;
      uint32_t off = (r < left ? kb0 : kb1) + tk[i];
      if (last && r >= tail) off = kb0 + static_cast<uint32_t>(kc * 16);
      kreg[i] = *reinterpret_cast<const u32x4*>(pool + off);
    }
    const uint32_t vb0 = s0 + v_head + static_cast<uint32_t>(lrow * 2);
    const uint32_t vb1 = s1 + v_head + static_cast<uint32_t>((lrow - N) * 2);
    const uint32_t vbase = 8 * vc < left ? vb0 : vb1;
    const bool vclamp = last && 8 * vc >= tail;
#pragma unroll
    for (int i = 0; i < VLOADS; ++i) {
      const uint32_t off = vclamp ? vb0 + static_cast<uint32_t>((vd0 + i * VROWS) * N * 2) : vbase + tv[i];
      vreg[i] = *reinterpret_cast<const u32x4*>(pool + off);
    }
    lrow += BN;
    if (lrow >= N) {
      lrow -= N;
      ++lp;
    }
    ++lnext;
  };
  auto load_next = [&]() {
    if (lnext == n_full) load_tile(std::true_type{});
    else load_tile(std::false_type{});
  };
  auto store_tile = [&](int stage) {
    __bf16* kt = lds[stage];
    __bf16* vt = lds[stage] + KTILE;
#pragma unroll
    for (int i = 0; i < KLOADS; ++i)
      *reinterpret_cast<u32x4*>(kt + (kr0 + i * KROWS) * KPITCH + kc * 8) = kreg[i];
#pragma unroll
    for (int i = 0; i < VLOADS; ++i)
      *reinterpret_cast<u32x4*>(vt + (vd0 + i * VROWS) * VPITCH + vc * 8) = vreg[i];
  };

  f32x16 oacc[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) oacc[i] = f32x16{};
  f32x16 sacc[2];
  bf16x8 pf[2][2];
  // The QK accumulators start from moff = -m - kBias (m = this lane's
  // running max), so they hold c s - m - kBias and P' = exp2(S) needs no
  // per-score arithmetic.
  f32x16 moff = f32x16{};
  bool first_tile = true;
  float l_run = 0.f;
  const bf16x2 ones = {static_cast<__bf16>(1.f), static_cast<__bf16>(1.f)};

  // ---- MFMA cluster: O^T += Vt(t-1) P(t-1)^T, then S^T(t) = K(t) Q^T.
  // Operand fragments are read from LDS kAhead MFMAs ahead; the scheduling
  // barriers pin that order (the register allocator would otherwise read
  // each fragment right before its MFMA and expose the LDS latency).
  constexpr int kAhead = 4;
  auto mfma_cluster = [&](int pv_stage, int qk_stage) {
    const char* vbase = lds_bytes + pv_stage * kStageBytes;
    const char* kbase = lds_bytes + qk_stage * kStageBytes;
    auto frag = [&](int i) -> bf16x8 {
      if (i < NPV) {
        const int kk = i / DT, dt = i % DT;
        return *reinterpret_cast<const bf16x8*>(vbase + va + (dt * 32 * VPITCH + kk * 16) * 2);
      }
      const int j = i - NPV, s = j >> 1, t2 = j & 1;
      return *reinterpret_cast<const bf16x8*>(kbase + ka + (t2 * 32 * KPITCH + s * 16) * 2);
    };
    constexpr int NI = NPV + NQK;
    bf16x8 fr[kAhead + 1];
#pragma unroll
    for (int i = 0; i < kAhead; ++i) fr[i] = frag(i);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      if (i + kAhead < NI) fr[(i + kAhead) % (kAhead + 1)] = frag(i + kAhead);
      const bf16x8 f = fr[i % (kAhead + 1)];
      if (i < NPV) {
        const int kk = i / DT, dt = i % DT;
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, pf[kk >> 1][kk & 1], oacc[dt], 0, 0, 0);
      } else {
        const int j = i - NPV, s = j >> 1, t2 = j & 1;
        sacc[t2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, qf[s], s == 0 ? moff : sacc[t2], 0, 0, 0);
      }
    }
    // Row sum of P(t-1), the same rounded weights the PV product uses, in
    // the VALU slots between this wave's MFMAs (it is added before the
    // softmax of tile t can rescale l).
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int a2 = 0; a2 < 2; ++a2)
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const bf16x2 pp = {pf[t2][a2][e], pf[t2][a2][e + 1]};
          l_run = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, l_run, false);
        }
    // order: kAhead LDS reads, then (MFMA, LDS read) pairs, then MFMAs
    __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i + kAhead < NI) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
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
  // later), the row max is taken and O, l and the weights are redone with
  // the new m.  The first tile takes the row max to start m.
  constexpr float kBias = 7.f;
  auto qk_again = [&](int qk_stage) {
    const char* kbase = lds_bytes + qk_stage * kStageBytes;
#pragma unroll
    for (int j = 0; j < NQK; ++j) {
      const int s = j >> 1, t2 = j & 1;
      const bf16x8 f = *reinterpret_cast<const bf16x8*>(kbase + ka + (t2 * 32 * KPITCH + s * 16) * 2);
      sacc[t2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, qf[s], s == 0 ? moff : sacc[t2], 0, 0, 0);
    }
  };
  auto mask = [&](int valid) {
    // value v of tile t2 is key 32 t2 + 16 (v / 8) + 8 half + (v % 8)
    if (valid < BN) {
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
      for (int i = 0; i < DT; ++i) oacc[i] *= alpha;
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
  const int pre = n_tiles < STAGES - 1 ? n_tiles : STAGES - 1;
  for (int t = 0; t < pre; ++t) {
    load_next();
    store_tile(t);
  }
  {
    const u32x4 z = {0u, 0u, 0u, 0u};
    __bf16* vz = lds[STAGES - 1] + KTILE;
    for (int i = tid; i < VTILE / 8; i += NT) *reinterpret_cast<u32x4*>(vz + i * 8) = z;
  }
#pragma unroll
  for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
    for (int a2 = 0; a2 < 2; ++a2)
#pragma unroll
      for (int e = 0; e < 8; ++e) pf[t2][a2][e] = static_cast<__bf16>(0.f);
  __syncthreads();

  // Ping-pong: the two wave groups run the same sequence of clusters one
  // cluster apart (group 1 first passes one extra barrier), so on every SIMD
  // one wave issues MFMAs while the other runs the softmax.  Every cluster
  // ends at a work-group barrier; both groups pass the same number.  The
  // last MFMA cluster's S^T is not used.
  // Nothing from before the loop (query fragments, prologue tiles) is in
  // flight any more; saying so keeps the loop's only vector-memory waits on
  // the staged tile loads, where their data is consumed.
  __builtin_amdgcn_s_waitcnt(0);
  if (pgroup == 1) __syncthreads();
  bool staged = false;
  // A wave whose 32 query rows all lie past N (the last query tile of a
  // chunk) has no products to compute: it only stages its share of every
  // tile and passes the same barriers, so its SIMD partner has the matrix
  // core to itself.
  if (__builtin_amdgcn_readfirstlane(qt * BM + wave * 32) >= N) {
    for (int t = 0; t <= n_tiles; ++t) {
      __syncthreads();
      if (t < n_tiles) {
        if (staged) store_tile((t + 2) & (STAGES - 1));
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
    // The wave in its MFMA cluster gets issue priority over the SIMD's other
    // wave (in its softmax cluster), so the matrix core is fed first.
    __builtin_amdgcn_s_setprio(1);
    mfma_cluster((t - 1) & (STAGES - 1), t & (STAGES - 1));
    __builtin_amdgcn_s_setprio(0);
    __syncthreads();
    if (t < n_tiles) {
      // tile t+2 was fetched into registers one tile ago; its stage last
      // held tile t-2, whose final reader ran two clusters ago.
      if (staged) store_tile((t + 2) & (STAGES - 1));
      staged = false;
      if (t + 3 < n_tiles) {
        load_next();
        staged = true;
      }
      softmax(t < n_full ? BN : tail, t & (STAGES - 1));
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
    __bf16* orow = static_cast<__bf16*>(a.out) +
                   ((static_cast<int64_t>(G.stage) * N + q) * H + h) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        bf16x4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] = static_cast<__bf16>(oacc[dt][4 * i4 + j] * inv);
        *reinterpret_cast<bf16x4*>(orow + 32 * dt + 8 * i4 + 4 * half) = o;
      }
  }
}

// ------------------------------------------------------------- fp32 ----
constexpr int kF32Threads = 256;
constexpr int kF32Lanes = 4;                 // lanes per query
constexpr int kF32BN = 32;                   // keys per tile
constexpr int kF32MaxD = 128;

__global__ __launch_bounds__(kF32Threads) void wf_attention_f32_kernel(const AttnArgs a) {
  constexpr int QPB = kAttnBM_f32;
  constexpr int DPL = kF32MaxD / kF32Lanes;  // dims per lane (max)
  __shared__ float ks[kF32BN][kF32MaxD + 1];
  __shared__ float vs[kF32BN][kF32MaxD + 1];

  const int item = blockIdx.x;
  if (item >= a.n_items) return;
  const int g = find_group(a, item);
  const AttnGroup& G = a.grp[g];
  const int li = item - G.item0;
  const int h = li / a.q_tiles;
  const int qt = li - h * a.q_tiles;
  const int N = a.N, H = a.H, D = a.D;
  const int tid = threadIdx.x;
  const int qi = tid / kF32Lanes, part = tid % kF32Lanes;
  const int q = qt * QPB + qi;
  const int qc = q < N ? q : N - 1;
  const float* pool = static_cast<const float*>(a.pool);
  const int64_t hnd = static_cast<int64_t>(H) * N * D;
  const int64_t total = static_cast<int64_t>(G.n_pages) * N;
  const int n_tiles = static_cast<int>((total + kF32BN - 1) / kF32BN);

  const float* qrow = static_cast<const float*>(a.q_rot) +
                      ((static_cast<int64_t>(G.stage) * N + qc) * H + h) * D;
  float qv[DPL], o[DPL];
#pragma unroll
  for (int j = 0; j < DPL; ++j) {
    const int d = part + kF32Lanes * j;
    qv[j] = d < D ? qrow[d] : 0.f;
    o[j] = 0.f;
  }
  float m_run = -__builtin_inff(), l_run = 0.f;
  const float c = a.scale_log2e;

  for (int t = 0; t < n_tiles; ++t) {
    const int64_t key0 = static_cast<int64_t>(t) * kF32BN;
    __syncthreads();
    for (int idx = tid; idx < kF32BN * D; idx += kF32Threads) {
      const int r = idx / D, d = idx - r * D;
      const int64_t key = key0 + r;
      float x = 0.f;
      if (key < total) {
        const int p = static_cast<int>(key / N);
        const int64_t row = key - static_cast<int64_t>(p) * N;
        x = pool[static_cast<int64_t>(G.slot[p]) * a.page_elems + (static_cast<int64_t>(h) * N + row) * D + d];
      }
      ks[r][d] = x;
    }
    for (int idx = tid; idx < kF32BN * D; idx += kF32Threads) {
      const int d = idx / kF32BN, r = idx - d * kF32BN;
      const int64_t key = key0 + r;
      float x = 0.f;
      if (key < total) {
        const int p = static_cast<int>(key / N);
        const int64_t row = key - static_cast<int64_t>(p) * N;
        x = pool[static_cast<int64_t>(G.slot[p]) * a.page_elems + hnd +
                 (static_cast<int64_t>(h) * D + d) * N + row];
      }
      vs[r][d] = x;
    }
    __syncthreads();
    float sc[kF32BN];
    float mx = -__builtin_inff();
#pragma unroll
    for (int r = 0; r < kF32BN; ++r) {
      float part_dot = 0.f;
#pragma unroll
      for (int j = 0; j < DPL; ++j) {
        const int d = part + kF32Lanes * j;
        if (d < D) part_dot = __builtin_fmaf(qv[j], ks[r][d], part_dot);
      }
      part_dot += __shfl_xor(part_dot, 1);
      part_dot += __shfl_xor(part_dot, 2);
      sc[r] = key0 + r < total ? part_dot * c : -__builtin_inff();
      mx = fmaxf(mx, sc[r]);
    }
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int j = 0; j < DPL; ++j) o[j] *= alpha;
#pragma unroll
    for (int r = 0; r < kF32BN; ++r) {
      const float p = __builtin_amdgcn_exp2f(sc[r] - m_new);
      l_run += p;
#pragma unroll
      for (int j = 0; j < DPL; ++j) {
        const int d = part + kF32Lanes * j;
        if (d < D) o[j] = __builtin_fmaf(p, vs[r][d], o[j]);
      }
    }
  }
  if (q < N) {
    float* orow = static_cast<float*>(a.out) + ((static_cast<int64_t>(G.stage) * N + q) * H + h) * D;
    const float inv = 1.f / l_run;
#pragma unroll
    for (int j = 0; j < DPL; ++j) {
      const int d = part + kF32Lanes * j;
      if (d < D) orow[d] = o[j] * inv;
    }
  }
}

// ------------------------------------------------------------ combine ----
// Merges the two halves of each split group into the bf16 output: one thread
// per 8 dims of one (row, head).  Exact softmax merge: with M = max(e_a, e_b)
// and w = 2^(e - M), O = (O_a w_a + O_b w_b) / (l_a w_a + l_b w_b).
constexpr int kCombineThreads = 256;

__global__ __launch_bounds__(kCombineThreads) void wf_combine_kernel(const CombineArgs a) {
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  const int chunks = a.D / 8;
  const int64_t per_split = static_cast<int64_t>(a.N) * a.H * chunks;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * kCombineThreads + threadIdx.x;
  if (idx >= per_split * a.n_split) return;
  const int sp = static_cast<int>(idx / per_split);
  const int64_t rem = idx - sp * per_split;
  const int64_t rh = rem / chunks;                  // row * H + head
  const int c = static_cast<int>(rem - rh * chunks);
  const int64_t nh = static_cast<int64_t>(a.N) * a.H;
  const int64_t ra = (2 * sp) * nh + rh, rb = ra + nh;
  const float2 ea = reinterpret_cast<const float2*>(a.part_el)[ra];
  const float2 eb = reinterpret_cast<const float2*>(a.part_el)[rb];
  const float m = fmaxf(ea.x, eb.x);
  const float wa = __builtin_amdgcn_exp2f(ea.x - m), wb = __builtin_amdgcn_exp2f(eb.x - m);
  const float inv = 1.f / (ea.y * wa + eb.y * wb);
  const float* oa = a.part_o + ra * a.D + 8 * c;
  const float* ob = a.part_o + rb * a.D + 8 * c;
  bf16x8 r;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const f32x4 xa = *reinterpret_cast<const f32x4*>(oa + 4 * k);
    const f32x4 xb = *reinterpret_cast<const f32x4*>(ob + 4 * k);
#pragma unroll
    for (int j = 0; j < 4; ++j) r[4 * k + j] = static_cast<__bf16>((xa[j] * wa + xb[j] * wb) * inv);
  }
  __bf16* orow = static_cast<__bf16*>(a.out) + (static_cast<int64_t>(a.stage[sp]) * nh + rh) * a.D;
  *reinterpret_cast<bf16x8*>(orow + 8 * c) = r;
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream) {
  if (a.n_split <= 0) return hipSuccess;
  if (a.D % 8 != 0 || a.n_split > kMaxSplit) return hipErrorInvalidValue;
  const int64_t threads = static_cast<int64_t>(a.n_split) * a.N * a.H * (a.D / 8);
  const int64_t blocks = (threads + kCombineThreads - 1) / kCombineThreads;
  hipLaunchKernelGGL(wf_combine_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kCombineThreads), 0,
                     stream, a);
  return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs& a, int dtype, hipStream_t stream) {
  if (a.n_items <= 0) return hipSuccess;
  const dim3 grid(a.n_items);
  if (dtype == WF_BF16) {
    if (a.D == 128) {
      hipLaunchKernelGGL(wf_attention_bf16_kernel<128>, grid, dim3(512), 0, stream, a);
    } else if (a.D == 64) {
      hipLaunchKernelGGL(wf_attention_bf16_kernel<64>, grid, dim3(512), 0, stream, a);
    } else {
      return hipErrorInvalidValue;
    }
  } else {
    hipLaunchKernelGGL(wf_attention_f32_kernel, grid, dim3(kF32Threads), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace wf
