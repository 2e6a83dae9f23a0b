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
//   * work item = (group, head, 128 query rows); 4 waves x 32 queries.
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
//   * K and Vt tiles (64 keys) are double-buffered in LDS (64 KB per
//     work-group, two work-groups per CU); the next tile's global loads are
//     in flight while the current one is multiplied.  16-byte chunks are
//     XOR-swizzled per row so the MFMA operand reads spread over banks.
//   * Online softmax in base 2 with the scale folded into one FMA.
//
// fp32 instance (head_dim <= 128, % 4): a plain tiled kernel (4 lanes per
// query, 32-key LDS tiles, fp32 FMA), used for fp32 rounds.
#include <hip/hip_runtime.h>

#include "wf_kernels.h"

namespace wf {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
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

// K tile swizzle: distinct for the 8 rows one 8-lane group reads.
__device__ inline int kswz(int r) { return (r & 3) | ((r >> 1) & 4); }

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
__global__ __launch_bounds__(256, 2) void wf_attention_bf16_kernel(const AttnArgs a) {
  constexpr int BM = kAttnBM_bf16;  // 128 query rows per work-group
  constexpr int BN = 64;            // keys per tile
  constexpr int KSTEPS = D / 16;    // MFMA k-steps of QK^T
  constexpr int DT = D / 32;        // 32-row output tiles of O^T
  constexpr int KCH = D / 8;        // 16-byte chunks per K row
  constexpr int VCH = BN / 8;       // 16-byte chunks per Vt row
  constexpr int TILE = BN * D;      // elements of one K (or Vt) tile
  constexpr int KLOADS = BN * KCH / 256;
  constexpr int VLOADS = D * VCH / 256;
  static_assert(KCH >= 8 && KLOADS * 256 == BN * KCH && VLOADS * 256 == D * VCH, "shape");

  __shared__ __attribute__((aligned(16))) __bf16 lds[2][2 * TILE];

  const int item = blockIdx.x;
  if (item >= a.n_items) return;
  const int g = find_group(a, item);
  const AttnGroup& G = a.grp[g];
  const int li = item - G.item0;
  const int h = li / a.q_tiles;
  const int qt = li - h * a.q_tiles;
  const int N = a.N, H = a.H;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int col = lane & 31, half = lane >> 5;

  const __bf16* pool = static_cast<const __bf16*>(a.pool);
  const int64_t hnd = static_cast<int64_t>(H) * N * D;
  const int64_t total = static_cast<int64_t>(G.n_pages) * N;
  const int n_tiles = static_cast<int>((total + BN - 1) / BN);

  // Query fragments (B operand of S^T = K Q^T): lane holds query `col`,
  // dims 16 s + 8 half .. +7.  Rows past N are clamped (never stored).
  const int q = qt * BM + wave * 32 + col;
  const int qc = q < N ? q : N - 1;
  const __bf16* qrow = static_cast<const __bf16*>(a.q_rot) +
                       ((static_cast<int64_t>(G.stage) * N + qc) * H + h) * D;
  bf16x8 qf[KSTEPS];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(qrow + 16 * s + 8 * half);

  // Per-thread load assignment.
  const int kc = tid % KCH, kr0 = tid / KCH;        // K: chunk, first row
  const int vc = tid % VCH, vd0 = tid / VCH;        // Vt: key chunk, first dim
  u32x4 kreg[KLOADS], vreg[VLOADS];

  auto load_tile = [&](int t) {
    const int64_t key0 = static_cast<int64_t>(t) * BN;
    const int p0 = static_cast<int>(key0 / N);
    const int64_t bound = static_cast<int64_t>(p0 + 1) * N;
#pragma unroll
    for (int i = 0; i < KLOADS; ++i) {
      const int r = kr0 + i * (256 / KCH);
      const int64_t key = key0 + r;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (key < total) {
        const int p = key < bound ? p0 : p0 + 1;
        const int64_t row = key - static_cast<int64_t>(p) * N;
        const __bf16* src = pool + static_cast<int64_t>(G.slot[p]) * a.page_elems +
                            (static_cast<int64_t>(h) * N + row) * D + kc * 8;
        x = *reinterpret_cast<const u32x4*>(src);
      }
      kreg[i] = x;
    }
    // 8 keys of one Vt chunk never straddle a page (N % 8 == 0).
    const int64_t vkey = key0 + vc * 8;
    const bool vok = vkey < total;
    const int vp = vkey < bound ? p0 : p0 + 1;
    const int64_t vrow = vkey - static_cast<int64_t>(vp) * N;
    const __bf16* vbase = pool + static_cast<int64_t>(vok ? G.slot[vp] : 0) * a.page_elems + hnd +
                          static_cast<int64_t>(h) * D * N + vrow;
#pragma unroll
    for (int i = 0; i < VLOADS; ++i) {
      const int d = vd0 + i * (256 / VCH);
      u32x4 x = {0u, 0u, 0u, 0u};
      if (vok) x = *reinterpret_cast<const u32x4*>(vbase + static_cast<int64_t>(d) * N);
      vreg[i] = x;
    }
  };
  auto store_tile = [&](int buf) {
    __bf16* kt = lds[buf];
    __bf16* vt = lds[buf] + TILE;
#pragma unroll
    for (int i = 0; i < KLOADS; ++i) {
      const int r = kr0 + i * (256 / KCH);
      *reinterpret_cast<u32x4*>(kt + r * D + ((kc ^ kswz(r)) * 8)) = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < VLOADS; ++i) {
      const int d = vd0 + i * (256 / VCH);
      *reinterpret_cast<u32x4*>(vt + d * BN + ((vc ^ (d & 7)) * 8)) = vreg[i];
    }
  };

  f32x16 oacc[DT];
#pragma unroll
  for (int i = 0; i < DT; ++i) oacc[i] = f32x16{};
  float m_run = -__builtin_inff();
  float l_run = 0.f;
  const float c = a.scale_log2e;

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int t = 0; t < n_tiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < n_tiles) load_tile(t + 1);
    const __bf16* kt = lds[buf];
    const __bf16* vt = lds[buf] + TILE;

    // ---- S^T = K Q^T for 64 keys (two 32-key MFMA tiles) ----
    f32x16 sacc[2];
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
      sacc[t2] = f32x16{};
      const int r = 32 * t2 + perm_row(col);
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        const int ch = 2 * s + half;
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kt + r * D + ((ch ^ kswz(r)) * 8));
        sacc[t2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], sacc[t2], 0, 0, 0);
      }
    }

    // ---- online softmax (base 2); value v of tile t2 is key
    //      32 t2 + 16 (v / 8) + 8 half + (v % 8) ----
    const int64_t kbase = static_cast<int64_t>(t) * BN;
    if (kbase + BN > total) {
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int64_t key = kbase + 32 * t2 + 16 * (v >> 3) + 8 * half + (v & 7);
          if (key >= total) sacc[t2][v] = -__builtin_inff();
        }
    }
    float mx = sacc[0][0];
#pragma unroll
    for (int v = 1; v < 16; ++v) mx = fmaxf(mx, sacc[0][v]);
#pragma unroll
    for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sacc[1][v]);
    mx = pair_max32(mx);
    const float m_new = fmaxf(m_run, mx * c);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    float ls = 0.f;
    bf16x8 pf[2][2];
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[t2][v], c, -m_new));
        ls += p;
        pf[t2][v >> 3][v & 7] = static_cast<__bf16>(p);
      }
    l_run = l_run * alpha + ls;
#pragma unroll
    for (int i = 0; i < DT; ++i) oacc[i] *= alpha;

    // ---- O^T += Vt P^T ----
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int d = 32 * dt + col;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int ch = 2 * kk + half;
        const bf16x8 vf = *reinterpret_cast<const bf16x8*>(vt + d * BN + ((ch ^ (d & 7)) * 8));
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[kk >> 1][kk & 1], oacc[dt], 0, 0, 0);
      }
    }

    if (t + 1 < n_tiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = O^T^T / l ----
  const float l_tot = pair_sum32(l_run);
  const float inv = 1.f / l_tot;
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

}  // namespace

hipError_t launch_attention(const AttnArgs& a, int dtype, hipStream_t stream) {
  if (a.n_items <= 0) return hipSuccess;
  const dim3 grid(a.n_items);
  if (dtype == WF_BF16) {
    if (a.D == 128) {
      hipLaunchKernelGGL(wf_attention_bf16_kernel<128>, grid, dim3(256), 0, stream, a);
    } else if (a.D == 64) {
      hipLaunchKernelGGL(wf_attention_bf16_kernel<64>, grid, dim3(256), 0, stream, a);
    } else {
      return hipErrorInvalidValue;
    }
  } else {
    hipLaunchKernelGGL(wf_attention_f32_kernel, grid, dim3(kF32Threads), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace wf
