// Fused 3D-RoPE + paged K/V publish for one layer of one round.
//
// Producer step P_{s,l} of "Wave Forcing: Towards Speed-of-Light Streaming
// Video Generation" (§4.1 Eq. 8: Q/K/V then RoPE) followed by the paged
// write of App. B.2 (Eq. 13): each chunk's K/V goes straight into its fixed
// attention slot, so attention reads the ordered context with no gather.
// App. B.3: chunk 0's unrotated key is kept so RoPE can be re-applied when
// the window shifts (TASK_CAPTURE / TASK_ANCHOR).
//
// Grid: (64-token blocks, head groups, tasks).  A work-group owns one block
// of 64 tokens of one task and the heads one pass of its threads covers (two
// at D = 128).  A thread owns 8 consecutive tokens x one 16-byte chunk of a
// head row (8 bf16 / 4 fp32 elements):
//   * the rotation angles depend on the token and the pair, not on the head:
//     the work-group stages its block's angle table in LDS once, for all its
//     heads: the frame axis's cos/sin computed in fp64 from the absolute frame
//     position (so positions are not bounded by the length of a table), the
//     row and column axes' copied from fixed tables;
//   * a thread issues all 24 row loads of a head (q, k, v) before it uses
//     any, with no branch between them (the rows of a token group are valid
//     together: N % 8 == 0 for bf16, FP8 and FP8K; fp32 clamps its rows);
//   * its 8 x 8 (bf16) block of V is transposed in registers, so the page's
//     Vt rows (keys contiguous) are written with 16-byte stores; eight
//     consecutive lanes own the 8 token groups of one chunk, which makes
//     every load and store a 128-byte contiguous segment.
// HBM-bound: every byte is read once and written once.
#include <hip/hip_runtime.h>

#include "wf_kernels.h"

namespace wf {
namespace {

constexpr int kTokens = 64;    // tokens per work-group
constexpr int kThreads = 256;
constexpr int kRows = 8;       // consecutive tokens per thread

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <typename T>
struct Vec;
template <>
struct Vec<float> {
  static constexpr int n = 4;
  typedef f32x4 raw;
};
template <>
struct Vec<__bf16> {
  static constexpr int n = 8;
  typedef bf16x8 raw;
};

// The thread's place in a work-group: item = 8 tokens x one 16-byte chunk of
// one head; lanes 8 c + g own chunk c of token group g.
struct Geom {
  int hpp;    // heads a pass of the work-group covers
  int slot;   // head of this thread within a pass (>= hpp: idle)
  int g, c;   // token group (tokens 8 g .. 8 g + 7 of the block), chunk
};

__device__ inline Geom geom(int D, int vec) {
  Geom q;
  const int ipt = kRows * (D / vec);
  q.hpp = kThreads / ipt;
  const int t = threadIdx.x;
  q.slot = t / ipt;
  const int it = t - q.slot * ipt;
  q.c = it >> 3;
  q.g = it & 7;
  return q;
}

// Angle table of the work-group in LDS (float2 cos/sin):
//   [0, frames_max nt)            the frame axis at the frames the block
//                                 spans, computed in fp64 from the absolute
//                                 frame position (positions are not bounded
//                                 by a table's length)
//   [rows0, rows0 + Hh nh)        the row axis        } copied from the fixed
//   [cols0, cols0 + Ww nw)        the column axis     } rope_hw tables
// The copy issues eight independent loads per thread before it stores any.
// Returns f_lo, the first frame (within the chunk) the block spans.
__device__ inline int stage_angles(const PublishArgs& a, int frame0, int tok0, float2* tab) {
  const int hw = a.Hh * a.Ww;
  const int last = min(tok0 + kTokens, a.N) - 1;
  const int f_lo = tok0 / hw;
  const int nf = (last / hw - f_lo + 1) * a.nt;
  for (int i = threadIdx.x; i < nf; i += kThreads) {
    const int f = i / a.nt, m = i - f * a.nt;
    const double ang = static_cast<double>(static_cast<int64_t>(frame0) + f_lo + f) * a.omega_t[m];
    double s, c;
    sincos(ang, &s, &c);
    tab[i] = make_float2(static_cast<float>(c), static_cast<float>(s));
  }
  constexpr int kBatch = 8;
  const int n_hw = a.Hh * a.nh + a.Ww * a.nw;
  float2* dst = tab + a.frames_max * a.nt;
  for (int i0 = threadIdx.x; i0 < n_hw; i0 += kBatch * kThreads) {
    float2 v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) v[u] = a.rope_hw[min(i0 + u * kThreads, n_hw - 1)];
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
      if (i0 + u * kThreads < n_hw) dst[i0 + u * kThreads] = v[u];
  }
  __syncthreads();
  return f_lo;
}

// A thread's view of the angle table.  Its tokens are walked in order (the
// column steps, wrapping into the next row and frame), and the table index
// of pair p of the current token is base + p, the base chosen by p's axis.
struct Pos {
  int f, y, x;
};

template <int VEC>
struct Angles {
  int f_lo, f_last, p0, rows0, cols0;
  Pos first;

  __device__ Angles(const PublishArgs& a, int f_lo_, int t0, int c) {
    const int hw = a.Hh * a.Ww;
    f_lo = f_lo_;
    f_last = (min(t0 + kRows, a.N) - 1) / hw;      // the last frame staged for this thread
    p0 = c * VEC / 2;
    rows0 = a.frames_max * a.nt;
    cols0 = rows0 + a.Hh * a.nh;
    const int rem = t0 - (t0 / hw) * hw;
    first = Pos{t0 / hw, rem / a.Ww, rem - (rem / a.Ww) * a.Ww};
  }

  __device__ static void next(const PublishArgs& a, Pos& q) {
    if (++q.x == a.Ww) {
      q.x = 0;
      if (++q.y == a.Hh) {
        q.y = 0;
        ++q.f;
      }
    }
  }

  // cos/sin of the thread's pairs at position q
  __device__ void get(const PublishArgs& a, const float2* tab, const Pos& q, float2 (&cs)[VEC / 2]) const {
    const int bf = (min(q.f, f_last) - f_lo) * a.nt;
    const int by = rows0 + q.y * a.nh - a.nt;
    const int bx = cols0 + q.x * a.nw - (a.nt + a.nh);
#pragma unroll
    for (int e = 0; e < VEC / 2; ++e) {
      const int p = p0 + e;
      cs[e] = tab[(p < a.nt ? bf : (p < a.nt + a.nh ? by : bx)) + p];
    }
  }
};

// Rotated pairs (x_2e, x_2e+1) -> (x0 cos - x1 sin, x0 sin + x1 cos), fp32;
// cs = the row's VEC / 2 (cos, sin) pairs.
template <int VEC, typename R>
__device__ inline void rotate_f32(const R& x, const float2 (&cs)[VEC / 2], float (&out)[VEC]) {
#pragma unroll
  for (int e = 0; e < VEC / 2; ++e) {
    const float2 w = cs[e];
    const float x0 = static_cast<float>(x[2 * e]), x1 = static_cast<float>(x[2 * e + 1]);
    out[2 * e] = x0 * w.x - x1 * w.y;
    out[2 * e + 1] = x0 * w.y + x1 * w.x;
  }
}

template <typename T>
__device__ inline typename Vec<T>::raw rotate(const typename Vec<T>::raw& x,
                                              const float2 (&cs)[Vec<T>::n / 2]) {
  constexpr int VEC = Vec<T>::n;
  float r[VEC];
  rotate_f32<VEC>(x, cs, r);
  typename Vec<T>::raw out;
#pragma unroll
  for (int e = 0; e < VEC; ++e) out[e] = static_cast<T>(r[e]);
  return out;
}

// 16-byte access at a 32-bit byte offset from a uniform base (one layer's
// tensors and slots stay below 4 GiB, checked on the host).
template <typename R>
__device__ inline R ld16(const void* base, uint32_t off) {
  return *reinterpret_cast<const R*>(static_cast<const char*>(base) + off);
}
template <typename R>
__device__ inline void st16(void* base, uint32_t off, const R& v) {
  *reinterpret_cast<R*>(static_cast<char*>(base) + off) = v;
}

template <typename T>
__global__ __launch_bounds__(kThreads) void wf_publish_kernel(const PublishArgs a) {
  using raw = typename Vec<T>::raw;
  constexpr int VEC = Vec<T>::n;
  constexpr int kPieces = kRows / VEC;          // 16-byte pieces of 8 tokens
  constexpr uint32_t E = sizeof(T);
  extern __shared__ float2 lds_tab[];

  const PublishTask task = a.task[blockIdx.z];
  const int tok0 = blockIdx.x * kTokens;
  const int hg0 = blockIdx.y * a.heads_per_group;
  const int hg1 = min(a.H, hg0 + a.heads_per_group);
  const int N = a.N, H = a.H, D = a.D;
  const int f_lo = stage_angles(a, task.frame0, tok0, lds_tab);
  const Geom q = geom(D, VEC);
  const int t0 = tok0 + kRows * q.g;
  // Rows of the group are valid together (bf16: N % 8 == 0) or, for fp32
  // (N % 4 == 0), the first four alone; loads clamp to row N - 1.
  if (q.slot >= q.hpp || t0 >= N) return;
  const bool full = t0 + kRows <= N;
  const Angles<VEC> ang(a, f_lo, t0, q.c);
  uint32_t row[kRows];
#pragma unroll
  for (int i = 0; i < kRows; ++i) row[i] = static_cast<uint32_t>(min(i, N - 1 - t0));

  char* slot = static_cast<char*>(a.pool) + static_cast<int64_t>(task.slot) * a.page_bytes;
  const uint32_t vt_part = static_cast<uint32_t>(H) * N * D * E;   // Vt after K, in a page
  const bool capture = task.mode == TASK_CAPTURE;
  const uint32_t in_step = static_cast<uint32_t>(H) * D * E;       // one token row of q/k/v

  for (int h = hg0 + q.slot; h < hg1; h += q.hpp) {
    const uint32_t krow = ((static_cast<uint32_t>(h) * N + t0) * D + VEC * q.c) * E;   // K[h][t0][VEC c]
    const uint32_t vrow = vt_part + ((static_cast<uint32_t>(h) * D + VEC * q.c) * N + t0) * E;
    const uint32_t kstep = static_cast<uint32_t>(D) * E, vstep = static_cast<uint32_t>(N) * E;
    if (task.mode == TASK_ANCHOR) {
      // Key: the kept raw key re-rotated at the anchor's current position;
      // value: the kept Vt rows copied unchanged.
      raw xk[kRows], xv[VEC][kPieces];
#pragma unroll
      for (int i = 0; i < kRows; ++i) xk[i] = ld16<raw>(a.anchor_raw, krow + row[i] * kstep);
#pragma unroll
      for (int e = 0; e < VEC; ++e)
#pragma unroll
        for (int j = 0; j < kPieces; ++j)
          xv[e][j] = ld16<raw>(a.anchor_raw, vrow + e * vstep + (full ? VEC * j * E : 0u));
      Pos pos = ang.first;
#pragma unroll
      for (int i = 0; i < kRows; ++i) {
        if (!full && i >= VEC) break;
        float2 cs[VEC / 2];
        ang.get(a, lds_tab, pos, cs);
        st16(slot, krow + i * kstep, rotate<T>(xk[i], cs));
        ang.next(a, pos);
      }
#pragma unroll
      for (int e = 0; e < VEC; ++e)
#pragma unroll
        for (int j = 0; j < kPieces; ++j)
          if (full || j == 0) st16(slot, vrow + e * vstep + VEC * j * E, xv[e][j]);
      continue;
    }
    const uint32_t in0 = (((static_cast<uint32_t>(task.stage) * N + t0) * H + h) * D + VEC * q.c) * E;
    raw xq[kRows], xk[kRows], xv[kRows];
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
      xq[i] = ld16<raw>(a.q, in0 + row[i] * in_step);
      xk[i] = ld16<raw>(a.k, in0 + row[i] * in_step);
      xv[i] = ld16<raw>(a.v, in0 + row[i] * in_step);
    }
    Pos pos = ang.first;
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
      if (!full && i >= VEC) break;             // fp32: the last four rows past N
      float2 cs[VEC / 2];
      ang.get(a, lds_tab, pos, cs);
      st16(a.q_rot, in0 + i * in_step, rotate<T>(xq[i], cs));
      st16(slot, krow + i * kstep, rotate<T>(xk[i], cs));
      if (capture) st16(a.anchor_raw, krow + i * kstep, xk[i]);
      ang.next(a, pos);
    }
    // Transposed write: element e of the chunk is value dim VEC c + e; its
    // 8 tokens go out as kPieces 16-byte pieces.
#pragma unroll
    for (int e = 0; e < VEC; ++e)
#pragma unroll
      for (int j = 0; j < kPieces; ++j) {
        if (!full && j > 0) break;
        raw o;
#pragma unroll
        for (int u = 0; u < VEC; ++u) o[u] = xv[VEC * j + u][e];
        const uint32_t off = vrow + e * vstep + VEC * j * E;
        st16(slot, off, o);
        if (capture) st16(a.anchor_raw, off, o);
      }
  }
}

// ---------------------------------------------------------------- FP8 ----
// FP8 pages ("Wave Forcing" App. C.6: 8-bit K/V halve the payload).  A
// work-group owns one 64-token tile (blockIdx.x) of a group of heads, two
// heads per pass.  Rotated K and V of each (tile, head) get one power-of-two
// scale 2^e each, e the smallest integer with amax(tile) <= 448 * 2^e, and
// are stored as OCP E4M3 codes of x / 2^e (round to nearest even).  q_rot
// stays bf16.  Tokens N..Npad-1 are zero.  With kBf16V (the 8-bit QK^T
// tier) only K is quantised; Vt is written in bf16 (its scale code is 2^0).
constexpr int kFp8D = 128;

// Smallest e with amax <= 448 * 2^e (0 for amax == 0), exactly: with
// amax = m 2^x, m in [0.5, 1), 448 * 2^e = 0.875 * 2^(e + 9).
__device__ inline int fp8_exponent(float amax) {
  if (!(amax > 0.f)) return 0;
  int x;
  const float m = frexpf(amax, &x);
  const int e = m <= 0.875f ? x - 9 : x - 8;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// Eight floats (already divided by the scale, |x| <= 448) as E4M3 codes.
__device__ inline uint2 fp8_pack8(const float (&v)[8]) {
  uint2 r;
  r.x = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
  r.x = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], r.x, true);
  r.y = __builtin_amdgcn_cvt_pk_fp8_f32(v[4], v[5], 0, false);
  r.y = __builtin_amdgcn_cvt_pk_fp8_f32(v[6], v[7], r.y, true);
  return r;
}

__device__ inline float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

template <bool kBf16V>
__global__ __launch_bounds__(kThreads) void wf_publish_fp8_kernel(const PublishArgs a) {
  constexpr int D = kFp8D;
  extern __shared__ float2 lds_tab[];
  __shared__ float red[kThreads / 64][2];

  const PublishTask task = a.task[blockIdx.z];
  const int tile = blockIdx.x;
  const int tok0 = tile * kTokens;
  const int hg0 = blockIdx.y * a.heads_per_group;
  const int hg1 = min(a.H, hg0 + a.heads_per_group);
  const int N = a.N, H = a.H, Np = a.Npad;
  const int f_lo = stage_angles(a, task.frame0, tok0, lds_tab);
  const Geom q = geom(D, 8);                    // two heads per pass, 2 waves each
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t0 = tok0 + kRows * q.g;
  const bool valid = t0 < N;                    // N % 8 == 0: all 8 rows or none
  const Angles<8> ang(a, f_lo, valid ? t0 : N - kRows, q.c);

  char* page = static_cast<char*>(a.pool) + static_cast<int64_t>(task.slot) * a.page_bytes;
  const uint32_t v8_part = static_cast<uint32_t>(H) * Np * D;          // Vt after K8
  const uint32_t code_part = (kBf16V ? 3u : 2u) * static_cast<uint32_t>(H) * Np * D;
  const uint32_t anc_vt = static_cast<uint32_t>(H) * N * D * 2u;       // raw Vt after raw K (bf16)
  const uint32_t in_step = static_cast<uint32_t>(H) * D * 2u;
  const bool capture = task.mode == TASK_CAPTURE;
  const bool anchor = task.mode == TASK_ANCHOR;

  for (int hb = hg0; hb < hg1; hb += q.hpp) {   // uniform over the work-group
    const int h = hb + q.slot;
    const bool act = h < hg1;
    float kr[kRows][8];                         // rotated keys (+0 on padding rows)
    bf16x8 vt[8];                               // values, dim-major: vt[e][i] = v(t0 + i, 8 c + e)
#pragma unroll
    for (int i = 0; i < kRows; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) kr[i][e] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) vt[e] = bf16x8{};
    const uint32_t krow = ((static_cast<uint32_t>(h) * N + t0) * D + 8 * q.c) * 2u;   // raw K (bf16)
    const uint32_t vrow = anc_vt + ((static_cast<uint32_t>(h) * D + 8 * q.c) * N + t0) * 2u;
    if (act && valid && anchor) {
      bf16x8 xk[kRows];
#pragma unroll
      for (int i = 0; i < kRows; ++i) xk[i] = ld16<bf16x8>(a.anchor_raw, krow + i * D * 2u);
#pragma unroll
      for (int e = 0; e < 8; ++e) vt[e] = ld16<bf16x8>(a.anchor_raw, vrow + e * N * 2u);
      Pos pos = ang.first;
#pragma unroll
      for (int i = 0; i < kRows; ++i) {
        float2 cs[4];
        ang.get(a, lds_tab, pos, cs);
        rotate_f32<8>(xk[i], cs, kr[i]);
        ang.next(a, pos);
      }
    } else if (act && valid) {
      const uint32_t in0 = (((static_cast<uint32_t>(task.stage) * N + t0) * H + h) * D + 8 * q.c) * 2u;
      bf16x8 xq[kRows], xk[kRows], xv[kRows];
#pragma unroll
      for (int i = 0; i < kRows; ++i) {
        xq[i] = ld16<bf16x8>(a.q, in0 + i * in_step);
        xk[i] = ld16<bf16x8>(a.k, in0 + i * in_step);
        xv[i] = ld16<bf16x8>(a.v, in0 + i * in_step);
      }
      Pos pos = ang.first;
#pragma unroll
      for (int i = 0; i < kRows; ++i) {
        float2 cs[4];
        ang.get(a, lds_tab, pos, cs);
        ang.next(a, pos);
        st16(a.q_rot, in0 + i * in_step, rotate<__bf16>(xq[i], cs));
        rotate_f32<8>(xk[i], cs, kr[i]);
        if (capture) st16(a.anchor_raw, krow + i * D * 2u, xk[i]);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int i = 0; i < kRows; ++i) vt[e][i] = xv[i][e];
    }
    float kmax = 0.f, vmax = 0.f;
#pragma unroll
    for (int i = 0; i < kRows; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        kmax = fmaxf(kmax, fabsf(kr[i][e]));
        vmax = fmaxf(vmax, fabsf(static_cast<float>(vt[e][i])));
      }
    // tile amax of K and V over the head's two waves
    kmax = wave_max(kmax);
    vmax = wave_max(vmax);
    if (lane == 0) {
      red[wave][0] = kmax;
      red[wave][1] = vmax;
    }
    __syncthreads();
    const int w0 = wave & ~1;
    kmax = fmaxf(red[w0][0], red[w0 + 1][0]);
    vmax = fmaxf(red[w0][1], red[w0 + 1][1]);
    if (act) {
      const int ek = fp8_exponent(kmax), ev = kBf16V ? 0 : fp8_exponent(vmax);
      const float sk = ldexpf(1.f, -ek), sv = ldexpf(1.f, -ev);
      // K rows (padding rows get +0 codes)
      const uint32_t k8row = (static_cast<uint32_t>(h) * Np + t0) * D + 8 * q.c;
#pragma unroll
      for (int i = 0; i < kRows; ++i) {
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = kr[i][e] * sk;
        *reinterpret_cast<uint2*>(page + k8row + i * D) = fp8_pack8(x);
      }
      // Vt rows: 8 consecutive tokens of one value dim
      const uint32_t v8row = (static_cast<uint32_t>(h) * D + 8 * q.c) * Np + t0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (kBf16V) {
          st16(page, v8_part + (v8row + e * Np) * 2u, vt[e]);
        } else {
          float x[8];
#pragma unroll
          for (int i = 0; i < kRows; ++i) x[i] = static_cast<float>(vt[e][i]) * sv;
          *reinterpret_cast<uint2*>(page + v8_part + v8row + e * Np) = fp8_pack8(x);
        }
        if (capture && valid) st16(a.anchor_raw, vrow + e * N * 2u, vt[e]);
      }
      if (q.g == 0 && q.c == 0) {
        const uint16_t code = static_cast<uint16_t>((ek + 127) | ((ev + 127) << 8));
        *reinterpret_cast<uint16_t*>(page + code_part + (static_cast<uint32_t>(h) * a.T + tile) * 2u) = code;
      }
    }
    __syncthreads();                            // red is rewritten by the next pass
  }
}

// Heads per work-group: the heads one pass covers (two at D = 128).  Walking
// more heads per work-group reuses the block's angle table longer but leaves
// fewer work-groups to hide memory latency: on the 1.3B round one pass per
// work-group (2664 work-groups) measured 0.103 ms per launch against 0.109 ms
// with two or four passes.
int heads_per_group(int hpp) { return hpp; }

}  // namespace

int publish_frames_max(int F, int Hh, int Ww) {
  const int spans = (kTokens - 1) / (Hh * Ww) + 2;   // frames 64 consecutive tokens can touch
  return spans < F ? spans : F;
}

size_t publish_lds_bytes(int F, int Hh, int Ww, int nt, int nh, int nw) {
  return (size_t(publish_frames_max(F, Hh, Ww)) * nt + size_t(Hh) * nh + size_t(Ww) * nw) * sizeof(float2);
}

hipError_t launch_publish(const PublishArgs& args, int dtype, hipStream_t stream) {
  if (args.n_tasks <= 0) return hipSuccess;
  PublishArgs a = args;
  a.frames_max = publish_frames_max(a.F, a.Hh, a.Ww);
  const size_t lds = publish_lds_bytes(a.F, a.Hh, a.Ww, a.nt, a.nh, a.nw);
  if (lds > kPublishMaxLds) return hipErrorInvalidValue;
  const int vec = dtype == WF_F32 ? 4 : 8;
  const int hpp = kThreads / (kRows * (a.D / vec));
  if (hpp < 1 || a.D % vec != 0) return hipErrorInvalidValue;
  if (dtype == WF_FP8 || dtype == WF_FP8K) {
    if (a.D != kFp8D) return hipErrorInvalidValue;
    a.heads_per_group = heads_per_group(hpp);
    const dim3 grid(a.T, (a.H + a.heads_per_group - 1) / a.heads_per_group, a.n_tasks);
    if (dtype == WF_FP8) hipLaunchKernelGGL(wf_publish_fp8_kernel<false>, grid, dim3(kThreads), lds, stream, a);
    else hipLaunchKernelGGL(wf_publish_fp8_kernel<true>, grid, dim3(kThreads), lds, stream, a);
    return hipGetLastError();
  }
  const int blocks = (a.N + kTokens - 1) / kTokens;
  a.heads_per_group = heads_per_group(hpp);
  const dim3 grid(blocks, (a.H + a.heads_per_group - 1) / a.heads_per_group, a.n_tasks);
  if (dtype == WF_BF16) {
    hipLaunchKernelGGL(wf_publish_kernel<__bf16>, grid, dim3(kThreads), lds, stream, a);
  } else {
    hipLaunchKernelGGL(wf_publish_kernel<float>, grid, dim3(kThreads), lds, stream, a);
  }
  return hipGetLastError();
}

}  // namespace wf
