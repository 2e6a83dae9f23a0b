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
// of 64 tokens of one task and a group of heads, which it walks a few heads
// at a time.  A thread owns 8 consecutive tokens x one 16-byte chunk of a
// head row (8 bf16 / 4 fp32 elements):
//   * its rotation angles depend on the token and the pair, not on the head,
//     so the thread forms its cos/sin once and reuses them for every head of
//     the group;
//   * the frame-axis cos/sin come from the absolute frame position, computed
//     in fp64 per work-group (frames x pairs of the block), so positions are
//     not bounded by the length of a table; the row and column tables are
//     fixed (Hh and Ww positions);
//   * the thread's 8 x 8 (bf16) block of V is transposed in registers, so the
//     page's Vt rows (keys contiguous) are written with 16-byte stores; eight
//     consecutive lanes own the 8 token groups of one chunk, which makes every
//     load and store a 128-byte contiguous segment.
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

// cos/sin of the frame-axis pairs at every frame the block's tokens span:
// angle = (frame0 + f) * omega_m in fp64, rounded to fp32.  ftab[f * nt + m].
__device__ inline int frame_table(const PublishArgs& a, int frame0, int tok0, float2* ftab) {
  const int hw = a.Hh * a.Ww;
  const int last = min(tok0 + kTokens, a.N) - 1;
  const int f_lo = tok0 / hw;
  const int n = (last / hw - f_lo + 1) * a.nt;
  for (int i = threadIdx.x; i < n; i += kThreads) {
    const int f = i / a.nt, m = i - f * a.nt;
    const double ang = static_cast<double>(static_cast<int64_t>(frame0) + f_lo + f) * a.omega_t[m];
    double s, c;
    sincos(ang, &s, &c);
    ftab[i] = make_float2(static_cast<float>(c), static_cast<float>(s));
  }
  return f_lo;
}

// cos/sin of this thread's pairs (VEC / 2 per token) for its 8 tokens.
template <int VEC>
__device__ inline void thread_angles(const PublishArgs& a, const float2* ftab, int f_lo, int t0,
                                     int c, float2 (&cs)[kRows][VEC / 2]) {
  const float2* th = a.rope_hw;              // [Hh][nh]
  const float2* tw = th + a.Hh * a.nh;       // [Ww][nw]
  const int hw = a.Hh * a.Ww;
#pragma unroll
  for (int i = 0; i < kRows; ++i) {
    const int tok = min(t0 + i, a.N - 1);    // rows past N are never stored
    const int f = tok / hw - f_lo, y = (tok / a.Ww) % a.Hh, x = tok % a.Ww;
#pragma unroll
    for (int e = 0; e < VEC / 2; ++e) {
      const int p = (c * VEC >> 1) + e;
      if (p < a.nt) {
        cs[i][e] = ftab[f * a.nt + p];
      } else if (p < a.nt + a.nh) {
        cs[i][e] = th[y * a.nh + (p - a.nt)];
      } else {
        cs[i][e] = tw[x * a.nw + (p - a.nt - a.nh)];
      }
    }
  }
}

// Rotated pairs (x_2e, x_2e+1) -> (x0 cos - x1 sin, x0 sin + x1 cos), fp32.
template <int VEC, typename R>
__device__ inline void rotate_f32(const R& x, const float2 (&cs)[VEC / 2], float (&out)[VEC]) {
#pragma unroll
  for (int e = 0; e < VEC / 2; ++e) {
    const float x0 = static_cast<float>(x[2 * e]), x1 = static_cast<float>(x[2 * e + 1]);
    out[2 * e] = x0 * cs[e].x - x1 * cs[e].y;
    out[2 * e + 1] = x0 * cs[e].y + x1 * cs[e].x;
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

template <typename T>
__global__ __launch_bounds__(kThreads) void wf_publish_kernel(const PublishArgs a) {
  using raw = typename Vec<T>::raw;
  constexpr int VEC = Vec<T>::n;
  constexpr int kPieces = kRows / VEC;          // 16-byte pieces of 8 tokens
  __shared__ float2 ftab[kMaxFrameEntries];

  const PublishTask task = a.task[blockIdx.z];
  const int tok0 = blockIdx.x * kTokens;
  const int hg0 = blockIdx.y * a.heads_per_group;
  const int hg1 = min(a.H, hg0 + a.heads_per_group);
  const int N = a.N, H = a.H, D = a.D;
  const Geom q = geom(D, VEC);
  const int f_lo = frame_table(a, task.frame0, tok0, ftab);
  __syncthreads();
  if (q.slot >= q.hpp) return;
  float2 cs[kRows][VEC / 2];
  const int t0 = tok0 + kRows * q.g;
  thread_angles<VEC>(a, ftab, f_lo, t0, q.c, cs);

  const int64_t hnd = static_cast<int64_t>(H) * N * D;
  T* pageK = static_cast<T*>(a.pool) + static_cast<int64_t>(task.slot) * a.page_elems;  // [H][N][D]
  T* pageVt = pageK + hnd;                                                             // [H][D][N]
  T* ancK = static_cast<T*>(a.anchor_raw);
  T* ancVt = ancK + hnd;
  const bool capture = task.mode == TASK_CAPTURE;

  for (int h = hg0 + q.slot; h < hg1; h += q.hpp) {
    const int64_t krow = (static_cast<int64_t>(h) * N + t0) * D + VEC * q.c;   // K[h][t0][VEC c]
    const int64_t vrow = (static_cast<int64_t>(h) * D + VEC * q.c) * N + t0;   // Vt[h][VEC c][t0]
    if (task.mode == TASK_ANCHOR) {
      // Key: the kept raw key re-rotated at the anchor's current position.
#pragma unroll
      for (int i = 0; i < kRows; ++i) {
        if (t0 + i >= N) break;
        const raw x = *reinterpret_cast<const raw*>(ancK + krow + int64_t(i) * D);
        *reinterpret_cast<raw*>(pageK + krow + int64_t(i) * D) = rotate<T>(x, cs[i]);
      }
      // Value: the kept Vt rows copied unchanged.
#pragma unroll
      for (int e = 0; e < VEC; ++e)
#pragma unroll
        for (int j = 0; j < kPieces; ++j) {
          if (t0 + VEC * j >= N) break;
          const int64_t off = vrow + int64_t(e) * N + VEC * j;
          *reinterpret_cast<raw*>(pageVt + off) = *reinterpret_cast<const raw*>(ancVt + off);
        }
      continue;
    }
    const T* qin = static_cast<const T*>(a.q);
    const T* kin = static_cast<const T*>(a.k);
    const T* vin = static_cast<const T*>(a.v);
    T* qr = static_cast<T*>(a.q_rot);
    const int64_t in0 = ((static_cast<int64_t>(task.stage) * N + t0) * H + h) * D + VEC * q.c;
    const int64_t in_step = static_cast<int64_t>(H) * D;
    raw xq[kRows], xk[kRows], xv[kRows];
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
      if (t0 + i < N) {
        xq[i] = *reinterpret_cast<const raw*>(qin + in0 + i * in_step);
        xk[i] = *reinterpret_cast<const raw*>(kin + in0 + i * in_step);
        xv[i] = *reinterpret_cast<const raw*>(vin + in0 + i * in_step);
      } else {
        xq[i] = raw{};
        xk[i] = raw{};
        xv[i] = raw{};
      }
    }
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
      if (t0 + i >= N) break;
      *reinterpret_cast<raw*>(qr + in0 + i * in_step) = rotate<T>(xq[i], cs[i]);
      *reinterpret_cast<raw*>(pageK + krow + int64_t(i) * D) = rotate<T>(xk[i], cs[i]);
      if (capture) *reinterpret_cast<raw*>(ancK + krow + int64_t(i) * D) = xk[i];
    }
    // Transposed write: element e of the chunk is value dim VEC c + e; its
    // 8 tokens go out as kPieces 16-byte pieces.
#pragma unroll
    for (int e = 0; e < VEC; ++e)
#pragma unroll
      for (int j = 0; j < kPieces; ++j) {
        if (t0 + VEC * j >= N) break;
        raw o;
#pragma unroll
        for (int u = 0; u < VEC; ++u) o[u] = xv[VEC * j + u][e];
        const int64_t off = vrow + int64_t(e) * N + VEC * j;
        *reinterpret_cast<raw*>(pageVt + off) = o;
        if (capture) *reinterpret_cast<raw*>(ancVt + off) = o;
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
  __shared__ float2 ftab[kMaxFrameEntries];
  __shared__ float red[kThreads / 64][2];

  const PublishTask task = a.task[blockIdx.z];
  const int tile = blockIdx.x;
  const int tok0 = tile * kTokens;
  const int hg0 = blockIdx.y * a.heads_per_group;
  const int hg1 = min(a.H, hg0 + a.heads_per_group);
  const int N = a.N, H = a.H, Np = a.Npad;
  const Geom q = geom(D, 8);                    // two heads per pass, 2 waves each
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int f_lo = frame_table(a, task.frame0, tok0, ftab);
  __syncthreads();
  float2 cs[kRows][4];
  const int t0 = tok0 + kRows * q.g;
  thread_angles<8>(a, ftab, f_lo, t0, q.c, cs);

  uint8_t* page = static_cast<uint8_t*>(a.pool) + static_cast<int64_t>(task.slot) * a.page_bytes;
  uint8_t* K8 = page;                                                      // [H][Np][D]
  uint8_t* V8 = page + static_cast<int64_t>(H) * Np * D;                   // [H][D][Np]
  uint8_t* codes = page + (kBf16V ? 3 : 2) * static_cast<int64_t>(H) * Np * D;   // [H][T][2]
  const int64_t hnd = static_cast<int64_t>(H) * N * D;
  __bf16* ancK = static_cast<__bf16*>(a.anchor_raw);                       // bf16 [H][N][D]
  __bf16* ancVt = ancK + hnd;                                              // bf16 [H][D][N]
  const bool capture = task.mode == TASK_CAPTURE;
  const bool anchor = task.mode == TASK_ANCHOR;

  for (int hb = hg0; hb < hg1; hb += q.hpp) {   // uniform over the work-group
    const int h = hb + q.slot;
    const bool act = h < hg1;
    float kr[kRows][8];                         // rotated keys (0 past N)
    bf16x8 vt[8];                               // values, dim-major: vt[e][i] = v(t0 + i, 8 c + e)
    float kmax = 0.f, vmax = 0.f;
    const int64_t krow = (static_cast<int64_t>(h) * N + t0) * D + 8 * q.c;
    const int64_t vrow = (static_cast<int64_t>(h) * D + 8 * q.c) * N + t0;
    if (act && anchor) {
#pragma unroll
      for (int i = 0; i < kRows; ++i) {
        if (t0 + i < N) {
          const bf16x8 x = *reinterpret_cast<const bf16x8*>(ancK + krow + int64_t(i) * D);
          rotate_f32<8>(x, cs[i], kr[i]);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) kr[i][e] = 0.f;   // padding: +0 codes (a rotated 0 may be -0)
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        vt[e] = bf16x8{};
        if (t0 < N) vt[e] = *reinterpret_cast<const bf16x8*>(ancVt + vrow + int64_t(e) * N);
      }
    } else if (act) {
      const __bf16* qin = static_cast<const __bf16*>(a.q);
      const __bf16* kin = static_cast<const __bf16*>(a.k);
      const __bf16* vin = static_cast<const __bf16*>(a.v);
      __bf16* qr = static_cast<__bf16*>(a.q_rot);
      const int64_t in0 = ((static_cast<int64_t>(task.stage) * N + t0) * H + h) * D + 8 * q.c;
      const int64_t in_step = static_cast<int64_t>(H) * D;
      bf16x8 xq[kRows], xk[kRows], xv[kRows];
#pragma unroll
      for (int i = 0; i < kRows; ++i) {
        xq[i] = bf16x8{};
        xk[i] = bf16x8{};
        xv[i] = bf16x8{};
        if (t0 + i < N) {
          xq[i] = *reinterpret_cast<const bf16x8*>(qin + in0 + i * in_step);
          xk[i] = *reinterpret_cast<const bf16x8*>(kin + in0 + i * in_step);
          xv[i] = *reinterpret_cast<const bf16x8*>(vin + in0 + i * in_step);
        }
      }
#pragma unroll
      for (int i = 0; i < kRows; ++i) {
        if (t0 + i < N) {
          rotate_f32<8>(xk[i], cs[i], kr[i]);
          *reinterpret_cast<bf16x8*>(qr + in0 + i * in_step) = rotate<__bf16>(xq[i], cs[i]);
          if (capture) *reinterpret_cast<bf16x8*>(ancK + krow + int64_t(i) * D) = xk[i];
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) kr[i][e] = 0.f;   // padding: +0 codes (a rotated 0 may be -0)
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int i = 0; i < kRows; ++i) vt[e][i] = xv[i][e];
    } else {
#pragma unroll
      for (int i = 0; i < kRows; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) kr[i][e] = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) vt[e] = bf16x8{};
    }
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
      // K rows (padding rows get zero codes)
#pragma unroll
      for (int i = 0; i < kRows; ++i) {
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = kr[i][e] * sk;
        *reinterpret_cast<uint2*>(K8 + (static_cast<int64_t>(h) * Np + t0 + i) * D + 8 * q.c) = fp8_pack8(x);
      }
      // Vt rows: 8 consecutive tokens of one value dim
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int64_t off = (static_cast<int64_t>(h) * D + 8 * q.c + e) * Np + t0;
        if (kBf16V) {
          *reinterpret_cast<bf16x8*>(reinterpret_cast<__bf16*>(V8) + off) = vt[e];
        } else {
          float x[8];
#pragma unroll
          for (int i = 0; i < kRows; ++i) x[i] = static_cast<float>(vt[e][i]) * sv;
          *reinterpret_cast<uint2*>(V8 + off) = fp8_pack8(x);
        }
        if (capture && t0 < N) *reinterpret_cast<bf16x8*>(ancVt + vrow + int64_t(e) * N) = vt[e];
      }
      if (q.g == 0 && q.c == 0) {
        const uint16_t code = static_cast<uint16_t>((ek + 127) | ((ev + 127) << 8));
        *reinterpret_cast<uint16_t*>(codes + (static_cast<int64_t>(h) * a.T + tile) * 2) = code;
      }
    }
    __syncthreads();                            // red is rewritten by the next pass
  }
}

// Heads per work-group: a multiple of the heads one pass covers, few enough
// groups that each work-group reuses its angles over several heads, enough
// that the grid holds about four work-groups per compute unit.
int heads_per_group(int H, int hpp, int blocks) {
  const int want_groups = (1024 + blocks - 1) / blocks;
  const int max_groups = (H + hpp - 1) / hpp;
  const int groups = want_groups < 1 ? 1 : (want_groups > max_groups ? max_groups : want_groups);
  int hpg = (H + groups - 1) / groups;
  hpg = (hpg + hpp - 1) / hpp * hpp;
  return hpg;
}

}  // namespace

hipError_t launch_publish(const PublishArgs& args, int dtype, hipStream_t stream) {
  if (args.n_tasks <= 0) return hipSuccess;
  if (args.nt > kMaxFramePairs) return hipErrorInvalidValue;
  PublishArgs a = args;
  const int vec = dtype == WF_F32 ? 4 : 8;
  const int hpp = kThreads / (kRows * (a.D / vec));
  if (hpp < 1 || a.D % vec != 0) return hipErrorInvalidValue;
  if (dtype == WF_FP8 || dtype == WF_FP8K) {
    if (a.D != kFp8D) return hipErrorInvalidValue;
    a.heads_per_group = heads_per_group(a.H, hpp, a.T * a.n_tasks);
    const dim3 grid(a.T, (a.H + a.heads_per_group - 1) / a.heads_per_group, a.n_tasks);
    if (dtype == WF_FP8) hipLaunchKernelGGL(wf_publish_fp8_kernel<false>, grid, dim3(kThreads), 0, stream, a);
    else hipLaunchKernelGGL(wf_publish_fp8_kernel<true>, grid, dim3(kThreads), 0, stream, a);
    return hipGetLastError();
  }
  const int blocks = (a.N + kTokens - 1) / kTokens;
  a.heads_per_group = heads_per_group(a.H, hpp, blocks * a.n_tasks);
  const dim3 grid(blocks, (a.H + a.heads_per_group - 1) / a.heads_per_group, a.n_tasks);
  if (dtype == WF_BF16) {
    hipLaunchKernelGGL(wf_publish_kernel<__bf16>, grid, dim3(kThreads), 0, stream, a);
  } else {
    hipLaunchKernelGGL(wf_publish_kernel<float>, grid, dim3(kThreads), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace wf
