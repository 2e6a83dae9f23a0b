// Fused 3D-RoPE + paged K/V publish for one layer of one round.
//
// Producer step P_{s,l} of "Wave Forcing: Towards Speed-of-Light Streaming
// Video Generation" (§4.1 Eq. 8: Q/K/V then RoPE) followed by the paged
// write of App. B.2 (Eq. 13): each chunk's K/V goes straight into its fixed
// attention slot, so attention reads the ordered context with no gather.
// App. B.3: chunk 0's unrotated key is kept so RoPE can be re-applied when
// the window shifts (TASK_CAPTURE / TASK_ANCHOR).
//
// Grid: (token blocks of 64, heads, tasks).  One work-group moves one
// 64-token x D block of one head: 16-byte global loads and stores, RoPE in
// fp32 from fp32 cos/sin tables, V transposed through LDS so the page's Vt
// rows (keys contiguous) are written with full 16-byte stores.
// HBM-bound: every byte is read once and written once.
#include <hip/hip_runtime.h>

#include "wf_kernels.h"

namespace wf {
namespace {

constexpr int kTokens = 64;    // tokens per work-group
constexpr int kThreads = 256;
constexpr int kMaxD = 128;

template <typename T>
struct Vec;
template <>
struct Vec<float> {
  static constexpr int n = 4;
  typedef float raw __attribute__((ext_vector_type(4)));
  __device__ static float get(const raw& r, int e) { return r[e]; }
  __device__ static void set(raw& r, int e, float x) { r[e] = x; }
};
template <>
struct Vec<__bf16> {
  static constexpr int n = 8;
  typedef __bf16 raw __attribute__((ext_vector_type(8)));
  __device__ static float get(const raw& r, int e) { return static_cast<float>(r[e]); }
  __device__ static void set(raw& r, int e, float x) { r[e] = static_cast<__bf16>(x); }
};

// Rotates the VEC elements starting at element d0 of one token row.
template <typename T>
__device__ inline typename Vec<T>::raw rope_chunk(const typename Vec<T>::raw& x, int d0,
                                                  int frame, int y, int xcol,
                                                  const PublishArgs& a) {
  using V = Vec<T>;
  typename V::raw out;
  const float2* tf = a.rope;
  const float2* th = tf + static_cast<int64_t>(a.n_frames) * a.nt;
  const float2* tw = th + a.Hh * a.nh;
#pragma unroll
  for (int e = 0; e < V::n; e += 2) {
    const int p = (d0 + e) >> 1;
    float2 cs;
    if (p < a.nt) {
      cs = tf[static_cast<int64_t>(frame) * a.nt + p];
    } else if (p < a.nt + a.nh) {
      cs = th[y * a.nh + (p - a.nt)];
    } else {
      cs = tw[xcol * a.nw + (p - a.nt - a.nh)];
    }
    const float x0 = V::get(x, e), x1 = V::get(x, e + 1);
    V::set(out, e, x0 * cs.x - x1 * cs.y);
    V::set(out, e + 1, x0 * cs.y + x1 * cs.x);
  }
  return out;
}

template <typename T>
__global__ __launch_bounds__(kThreads) void wf_publish_kernel(const PublishArgs a) {
  using V = Vec<T>;
  using raw = typename V::raw;
  constexpr int VEC = V::n;
  // V block staged for the transpose; the +2 element pad spreads rows over
  // LDS banks when a column is gathered.
  __shared__ T vtile[kTokens][kMaxD + 2];

  const PublishTask task = a.task[blockIdx.z];
  const int h = blockIdx.y;
  const int tok0 = blockIdx.x * kTokens;
  const int N = a.N, H = a.H, D = a.D;
  const int cpr = D / VEC;                       // 16-byte chunks per row
  const int64_t hnd = static_cast<int64_t>(H) * N * D;
  T* page = static_cast<T*>(a.pool) + static_cast<int64_t>(task.slot) * a.page_elems;
  T* pageK = page;                               // [H][N][D]
  T* pageVt = page + hnd;                        // [H][D][N]
  T* anc = static_cast<T*>(a.anchor_raw);
  T* ancK = anc;
  T* ancVt = anc + hnd;
  const int hw = a.Hh * a.Ww;

  if (task.mode == TASK_ANCHOR) {
    // Key: re-rotate the kept raw key at the anchor's current position.
    for (int idx = threadIdx.x; idx < kTokens * cpr; idx += kThreads) {
      const int r = idx / cpr, c = idx - r * cpr;
      const int tok = tok0 + r;
      if (tok >= N) continue;
      const int64_t off = (static_cast<int64_t>(h) * N + tok) * D + c * VEC;
      const raw x = *reinterpret_cast<const raw*>(ancK + off);
      const int f = tok / hw, y = (tok / a.Ww) % a.Hh, xc = tok % a.Ww;
      *reinterpret_cast<raw*>(pageK + off) = rope_chunk<T>(x, c * VEC, task.frame0 + f, y, xc, a);
    }
    // Value: copied unchanged (Vt rows of this token block).
    const int gpr = kTokens / VEC;
    for (int idx = threadIdx.x; idx < D * gpr; idx += kThreads) {
      const int d = idx / gpr, g = idx - d * gpr;
      const int tok = tok0 + g * VEC;
      if (tok >= N) continue;
      const int64_t off = (static_cast<int64_t>(h) * D + d) * N + tok;
      *reinterpret_cast<raw*>(pageVt + off) = *reinterpret_cast<const raw*>(ancVt + off);
    }
    return;
  }

  const bool capture = task.mode == TASK_CAPTURE;
  const T* q = static_cast<const T*>(a.q);
  const T* k = static_cast<const T*>(a.k);
  const T* v = static_cast<const T*>(a.v);
  T* qr = static_cast<T*>(a.q_rot);
  const int64_t stage_base = static_cast<int64_t>(task.stage) * N;

  for (int idx = threadIdx.x; idx < kTokens * cpr; idx += kThreads) {
    const int r = idx / cpr, c = idx - r * cpr;
    const int tok = tok0 + r;
    if (tok >= N) continue;
    const int64_t in = ((stage_base + tok) * H + h) * D + c * VEC;
    const int f = tok / hw, y = (tok / a.Ww) % a.Hh, xc = tok % a.Ww;
    const int frame = task.frame0 + f;
    const raw xq = *reinterpret_cast<const raw*>(q + in);
    const raw xk = *reinterpret_cast<const raw*>(k + in);
    const raw xv = *reinterpret_cast<const raw*>(v + in);
    *reinterpret_cast<raw*>(qr + in) = rope_chunk<T>(xq, c * VEC, frame, y, xc, a);
    const int64_t kofs = (static_cast<int64_t>(h) * N + tok) * D + c * VEC;
    *reinterpret_cast<raw*>(pageK + kofs) = rope_chunk<T>(xk, c * VEC, frame, y, xc, a);
    if (capture) *reinterpret_cast<raw*>(ancK + kofs) = xk;
#pragma unroll
    for (int e = 0; e < VEC; ++e) vtile[r][c * VEC + e] = static_cast<T>(V::get(xv, e));
  }
  __syncthreads();
  // Transposed write: VEC consecutive tokens of one value dimension.
  const int gpr = kTokens / VEC;
  for (int idx = threadIdx.x; idx < D * gpr; idx += kThreads) {
    const int d = idx / gpr, g = idx - d * gpr;
    const int tok = tok0 + g * VEC;
    if (tok >= N) continue;
    raw o;
#pragma unroll
    for (int e = 0; e < VEC; ++e) V::set(o, e, static_cast<float>(vtile[g * VEC + e][d]));
    const int64_t off = (static_cast<int64_t>(h) * D + d) * N + tok;
    *reinterpret_cast<raw*>(pageVt + off) = o;
    if (capture) *reinterpret_cast<raw*>(ancVt + off) = o;
  }
}

// ---------------------------------------------------------------- FP8 ----
// FP8 pages ("Wave Forcing" App. C.6: 8-bit K/V halve the payload).  One
// work-group quantises one 64-token tile of one head: rotated K and V each
// get one power-of-two scale 2^e with e the smallest integer such that
// amax(tile) <= 448 * 2^e, and are stored as OCP E4M3 codes of x / 2^e
// (round to nearest even).  q_rot stays bf16.  Tokens N..Npad-1 are zero.
// With kBf16V (the 8-bit QK^T tier) only K is quantised; Vt is written in
// bf16 (its scale code stays 2^0).
constexpr int kFp8D = 128;
constexpr int kFp8Items = kTokens * (kFp8D / 8) / kThreads;   // (row, 8-dim chunk) per thread

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// RoPE of 8 consecutive elements starting at d0 (even), fp32 result.
__device__ inline void rope8_f32(const bf16x8& x, int d0, int frame, int y, int xcol,
                                 const PublishArgs& a, float out[8]) {
  const float2* tf = a.rope;
  const float2* th = tf + static_cast<int64_t>(a.n_frames) * a.nt;
  const float2* tw = th + a.Hh * a.nh;
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    const int p = (d0 + e) >> 1;
    float2 cs;
    if (p < a.nt) {
      cs = tf[static_cast<int64_t>(frame) * a.nt + p];
    } else if (p < a.nt + a.nh) {
      cs = th[y * a.nh + (p - a.nt)];
    } else {
      cs = tw[xcol * a.nw + (p - a.nt - a.nh)];
    }
    const float x0 = static_cast<float>(x[e]), x1 = static_cast<float>(x[e + 1]);
    out[e] = x0 * cs.x - x1 * cs.y;
    out[e + 1] = x0 * cs.y + x1 * cs.x;
  }
}

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
__device__ inline uint2 fp8_pack8(const float v[8]) {
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
  // V tile staged token-major in fp32 for the amax and the transposed write.
  __shared__ float vtile[kTokens][kFp8D + 1];
  __shared__ float red[2][kThreads / 64];

  const PublishTask task = a.task[blockIdx.z];
  const int h = blockIdx.y;
  const int tile = blockIdx.x;
  const int tok0 = tile * kTokens;
  const int N = a.N, H = a.H, Np = a.Npad;
  constexpr int D = kFp8D;
  const int tid = threadIdx.x;
  uint8_t* page = static_cast<uint8_t*>(a.pool) + static_cast<int64_t>(task.slot) * a.page_bytes;
  uint8_t* K8 = page;                                             // [H][Np][D]
  uint8_t* V8 = page + static_cast<int64_t>(H) * Np * D;          // [H][D][Np] (bf16 with kBf16V)
  uint8_t* codes = page + (kBf16V ? 3 : 2) * static_cast<int64_t>(H) * Np * D;   // [H][T][2]
  const int64_t hnd = static_cast<int64_t>(H) * N * D;
  __bf16* ancK = static_cast<__bf16*>(a.anchor_raw);              // bf16 [H][N][D]
  __bf16* ancVt = ancK + hnd;                                     // bf16 [H][D][N]
  const int hw = a.Hh * a.Ww;

  float kr[kFp8Items][8];
  float kmax = 0.f, vmax = 0.f;
  if (task.mode == TASK_ANCHOR) {
    // anchor: re-rotate the kept raw key; the kept Vt is re-quantised
#pragma unroll
    for (int i = 0; i < kFp8Items; ++i) {
      const int idx = tid + i * kThreads, r = idx >> 4, c = idx & 15;
      const int tok = tok0 + r;
#pragma unroll
      for (int e = 0; e < 8; ++e) kr[i][e] = 0.f;
      if (tok < N) {
        const bf16x8 x = *reinterpret_cast<const bf16x8*>(ancK + (static_cast<int64_t>(h) * N + tok) * D + 8 * c);
        const int f = tok / hw, y = (tok / a.Ww) % a.Hh, xc = tok % a.Ww;
        rope8_f32(x, 8 * c, task.frame0 + f, y, xc, a, kr[i]);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) kmax = fmaxf(kmax, fabsf(kr[i][e]));
    }
#pragma unroll
    for (int i = 0; i < kFp8Items; ++i) {
      const int idx = tid + i * kThreads, d = idx >> 3, g = idx & 7;
      const int tok = tok0 + 8 * g;     // N % 8 == 0: a group is all real or all padding
      bf16x8 x = {};
      if (tok < N) x = *reinterpret_cast<const bf16x8*>(ancVt + (static_cast<int64_t>(h) * D + d) * N + tok);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = static_cast<float>(x[e]);
        vtile[8 * g + e][d] = v;
        vmax = fmaxf(vmax, fabsf(v));
      }
    }
  } else {
    const bool capture = task.mode == TASK_CAPTURE;
    const __bf16* q = static_cast<const __bf16*>(a.q);
    const __bf16* k = static_cast<const __bf16*>(a.k);
    const __bf16* v = static_cast<const __bf16*>(a.v);
    __bf16* qr = static_cast<__bf16*>(a.q_rot);
    const int64_t stage_base = static_cast<int64_t>(task.stage) * N;
#pragma unroll
    for (int i = 0; i < kFp8Items; ++i) {
      const int idx = tid + i * kThreads, r = idx >> 4, c = idx & 15;
      const int tok = tok0 + r;
#pragma unroll
      for (int e = 0; e < 8; ++e) kr[i][e] = 0.f;
      bf16x8 xv = {};
      if (tok < N) {
        const int64_t in = ((stage_base + tok) * H + h) * D + 8 * c;
        const int f = tok / hw, y = (tok / a.Ww) % a.Hh, xc = tok % a.Ww;
        const int frame = task.frame0 + f;
        const bf16x8 xq = *reinterpret_cast<const bf16x8*>(q + in);
        const bf16x8 xk = *reinterpret_cast<const bf16x8*>(k + in);
        xv = *reinterpret_cast<const bf16x8*>(v + in);
        float qv[8];
        rope8_f32(xq, 8 * c, frame, y, xc, a, qv);
        bf16x8 qo;
#pragma unroll
        for (int e = 0; e < 8; ++e) qo[e] = static_cast<__bf16>(qv[e]);
        *reinterpret_cast<bf16x8*>(qr + in) = qo;
        rope8_f32(xk, 8 * c, frame, y, xc, a, kr[i]);
        if (capture) *reinterpret_cast<bf16x8*>(ancK + (static_cast<int64_t>(h) * N + tok) * D + 8 * c) = xk;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        kmax = fmaxf(kmax, fabsf(kr[i][e]));
        const float vf = static_cast<float>(xv[e]);
        vtile[r][8 * c + e] = vf;
        vmax = fmaxf(vmax, fabsf(vf));
      }
    }
  }
  // tile amax of K and V over the work-group
  kmax = wave_max(kmax);
  vmax = wave_max(vmax);
  if ((tid & 63) == 0) {
    red[0][tid >> 6] = kmax;
    red[1][tid >> 6] = vmax;
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) {
    kmax = fmaxf(kmax, red[0][w]);
    vmax = fmaxf(vmax, red[1][w]);
  }
  const int ek = fp8_exponent(kmax), ev = kBf16V ? 0 : fp8_exponent(vmax);
  const float sk = ldexpf(1.f, -ek), sv = ldexpf(1.f, -ev);

  // K rows: 8 codes per (row, chunk); padding rows are zero codes
#pragma unroll
  for (int i = 0; i < kFp8Items; ++i) {
    const int idx = tid + i * kThreads, r = idx >> 4, c = idx & 15;
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = kr[i][e] * sk;
    *reinterpret_cast<uint2*>(K8 + (static_cast<int64_t>(h) * Np + tok0 + r) * D + 8 * c) = fp8_pack8(x);
  }
  // Vt rows: 8 consecutive tokens of one value dimension
#pragma unroll
  for (int i = 0; i < kFp8Items; ++i) {
    const int idx = tid + i * kThreads, d = idx >> 3, g = idx & 7;
    if (kBf16V) {
      bf16x8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = static_cast<__bf16>(vtile[8 * g + e][d]);
      *reinterpret_cast<bf16x8*>(reinterpret_cast<__bf16*>(V8) + (static_cast<int64_t>(h) * D + d) * Np + tok0 + 8 * g) = o;
    } else {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = vtile[8 * g + e][d] * sv;
      const uint2 o = fp8_pack8(x);
      *reinterpret_cast<uint2*>(V8 + (static_cast<int64_t>(h) * D + d) * Np + tok0 + 8 * g) = o;
    }
    if (task.mode == TASK_CAPTURE && tok0 + 8 * g < N) {
      bf16x8 raw;
#pragma unroll
      for (int e = 0; e < 8; ++e) raw[e] = static_cast<__bf16>(vtile[8 * g + e][d]);
      *reinterpret_cast<bf16x8*>(ancVt + (static_cast<int64_t>(h) * D + d) * N + tok0 + 8 * g) = raw;
    }
  }
  if (tid == 0) {
    const uint16_t code = static_cast<uint16_t>((ek + 127) | ((ev + 127) << 8));
    *reinterpret_cast<uint16_t*>(codes + (static_cast<int64_t>(h) * a.T + tile) * 2) = code;
  }
}

}  // namespace

hipError_t launch_publish(const PublishArgs& a, int dtype, hipStream_t stream) {
  if (a.n_tasks <= 0) return hipSuccess;
  if (dtype == WF_FP8 || dtype == WF_FP8K) {
    const dim3 grid(a.T, a.H, a.n_tasks);
    if (dtype == WF_FP8) hipLaunchKernelGGL(wf_publish_fp8_kernel<false>, grid, dim3(kThreads), 0, stream, a);
    else hipLaunchKernelGGL(wf_publish_fp8_kernel<true>, grid, dim3(kThreads), 0, stream, a);
    return hipGetLastError();
  }
  const dim3 grid((a.N + kTokens - 1) / kTokens, a.H, a.n_tasks);
  if (dtype == WF_BF16) {
    hipLaunchKernelGGL(wf_publish_kernel<__bf16>, grid, dim3(kThreads), 0, stream, a);
  } else {
    hipLaunchKernelGGL(wf_publish_kernel<float>, grid, dim3(kThreads), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace wf
