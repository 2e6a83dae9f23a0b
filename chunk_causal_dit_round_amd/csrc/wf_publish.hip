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

}  // namespace

hipError_t launch_publish(const PublishArgs& a, int dtype, hipStream_t stream) {
  if (a.n_tasks <= 0) return hipSuccess;
  const dim3 grid((a.N + kTokens - 1) / kTokens, a.H, a.n_tasks);
  if (dtype == WF_BF16) {
    hipLaunchKernelGGL(wf_publish_kernel<__bf16>, grid, dim3(kThreads), 0, stream, a);
  } else {
    hipLaunchKernelGGL(wf_publish_kernel<float>, grid, dim3(kThreads), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace wf
