// Row-wise kernels of the Wan-shaped DiT block around the round (the block is
// written out in include/wf_dit.h).  Both are HBM-bound: one wave per token
// row keeps the row in registers, so every byte is read and written once.
//
//   wf_norm_kernel     optional gated residual x += gate * y (fp32), then
//                      optional LayerNorm (no affine) modulated by the cell's
//                      shift / scale, stored bf16 for the next product
//   wf_qk_norm_kernel  splits the QKV product into q, k, v and applies the
//                      RMSNorm gains to q and k (over all C channels)
#include "wf_dit_kernels.h"

namespace wf {
namespace {

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// VPL float4 per lane: channels 4 (64 j + lane) .. +3 for j < VPL.
template <int VPL>
__global__ __launch_bounds__(256) void wf_norm_kernel(NormArgs a) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.rows) return;
  const int C = a.C;
  const float* md = a.mod + static_cast<int64_t>(a.s_lo + row / a.N) * 6 * C;
  float* xr = a.x + static_cast<int64_t>(row) * C;
  float4 v[VPL];
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const int c = 4 * (j * 64 + lane);
    v[j] = c < C ? *reinterpret_cast<const float4*>(xr + c) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  if (a.y != nullptr) {
    const float* yr = a.y + static_cast<int64_t>(row) * C;
    const float* g = md + a.gate * C;
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      const int c = 4 * (j * 64 + lane);
      if (c < C) {
        const float4 y = *reinterpret_cast<const float4*>(yr + c);
        const float4 w = *reinterpret_cast<const float4*>(g + c);
        v[j].x = __builtin_fmaf(w.x, y.x, v[j].x);
        v[j].y = __builtin_fmaf(w.y, y.y, v[j].y);
        v[j].z = __builtin_fmaf(w.z, y.z, v[j].z);
        v[j].w = __builtin_fmaf(w.w, y.w, v[j].w);
        *reinterpret_cast<float4*>(xr + c) = v[j];
      }
    }
  }
  if (a.ln < 0) return;
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < VPL; ++j) s += (v[j].x + v[j].y) + (v[j].z + v[j].w);
  const float mean = wave_sum(s) / static_cast<float>(C);
  float q = 0.f;
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    if (4 * (j * 64 + lane) < C) {
      const float dx = v[j].x - mean, dy = v[j].y - mean, dz = v[j].z - mean, dw = v[j].w - mean;
      q += (dx * dx + dy * dy) + (dz * dz + dw * dw);
    }
  }
  const float rstd = 1.f / sqrtf(wave_sum(q) / static_cast<float>(C) + a.eps);
  const float* sh = md + (3 * a.ln) * C;
  const float* sc = sh + C;
  __bf16* hr = static_cast<__bf16*>(a.h) + static_cast<int64_t>(row) * C;
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const int c = 4 * (j * 64 + lane);
    if (c < C) {
      const float4 b = *reinterpret_cast<const float4*>(sh + c);
      const float4 m = *reinterpret_cast<const float4*>(sc + c);
      bf16x4 o;
      o[0] = static_cast<__bf16>(__builtin_fmaf((v[j].x - mean) * rstd, 1.f + m.x, b.x));
      o[1] = static_cast<__bf16>(__builtin_fmaf((v[j].y - mean) * rstd, 1.f + m.y, b.y));
      o[2] = static_cast<__bf16>(__builtin_fmaf((v[j].z - mean) * rstd, 1.f + m.z, b.z));
      o[3] = static_cast<__bf16>(__builtin_fmaf((v[j].w - mean) * rstd, 1.f + m.w, b.w));
      *reinterpret_cast<bf16x4*>(hr + c) = o;
    }
  }
}

// VPL8 groups of 8 bf16 per lane: channels 8 (64 j + lane) .. +7 for j < VPL8.
template <int VPL8>
__global__ __launch_bounds__(256) void wf_qk_norm_kernel(QkNormArgs a) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.rows) return;
  const int C = a.C;
  const __bf16* src = static_cast<const __bf16*>(a.qkv) + static_cast<int64_t>(row) * 3 * C;
#pragma unroll
  for (int part = 0; part < 2; ++part) {
    const __bf16* in = src + part * C;
    bf16x8 x[VPL8];
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < VPL8; ++j) {
      const int c = 8 * (j * 64 + lane);
      x[j] = c < C ? *reinterpret_cast<const bf16x8*>(in + c) : bf16x8{};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float f = static_cast<float>(x[j][e]);
        ss = __builtin_fmaf(f, f, ss);
      }
    }
    const float r = 1.f / sqrtf(wave_sum(ss) / static_cast<float>(C) + a.eps);
    const float* g = part == 0 ? a.g_q : a.g_k;
    __bf16* out = static_cast<__bf16*>(part == 0 ? a.q : a.k) + static_cast<int64_t>(row) * C;
#pragma unroll
    for (int j = 0; j < VPL8; ++j) {
      const int c = 8 * (j * 64 + lane);
      if (c < C) {
        const float4 g0 = *reinterpret_cast<const float4*>(g + c);
        const float4 g1 = *reinterpret_cast<const float4*>(g + c + 4);
        const float gg[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
        bf16x8 o;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = static_cast<__bf16>(static_cast<float>(x[j][e]) * r * gg[e]);
        *reinterpret_cast<bf16x8*>(out + c) = o;
      }
    }
  }
  const __bf16* vin = src + 2 * C;
  __bf16* vout = static_cast<__bf16*>(a.v) + static_cast<int64_t>(row) * C;
#pragma unroll
  for (int j = 0; j < VPL8; ++j) {
    const int c = 8 * (j * 64 + lane);
    if (c < C) *reinterpret_cast<bf16x8*>(vout + c) = *reinterpret_cast<const bf16x8*>(vin + c);
  }
}

template <int V>
hipError_t norm_with(const NormArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(wf_norm_kernel<V>, dim3((a.rows + 3) / 4), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <int V>
hipError_t qk_with(const QkNormArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(wf_qk_norm_kernel<V>, dim3((a.rows + 3) / 4), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_norm(const NormArgs& a, hipStream_t stream) {
  if (a.rows <= 0) return hipSuccess;
  if (a.C <= 0 || a.C % 8 != 0 || a.C > kDitMaxC) return hipErrorInvalidValue;
  const int need = (a.C + 255) / 256;
  if (need <= 1) return norm_with<1>(a, stream);
  if (need <= 2) return norm_with<2>(a, stream);
  if (need <= 3) return norm_with<3>(a, stream);
  if (need <= 4) return norm_with<4>(a, stream);
  if (need <= 6) return norm_with<6>(a, stream);
  if (need <= 8) return norm_with<8>(a, stream);
  if (need <= 12) return norm_with<12>(a, stream);
  if (need <= 16) return norm_with<16>(a, stream);
  if (need <= 20) return norm_with<20>(a, stream);
  if (need <= 24) return norm_with<24>(a, stream);
  return norm_with<32>(a, stream);
}

hipError_t launch_qk_norm(const QkNormArgs& a, hipStream_t stream) {
  if (a.rows <= 0) return hipSuccess;
  if (a.C <= 0 || a.C % 8 != 0 || a.C > kDitMaxC) return hipErrorInvalidValue;
  const int need = (a.C + 511) / 512;
  if (need <= 1) return qk_with<1>(a, stream);
  if (need <= 2) return qk_with<2>(a, stream);
  if (need <= 3) return qk_with<3>(a, stream);
  if (need <= 4) return qk_with<4>(a, stream);
  if (need <= 6) return qk_with<6>(a, stream);
  if (need <= 8) return qk_with<8>(a, stream);
  if (need <= 10) return qk_with<10>(a, stream);
  if (need <= 12) return qk_with<12>(a, stream);
  return qk_with<16>(a, stream);
}

}  // namespace wf
