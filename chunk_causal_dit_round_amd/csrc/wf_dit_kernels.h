// Kernel argument blocks of the DiT block's row-wise kernels (LayerNorm with
// modulation and gated residuals; RMSNorm of q and k).  One wave per token
// row; every row is C channels with C % 8 == 0 and C <= 8192.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace wf {

// Row r of this launch is token r % N of the cell at stage s_lo + r / N.
struct NormArgs {
  float* x;            // [rows][C] fp32 residual stream (first row of the launch)
  const float* y;      // [rows][C] fp32 branch output added as x += gate * y; NULL: none
  const float* mod;    // this layer's [S+1][6][C]
  void* h;             // [rows][C] bf16 modulated LN output; NULL: none
  int32_t rows, C, N, s_lo;
  int32_t gate;        // modulation row of the gate applied to y (2 or 5)
  int32_t ln;          // 0: shift1/scale1, 1: shift2/scale2, -1: no LN output
  float eps;
  int32_t pad_;
};

struct QkNormArgs {
  const void* qkv;     // [rows][3C] bf16: q, k, v channels of each token
  const float* g_q;    // [C]
  const float* g_k;    // [C]
  void* q;             // [rows][C] bf16 outputs
  void* k;
  void* v;
  int32_t rows, C;
  float eps;
  int32_t pad_;
};

constexpr int kDitMaxC = 8192;

hipError_t launch_norm(const NormArgs& a, hipStream_t stream);
hipError_t launch_qk_norm(const QkNormArgs& a, hipStream_t stream);

}  // namespace wf
