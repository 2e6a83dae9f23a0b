// Partial results of a split group (AttnGroup::part >= 0), shared by the
// attention kernels.  The two halves of a split group attend to disjoint page
// ranges of the same context; each leaves its unnormalised O, its exponent
// offset e (every weight it summed is 2^(S - e), S the base-2 score) and its
// weight sum l, and the combine kernel merges the two softmax partials
// exactly (up to fp32 rounding).
#pragma once

#include <hip/hip_runtime.h>

#include "wf_kernels.h"

namespace wf {

// Lane (col, half) of the O^T accumulators holds dims 32 dt + 8 i4 + 4 half
// + j (j = 0..3) of query q, the layout all the attention kernels share.
template <class Acc, int DT>
__device__ inline void store_partial(const AttnArgs& a, int part, int q, int h, float e, float l,
                                     const Acc (&oacc)[DT], int half) {
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  const int64_t row = (static_cast<int64_t>(part) * a.N + q) * a.H + h;
  float* o = a.part_o + row * a.D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      f32x4 v;
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = oacc[dt][4 * i4 + j];
      *reinterpret_cast<f32x4*>(o + 32 * dt + 8 * i4 + 4 * half) = v;
    }
  if (half == 0) {
    float2 el;
    el.x = e;
    el.y = l;
    reinterpret_cast<float2*>(a.part_el)[row] = el;
  }
}

}  // namespace wf
