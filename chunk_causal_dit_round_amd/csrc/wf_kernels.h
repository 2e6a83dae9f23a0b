// Kernel argument blocks and launchers shared by the host runtime and the
// HIP kernels.  Arguments travel by value in the kernarg segment; nothing is
// staged through device memory.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "wf.h"
#include "wf_plan.h"

namespace wf {

// ------------------------------------------------------------ publish ----
enum : int32_t {
  TASK_CELL = 0,     // rotate q and k of one cell, write q_rot and its page
  TASK_CAPTURE = 1,  // TASK_CELL that also keeps the raw k and v^T (anchor)
  TASK_ANCHOR = 2    // re-rotate the kept anchor key into the anchor slot
};

struct PublishTask {
  int32_t stage;   // input stage (cell) the rows come from; unused for anchor
  int32_t slot;    // destination slot in this layer's pool
  int32_t frame0;  // frame position of the chunk's first frame
  int32_t mode;    // TASK_*
};

struct PublishArgs {
  const void* q;          // this layer's [S+1][N][H][D]
  const void* k;
  const void* v;
  void* q_rot;            // this layer's [S+1][N][H][D]
  void* pool;             // this layer's [n_slots] pages
  void* anchor_raw;       // this layer's anchor page (raw K, Vt)
  const double* omega_t;  // [nt] frame-axis frequencies theta^(-m / nt)
  const float2* rope_hw;  // [Hh*nh | Ww*nw] (cos, sin) of the row and column axes
  int64_t page_elems;     // 2 H N D (fp32 / bf16 pages)
  int64_t page_bytes;     // bytes per pool page (all dtypes)
  int32_t N, H, D, F, Hh, Ww;
  int32_t nt, nh, nw;
  int32_t heads_per_group;  // set by the launcher
  int32_t frames_max;       // set by the launcher: frames a 64-token block can span
  int32_t pad0_;
  int32_t Npad, T;        // FP8 pages: tokens padded to 64 T, T tiles
  int32_t n_tasks;
  int32_t pad_;
  PublishTask task[WF_MAX_GROUPS + 1];
};

// ---------------------------------------------------------- attention ----
struct AttnGroup {
  int32_t stage;     // query rows come from q_rot[stage]
  int32_t n_pages;   // key pages in context order
  int32_t item0;     // first work item of this group
  int32_t part;      // -1: whole context, O goes to out; else the partial
                     // result slot (O unnormalised, exponent offset, l)
  uint16_t slot[WF_MAX_PAGES];
};

struct AttnArgs {
  const void* q_rot;   // [S+1][N][H][D]
  void* out;           // [S+1][N][H][D]
  const void* pool;    // this layer's [n_slots] pages
  int64_t page_elems;  // fp32 / bf16 pages
  int64_t page_bytes;  // bytes per pool page (all dtypes)
  int32_t N, H, D;
  float scale_log2e;   // softmax scale * log2(e)
  int32_t n_groups;    // active groups, longest context first
  int32_t q_tiles;     // query tiles per (group, head)
  int32_t n_items;     // sum over groups of H * q_tiles
  int32_t Npad, T;     // FP8 pages: tokens padded to 64 T, T tiles
  int32_t pad_;
  float* part_o;       // [kMaxSplit * 2][N][H][D] partial O (unnormalised)
  float* part_el;      // [kMaxSplit * 2][N][H][2] (exponent offset e, l)
  AttnGroup grp[WF_MAX_GROUPS + kMaxSplit];
};

// A split group's two halves (pages [0, n/2) and [n/2, n)) run as separate
// work items that leave partial results; the combine kernel merges them:
// with M = max(e_a, e_b), w = 2^(e - M), O = (O_a w_a + O_b w_b) / (l_a w_a + l_b w_b).
struct CombineArgs {
  const float* part_o;
  const float* part_el;
  void* out;           // [S+1][N][H][D] bf16
  int32_t N, H, D;
  int32_t n_split;
  int32_t stage[kMaxSplit];
};

// Query rows per work item of each attention instance.
constexpr int kAttnBM_bf16 = 256;
constexpr int kAttnBM_fp8 = 256;
constexpr int kAttnBM_fp8k = 256;
constexpr int kAttnBM_f32 = 64;
// FP8 / FP8K attention keeps the scale codes of a group's whole context in LDS.
constexpr int kFp8MaxCtxTiles = 4096;

// The publish kernels stage a 64-token block's rotation angles in LDS: the
// frame axis's cos/sin at the frames the block spans, then the row and
// column tables.  Bytes of that table, and the most allowed.
size_t publish_lds_bytes(int F, int Hh, int Ww, int nt, int nh, int nw);
constexpr size_t kPublishMaxLds = 60 * 1024;

hipError_t launch_publish(const PublishArgs& a, int dtype, hipStream_t stream);
hipError_t launch_attention(const AttnArgs& a, int dtype, hipStream_t stream);
hipError_t launch_attention_fp8(const AttnArgs& a, hipStream_t stream);
hipError_t launch_attention_fp8k(const AttnArgs& a, hipStream_t stream);
hipError_t launch_combine(const CombineArgs& a, hipStream_t stream);

}  // namespace wf
