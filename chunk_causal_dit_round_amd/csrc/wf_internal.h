// Host-side internals shared by the C ABI entry points (wf_runtime.cpp for
// the round, wf_dit.cpp for the DiT block around it).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <map>
#include <string>
#include <vector>

#include "wf.h"
#include "wf_plan.h"

namespace wf {
struct DitState;  // hipBLASLt handle and product plans, created on first use
// A split query group: its context runs as pages [0, at) and [at, n).
struct SplitAt {
  int stage, at;
};
}

struct wf_handle {
  wf_config cfg;
  wf::Shape sh;
  uint64_t hash = 0;
  int64_t next_k = 0;
  void* pool = nullptr;
  void* anchor = nullptr;
  void* tables = nullptr;
  bool bound = false;
  std::vector<uint8_t> published;  // per layer, current round
  wf::DitState* dit = nullptr;
  // Attention work split (wf_set_attention_split): compute units of the bound
  // device, the mode, and the split chosen per list of group page counts.
  int n_cu = 256;
  int split_mode = WF_SPLIT_AUTO;
  std::map<std::vector<int>, std::vector<wf::SplitAt>> split_cache;
};

namespace wf {

// Frees the DiT state of a handle (no-op if none was created).
void dit_release(wf_handle* h);

namespace rt {

wf_status fail(wf_status s, const std::string& why);
wf_status ok();
bool aligned16(const void* p);
// The caller's plan checked against the handle; `fresh` receives the rebuilt plan.
wf_status check_plan(const wf_handle* h, const wf_plan* p, wf_plan* fresh);
wf_status check_layer_call(const wf_handle* h, int32_t layer);
wf_status do_publish(wf_handle* h, const wf_plan& p, int layer, const void* q, const void* k,
                     const void* v, void* q_rot, hipStream_t stream);
// Split groups leave their partial results in `scratch` (capacity
// `scratch_cap` bytes), by default the split scratch of the handle's table
// buffer; WF_ESMALL before any launch when the split chosen needs more.
wf_status do_attention(wf_handle* h, const wf_plan& p, int layer, const void* q_rot, void* out,
                       hipStream_t stream, char* scratch = nullptr, size_t scratch_cap = 0);

}  // namespace rt
}  // namespace wf
