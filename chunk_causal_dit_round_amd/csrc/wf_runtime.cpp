// Host runtime behind include/wf.h: handle state, validation, RoPE tables,
// kernel launches on the caller's stream.  Every check runs before any
// device work; the library never allocates device memory and never
// synchronises a stream (wf_bind's table upload is the one blocking copy).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <functional>
#include <mutex>
#include <queue>
#include <string>
#include <vector>

#include "wf.h"
#include "wf_internal.h"
#include "wf_kernels.h"
#include "wf_plan.h"

namespace {

thread_local std::string g_last_error;

}  // namespace

namespace wf {
namespace rt {

wf_status fail(wf_status s, const std::string& why) {
  g_last_error = why;
  return s;
}

wf_status ok() { return WF_OK; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Kernel support for a valid config (checked at bind time so that plans of
// any valid config can be built without a device).
wf_status check_supported(const wf::Shape& sh) {
  if (wf::publish_lds_bytes(sh.F, sh.Hh, sh.Ww, sh.nt, sh.nh, sh.nw) > wf::kPublishMaxLds)
    return fail(WF_EUNSUPPORTED, "publish: the RoPE tables of a 64-token block (frames, rows, columns) exceed its LDS");
  // The publish kernels address one layer's slots, inputs and anchor store
  // with 32-bit byte offsets.
  if (double(sh.n_slots) * double(sh.page_bytes) >= 4294967296.0)
    return fail(WF_EUNSUPPORTED, "one layer's slot pool must stay below 4 GiB");
  if (sh.dtype == WF_BF16) {
    if (sh.D != 64 && sh.D != 128)
      return fail(WF_EUNSUPPORTED, "bf16 kernels need head_dim 64 or 128");
    if (sh.N % 8 != 0) return fail(WF_EUNSUPPORTED, "bf16 kernels need tokens per chunk % 8 == 0");
    // A 64-key tile then straddles at most one page boundary.
    if (sh.N < 64) return fail(WF_EUNSUPPORTED, "bf16 kernels need tokens per chunk >= 64");
    // Attention addresses a layer's slots with 32-bit byte offsets.
    if (double(sh.n_slots) * double(sh.page_elems) * 2.0 >= 4294967296.0)
      return fail(WF_EUNSUPPORTED, "bf16 kernels need one layer's slot pool below 4 GiB");
  } else if (sh.dtype == WF_FP8 || sh.dtype == WF_FP8K) {
    const char* name = sh.dtype == WF_FP8 ? "FP8" : "FP8K";
    if (sh.D != 128) return fail(WF_EUNSUPPORTED, std::string(name) + " kernels need head_dim 128");
    if (sh.N % 8 != 0) return fail(WF_EUNSUPPORTED, std::string(name) + " kernels need tokens per chunk % 8 == 0");
    if (double(sh.n_slots) * double(sh.page_bytes) >= 4294967296.0)
      return fail(WF_EUNSUPPORTED, std::string(name) + " kernels need one layer's slot pool below 4 GiB");
    const int worst = 1 + sh.Wmax + 1 + sh.S;
    if (worst * sh.T > wf::kFp8MaxCtxTiles)
      return fail(WF_EUNSUPPORTED,
                  std::string(name) + " attention needs (longest context pages) * ceil(N/64) <= 4096");
  } else {
    if (sh.D % 4 != 0 || sh.D > 128)
      return fail(WF_EUNSUPPORTED, "fp32 kernels need head_dim % 4 == 0 and <= 128");
    if (sh.N % 4 != 0) return fail(WF_EUNSUPPORTED, "fp32 kernels need tokens per chunk % 4 == 0");
  }
  return ok();
}

// Plan of the caller, checked against the handle: made for this config,
// for the round the handle expects, and unmodified.
wf_status check_plan(const wf_handle* h, const wf_plan* p, wf_plan* fresh) {
  if (!h || !p) return fail(WF_EINVAL, "handle or plan is NULL");
  if (p->config_hash != h->hash) return fail(WF_EORDER, "plan was made for another config");
  if (p->k != h->next_k) {
    return fail(WF_EORDER, "plan is for round " + std::to_string(p->k) + " but the handle expects round " +
                               std::to_string(h->next_k));
  }
  wf::build_plan(h->sh, h->hash, p->k, fresh);
  if (std::memcmp(fresh, p, sizeof(wf_plan)) != 0) return fail(WF_EINVAL, "plan contents were modified");
  return ok();
}

size_t stage_bytes(const wf::Shape& sh) {
  return size_t(sh.S + 1) * size_t(sh.N) * size_t(sh.H) * size_t(sh.D) * sh.elem;
}

char* layer_ptr(void* base, size_t per_layer, int layer) {
  return static_cast<char*>(base) + per_layer * size_t(layer);
}

wf_status do_publish(wf_handle* h, const wf_plan& p, int layer, const void* q, const void* k,
                     const void* v, void* q_rot, hipStream_t stream) {
  const wf::Shape& sh = h->sh;
  wf::PublishArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.q_rot = q_rot;
  a.pool = layer_ptr(h->pool, size_t(sh.n_slots) * sh.page_bytes, layer);
  a.anchor_raw = layer_ptr(h->anchor, sh.anchor_page_bytes, layer);
  a.omega_t = static_cast<const double*>(h->tables);
  a.rope_hw = reinterpret_cast<const float2*>(static_cast<const char*>(h->tables) + wf::rope_hw_offset(sh));
  a.page_elems = static_cast<int64_t>(sh.page_elems);
  a.page_bytes = static_cast<int64_t>(sh.page_bytes);
  a.Npad = sh.Npad;
  a.T = sh.T;
  a.N = sh.N;
  a.H = sh.H;
  a.D = sh.D;
  a.F = sh.F;
  a.Hh = sh.Hh;
  a.Ww = sh.Ww;
  a.nt = sh.nt;
  a.nh = sh.nh;
  a.nw = sh.nw;
  int n = 0;
  for (int s = 0; s <= sh.S; ++s) {
    const wf_cell& c = p.cells[s];
    if (!c.active) continue;
    const bool capture = s == sh.S && p.anchor.capture;
    a.task[n++] = {s, c.slot, c.frame0, capture ? wf::TASK_CAPTURE : wf::TASK_CELL};
  }
  if (p.anchor.present) a.task[n++] = {0, p.anchor.slot, p.anchor.frame0, wf::TASK_ANCHOR};
  a.n_tasks = n;
  (void)hipGetLastError();
  const hipError_t e = wf::launch_publish(a, sh.dtype, stream);
  if (e != hipSuccess) return fail(WF_EDEVICE, std::string("publish launch: ") + hipGetErrorString(e));
  h->published[layer] = 1;
  return ok();
}

// Model of one attention launch: work-groups taken longest first by n_cu
// compute units, one at a time each; a work-group over p pages costs its key
// tiles plus a fixed 2 (query load, epilogue).  Returns the end time in tiles.
double launch_end(const wf::Shape& sh, int n_cu, int per_group, const std::vector<int>& pages) {
  std::vector<int> len(pages);
  std::sort(len.begin(), len.end(), std::greater<int>());
  std::priority_queue<double, std::vector<double>, std::greater<double>> free_at;
  for (int i = 0; i < n_cu; ++i) free_at.push(0.0);
  double end = 0.0;
  for (const int p : len) {
    const double tiles = (sh.dtype == WF_BF16 ? std::ceil(double(p) * sh.N / 64.0) : double(p) * sh.T) + 2.0;
    for (int i = 0; i < per_group; ++i) {
      const double t = free_at.top() + tiles;
      free_at.pop();
      free_at.push(t);
      end = std::max(end, t);
    }
  }
  return end;
}

// Groups to split and where, for the handle's mode: under WF_SPLIT_AUTO at
// most max_split groups (those whose partial results the scratch holds).
std::vector<wf::SplitAt> choose_split(wf_handle* h, const wf_plan& p, const std::vector<int>& active,
                                      int max_split) {
  const wf::Shape& sh = h->sh;
  std::vector<wf::SplitAt> none;
  if (sh.dtype == WF_F32 || h->split_mode == WF_SPLIT_OFF) return none;
  std::vector<int> cand;   // splittable groups, longest first (ties: lower stage)
  for (const int s : active)
    if (p.groups[s].n_pages >= 2) cand.push_back(s);
  std::stable_sort(cand.begin(), cand.end(),
                   [&](int x, int y) { return p.groups[x].n_pages > p.groups[y].n_pages; });
  if (h->split_mode == WF_SPLIT_FORCE) {
    if (cand.size() > size_t(wf::kMaxSplit)) cand.resize(wf::kMaxSplit);
    std::vector<wf::SplitAt> halves;
    for (const int s : cand) halves.push_back({s, p.groups[s].n_pages / 2});
    return halves;
  }
  std::vector<int> key{max_split};
  for (const int s : active) key.push_back(p.groups[s].n_pages);
  const auto hit = h->split_cache.find(key);
  if (hit != h->split_cache.end()) return hit->second;

  const int bm = sh.dtype == WF_BF16 ? wf::kAttnBM_bf16 : sh.dtype == WF_FP8 ? wf::kAttnBM_fp8 : wf::kAttnBM_fp8k;
  const int per_group = sh.H * ((sh.N + bm - 1) / bm);
  // The merge of one split group moves 10 N H D bytes (two fp32 partials in,
  // bf16 out); priced at 5 TB/s against a tile of bm x 64 x D x 4 FLOP on
  // one compute unit at 1.1 PFLOP/s over n_cu units, plus 2 tiles of launch gap.
  const double tile_s = double(bm) * 64.0 * sh.D * 4.0 / (1.1e15 / h->n_cu);
  const double merge = 2.0 + 10.0 * double(sh.N) * sh.H * sh.D / 5e12 / tile_s;
  auto cost = [&](const std::vector<wf::SplitAt>& sp) {
    std::vector<int> pages;
    for (const int s : active) {
      const int n = p.groups[s].n_pages;
      int at = 0;
      for (const wf::SplitAt& x : sp)
        if (x.stage == s) at = x.at;
      if (at == 0) {
        pages.push_back(n);
      } else {
        pages.push_back(at);
        pages.push_back(n - at);
      }
    }
    return launch_end(sh, h->n_cu, per_group, pages) + merge * double(sp.size());
  };
  // Halves of any one group, then of any two; a strictly lower modelled end
  // is needed to split, or to split more.
  std::vector<wf::SplitAt> best;
  double best_cost = cost(best);
  for (size_t i = 0; i < cand.size() && max_split >= 1; ++i) {
    const std::vector<wf::SplitAt> one{{cand[i], p.groups[cand[i]].n_pages / 2}};
    const double c1 = cost(one);
    if (c1 < best_cost) best_cost = c1, best = one;
  }
  if (max_split >= 2) {
    for (size_t i = 0; i < cand.size(); ++i)
      for (size_t j = i + 1; j < cand.size(); ++j) {
        const std::vector<wf::SplitAt> two{{cand[i], p.groups[cand[i]].n_pages / 2},
                                           {cand[j], p.groups[cand[j]].n_pages / 2}};
        const double c2 = cost(two);
        if (c2 < best_cost) best_cost = c2, best = two;
      }
  }
  h->split_cache.emplace(key, best);
  return best;
}

wf_status do_attention(wf_handle* h, const wf_plan& p, int layer, const void* q_rot, void* out,
                       hipStream_t stream, char* scratch, size_t scratch_cap) {
  const wf::Shape& sh = h->sh;
  wf::AttnArgs a{};
  a.q_rot = q_rot;
  a.out = out;
  a.pool = layer_ptr(h->pool, size_t(sh.n_slots) * sh.page_bytes, layer);
  a.page_elems = static_cast<int64_t>(sh.page_elems);
  a.page_bytes = static_cast<int64_t>(sh.page_bytes);
  a.Npad = sh.Npad;
  a.T = sh.T;
  a.N = sh.N;
  a.H = sh.H;
  a.D = sh.D;
  a.scale_log2e = static_cast<float>(sh.scale * 1.4426950408889634);
  const int bm = sh.dtype == WF_BF16  ? wf::kAttnBM_bf16
                 : sh.dtype == WF_FP8  ? wf::kAttnBM_fp8
                 : sh.dtype == WF_FP8K ? wf::kAttnBM_fp8k
                                       : wf::kAttnBM_f32;
  a.q_tiles = (sh.N + bm - 1) / bm;
  const int per_group = sh.H * a.q_tiles;
  std::vector<int> active;
  for (int s = 0; s <= sh.S; ++s)
    if (p.groups[s].n_pages > 0) active.push_back(s);
  if (!scratch) {
    scratch = static_cast<char*>(h->tables) + (wf::rope_table_bytes(sh) + 255) / 256 * 256;
    scratch_cap = wf::split_scratch_bytes(sh);
  }
  // Two parts per split group: O [N][H][D] fp32 of every part, then (e, l)
  // [N][H] of every part.
  const size_t nh = size_t(sh.N) * size_t(sh.H);
  const size_t nhd = nh * size_t(sh.D);
  const size_t per_split = 2 * (nhd + 2 * nh) * sizeof(float);
  const int max_split = static_cast<int>(std::min<size_t>(wf::kMaxSplit, scratch_cap / per_split));
  const std::vector<wf::SplitAt> split = choose_split(h, p, active, max_split);

  // Runs of the launch: whole groups, or the two parts of a split group
  // (pages [0, at) and [at, n)), longest first (ties: lower stage first).
  struct Run {
    int stage, page0, n_pages, part;
  };
  std::vector<Run> runs;
  wf::CombineArgs c{};
  for (const int s : active) {
    const int n = p.groups[s].n_pages;
    int i = 0;
    while (i < static_cast<int>(split.size()) && split[i].stage != s) ++i;
    if (i == static_cast<int>(split.size())) {
      runs.push_back({s, 0, n, -1});
    } else {
      const int at = split[i].at;
      runs.push_back({s, 0, at, 2 * i});
      runs.push_back({s, at, n - at, 2 * i + 1});
      c.stage[i] = s;
    }
  }
  std::stable_sort(runs.begin(), runs.end(), [](const Run& x, const Run& y) { return x.n_pages > y.n_pages; });
  int item = 0;
  for (size_t i = 0; i < runs.size(); ++i) {
    const Run& r = runs[i];
    const wf_group& g = p.groups[r.stage];
    wf::AttnGroup& o = a.grp[i];
    o.stage = g.stage;
    o.n_pages = r.n_pages;
    o.item0 = item;
    o.part = r.part;
    for (int j = 0; j < r.n_pages; ++j) o.slot[j] = static_cast<uint16_t>(g.slot[r.page0 + j]);
    item += per_group;
  }
  a.n_groups = static_cast<int>(runs.size());
  a.n_items = item;
  const size_t parts = 2 * split.size();
  const size_t need = split.size() * per_split;
  if (need > scratch_cap) {
    return fail(WF_ESMALL, "the split chosen needs " + std::to_string(need) +
                               " bytes of split scratch, above the " + std::to_string(scratch_cap) +
                               " available (WF_SPLIT_OFF needs none)");
  }
  a.part_o = reinterpret_cast<float*>(scratch);
  a.part_el = reinterpret_cast<float*>(scratch + parts * nhd * sizeof(float));
  (void)hipGetLastError();
  hipError_t e = sh.dtype == WF_FP8    ? wf::launch_attention_fp8(a, stream)
                 : sh.dtype == WF_FP8K ? wf::launch_attention_fp8k(a, stream)
                                       : wf::launch_attention(a, sh.dtype, stream);
  if (e != hipSuccess) return fail(WF_EDEVICE, std::string("attention launch: ") + hipGetErrorString(e));
  if (!split.empty()) {
    c.part_o = a.part_o;
    c.part_el = a.part_el;
    c.out = out;
    c.N = sh.N;
    c.H = sh.H;
    c.D = sh.D;
    c.n_split = static_cast<int>(split.size());
    e = wf::launch_combine(c, stream);
    if (e != hipSuccess) return fail(WF_EDEVICE, std::string("combine launch: ") + hipGetErrorString(e));
  }
  return ok();
}

// ---- split scratch of the allocation-free attention entry point ----
// One file-scope device array, which every GPU the library runs on holds
// until the process ends.  Host code never names it directly: the array's
// host-side name is no device address.  Its address on each device is
// looked up once, with that device current, and kept here.
constexpr size_t kStaticScratchBytes = size_t(WF_STATIC_SCRATCH_BYTES);
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxDevices] = {};

wf_status static_scratch(char** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(WF_EDEVICE, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(WF_EUNSUPPORTED, "device index above 63");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(WF_EDEVICE, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    g_scratch_ptr[dev] = static_cast<char*>(ptr);
  }
  *out = g_scratch_ptr[dev];
  return ok();
}

wf_status check_layer_call(const wf_handle* h, int32_t layer) {
  if (layer < 0 || layer >= h->sh.L) return fail(WF_EINVAL, "layer out of range");
  if (!h->bound) return fail(WF_EINVAL, "handle is not bound (call wf_bind first)");
  return ok();
}

}  // namespace rt
}  // namespace wf

using namespace wf::rt;

extern "C" {

const char* wf_strerror(int32_t s) {
  switch (s) {
    case WF_OK: return "ok";
    case WF_EINVAL: return "invalid argument";
    case WF_ERANGE: return "round out of range";
    case WF_EORDER: return "call out of order";
    case WF_ESMALL: return "buffer too small";
    case WF_EDEVICE: return "device error";
    case WF_EUNSUPPORTED: return "unsupported configuration";
  }
  return "unknown status";
}

const char* wf_last_error(void) { return g_last_error.c_str(); }

wf_status wf_create(const wf_config* cfg, wf_handle** out) {
  if (!out) return fail(WF_EINVAL, "out is NULL");
  *out = nullptr;
  wf::Shape sh;
  std::string why;
  if (!wf::derive_shape(cfg, &sh, &why)) return fail(WF_EINVAL, why);
  wf_handle* h = new (std::nothrow) wf_handle();
  if (!h) return fail(WF_EINVAL, "out of host memory");
  h->cfg = *cfg;
  h->sh = sh;
  h->hash = wf::config_hash(*cfg);
  h->published.assign(size_t(sh.L), 0);
  *out = h;
  return ok();
}

void wf_destroy(wf_handle* h) {
  if (h) wf::dit_release(h);
  delete h;
}

wf_status wf_pool_bytes(const wf_config* cfg, size_t* pool, size_t* anchor, size_t* tables) {
  wf::Shape sh;
  std::string why;
  if (!wf::derive_shape(cfg, &sh, &why)) return fail(WF_EINVAL, why);
  if (pool) *pool = wf::pool_bytes(sh);
  if (anchor) *anchor = wf::anchor_bytes(sh);
  if (tables) *tables = wf::table_bytes(sh);
  return ok();
}

wf_status wf_page_layout(const wf_config* cfg, wf_layout* out) {
  if (!out) return fail(WF_EINVAL, "out is NULL");
  wf::Shape sh;
  std::string why;
  if (!wf::derive_shape(cfg, &sh, &why)) return fail(WF_EINVAL, why);
  wf_layout l{};
  l.n_slots = sh.n_slots;
  l.page_bytes = int64_t(sh.page_bytes);
  l.pool_bytes = int64_t(wf::pool_bytes(sh));
  l.anchor_page_bytes = int64_t(sh.anchor_page_bytes);
  l.anchor_bytes = int64_t(wf::anchor_bytes(sh));
  l.tokens = sh.N;
  const bool fp8 = sh.dtype == WF_FP8 || sh.dtype == WF_FP8K;
  l.tokens_padded = fp8 ? sh.Npad : sh.N;
  l.tiles = sh.T;
  l.vt_offset = int64_t(wf::page_vt_offset(sh));
  l.codes_offset = wf::page_codes_offset(sh);
  l.table_bytes = int64_t(wf::table_bytes(sh));
  l.split_scratch_offset = int64_t((wf::rope_table_bytes(sh) + 255) / 256 * 256);
  l.split_scratch_bytes = int64_t(wf::split_scratch_bytes(sh));
  *out = l;
  return ok();
}

wf_status wf_bind(wf_handle* h, void* d_pool, size_t pool_bytes, void* d_anchor_raw,
                  size_t anchor_bytes, void* d_tables, size_t table_bytes) {
  if (!h) return fail(WF_EINVAL, "handle is NULL");
  if (!d_pool || !d_anchor_raw || !d_tables) return fail(WF_EINVAL, "device buffer is NULL");
  const wf::Shape& sh = h->sh;
  if (pool_bytes < wf::pool_bytes(sh)) return fail(WF_ESMALL, "slot pool smaller than wf_pool_bytes");
  if (anchor_bytes < wf::anchor_bytes(sh)) return fail(WF_ESMALL, "anchor buffer smaller than wf_pool_bytes");
  if (table_bytes < wf::table_bytes(sh)) return fail(WF_ESMALL, "table buffer smaller than wf_pool_bytes");
  if (!aligned16(d_pool) || !aligned16(d_anchor_raw) || !aligned16(d_tables))
    return fail(WF_EINVAL, "device buffers must be 16-byte aligned");
  const wf_status sup = check_supported(sh);
  if (sup != WF_OK) return sup;

  // The frame axis's frequencies theta^(-m/nt) in fp64 (the kernels form
  // the angle (frame * omega) and its cos/sin in fp64 on the device), then
  // cos/sin of every (row, pair) and (column, pair), computed in fp64.
  std::vector<unsigned char> tab(wf::rope_table_bytes(sh), 0);
  double* omega = reinterpret_cast<double*>(tab.data());
  for (int m = 0; m < sh.nt; ++m) omega[m] = std::pow(sh.theta, -double(m) / double(sh.nt));
  float* hw = reinterpret_cast<float*>(tab.data() + wf::rope_hw_offset(sh));
  size_t at = 0;
  auto axis = [&](int n_pos, int n_pairs) {
    for (int pos = 0; pos < n_pos; ++pos) {
      for (int m = 0; m < n_pairs; ++m) {
        const double w = std::pow(sh.theta, -double(m) / double(n_pairs));
        const double ang = double(pos) * w;
        hw[at++] = static_cast<float>(std::cos(ang));
        hw[at++] = static_cast<float>(std::sin(ang));
      }
    }
  };
  axis(sh.Hh, sh.nh);
  axis(sh.Ww, sh.nw);
  const hipError_t e = hipMemcpy(d_tables, tab.data(), tab.size(), hipMemcpyHostToDevice);
  if (e != hipSuccess) return fail(WF_EDEVICE, std::string("table upload: ") + hipGetErrorString(e));
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) == hipSuccess &&
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0)
    h->n_cu = cus;
  h->split_cache.clear();
  h->pool = d_pool;
  h->anchor = d_anchor_raw;
  h->tables = d_tables;
  h->bound = true;
  return ok();
}

wf_status wf_set_attention_split(wf_handle* h, int32_t mode) {
  if (!h) return fail(WF_EINVAL, "handle is NULL");
  if (mode != WF_SPLIT_AUTO && mode != WF_SPLIT_OFF && mode != WF_SPLIT_FORCE)
    return fail(WF_EINVAL, "unknown split mode " + std::to_string(mode));
  h->split_mode = mode;
  return ok();
}

wf_status wf_attention_split_choice(wf_handle* h, const wf_plan* plan, int32_t* n_split,
                                    int32_t* stage, int32_t* at) {
  if (!h || !plan || !n_split || !stage || !at) return fail(WF_EINVAL, "NULL argument");
  if (plan->config_hash != h->hash) return fail(WF_EORDER, "plan was made for another config");
  if (!wf::round_in_range(h->sh, plan->k)) return fail(WF_ERANGE, "plan's round outside the request");
  wf_plan p;
  wf::build_plan(h->sh, h->hash, plan->k, &p);
  if (std::memcmp(&p, plan, sizeof(wf_plan)) != 0) return fail(WF_EINVAL, "plan contents were modified");
  std::vector<int> active;
  for (int s = 0; s <= h->sh.S; ++s)
    if (p.groups[s].n_pages > 0) active.push_back(s);
  const std::vector<wf::SplitAt> split = choose_split(h, p, active, wf::kMaxSplit);
  *n_split = static_cast<int32_t>(split.size());
  for (size_t i = 0; i < split.size(); ++i) {
    stage[i] = split[i].stage;
    at[i] = split[i].at;
  }
  return ok();
}

wf_status wf_round_plan(const wf_handle* h, int64_t k, wf_plan* out) {
  if (!h || !out) return fail(WF_EINVAL, "handle or out is NULL");
  if (!wf::round_in_range(h->sh, k)) {
    return fail(WF_ERANGE, h->sh.unbounded
                               ? "round " + std::to_string(k) + " needs more than max_frames = " +
                                     std::to_string(h->sh.max_frames) + " frames"
                               : "round " + std::to_string(k) + " outside [0, n_chunk + S)");
  }
  wf::build_plan(h->sh, h->hash, k, out);
  return ok();
}

wf_status wf_next_round(const wf_handle* h, int64_t* k) {
  if (!h || !k) return fail(WF_EINVAL, "handle or out is NULL");
  *k = h->next_k;
  return ok();
}

wf_status wf_finish_stream(wf_handle* h, int64_t n_chunk) {
  if (!h) return fail(WF_EINVAL, "handle is NULL");
  if (!h->sh.unbounded) return fail(WF_EINVAL, "the request is bounded (n_chunk >= 1); nothing to finish");
  for (const uint8_t p : h->published)
    if (p) return fail(WF_EORDER, "a layer of round " + std::to_string(h->next_k) + " is already published");
  if (n_chunk < h->next_k || n_chunk < 1 || n_chunk > (int64_t(1) << 30)) {
    return fail(WF_EINVAL, "n_chunk " + std::to_string(n_chunk) + " must be >= the next round " +
                               std::to_string(h->next_k) + " and >= 1");
  }
  wf_config c = h->cfg;
  c.n_chunk = static_cast<int32_t>(n_chunk);
  c.max_frames = 0;
  wf::Shape sh;
  std::string why;
  if (!wf::derive_shape(&c, &sh, &why)) return fail(WF_EINVAL, why);
  if (wf::pool_bytes(sh) != wf::pool_bytes(h->sh) || wf::table_bytes(sh) != wf::table_bytes(h->sh) ||
      wf::anchor_bytes(sh) != wf::anchor_bytes(h->sh))
    return fail(WF_EINVAL, "buffer sizes would change");
  h->cfg = c;
  h->sh = sh;
  h->hash = wf::config_hash(c);
  return ok();
}

wf_status wf_reset(wf_handle* h) {
  if (!h) return fail(WF_EINVAL, "handle is NULL");
  h->next_k = 0;
  std::fill(h->published.begin(), h->published.end(), 0);
  return ok();
}

wf_status wf_kv_publish(wf_handle* h, const wf_plan* plan, int32_t layer, const void* d_q,
                        const void* d_k, const void* d_v, void* d_q_rot, void* stream) {
  wf_plan p;
  wf_status s = check_plan(h, plan, &p);
  if (s != WF_OK) return s;
  if ((s = check_layer_call(h, layer)) != WF_OK) return s;
  if (!d_q || !d_k || !d_v || !d_q_rot) return fail(WF_EINVAL, "q, k, v or q_rot is NULL");
  if (!aligned16(d_q) || !aligned16(d_k) || !aligned16(d_v) || !aligned16(d_q_rot))
    return fail(WF_EINVAL, "q, k, v and q_rot must be 16-byte aligned");
  return do_publish(h, p, layer, d_q, d_k, d_v, d_q_rot, static_cast<hipStream_t>(stream));
}

wf_status wf_wave_attention(wf_handle* h, const wf_plan* plan, int32_t layer, const void* d_q_rot,
                            void* d_out, void* stream) {
  wf_plan p;
  wf_status s = check_plan(h, plan, &p);
  if (s != WF_OK) return s;
  if ((s = check_layer_call(h, layer)) != WF_OK) return s;
  if (!h->published[layer]) return fail(WF_EORDER, "layer not published in this round");
  if (!d_q_rot || !d_out) return fail(WF_EINVAL, "q_rot or out is NULL");
  if (!aligned16(d_q_rot) || !aligned16(d_out))
    return fail(WF_EINVAL, "q_rot and out must be 16-byte aligned");
  return do_attention(h, p, layer, d_q_rot, d_out, static_cast<hipStream_t>(stream));
}

wf_status wf_wave_attention_noalloc(wf_handle* h, const wf_plan* plan, int32_t layer,
                                    const void* d_q_rot, void* d_out, void* stream) {
  wf_plan p;
  wf_status s = check_plan(h, plan, &p);
  if (s != WF_OK) return s;
  if ((s = check_layer_call(h, layer)) != WF_OK) return s;
  if (!h->published[layer]) return fail(WF_EORDER, "layer not published in this round");
  if (!d_q_rot || !d_out) return fail(WF_EINVAL, "q_rot or out is NULL");
  if (!aligned16(d_q_rot) || !aligned16(d_out))
    return fail(WF_EINVAL, "q_rot and out must be 16-byte aligned");
  char* base = nullptr;
  if ((s = static_scratch(&base)) != WF_OK) return s;
  return do_attention(h, p, layer, d_q_rot, d_out, static_cast<hipStream_t>(stream), base,
                      kStaticScratchBytes);
}

wf_status wf_round_commit(wf_handle* h, const wf_plan* plan) {
  wf_plan p;
  const wf_status s = check_plan(h, plan, &p);
  if (s != WF_OK) return s;
  for (int l = 0; l < h->sh.L; ++l)
    if (!h->published[l]) return fail(WF_EORDER, "layer " + std::to_string(l) + " not published");
  h->next_k += 1;
  std::fill(h->published.begin(), h->published.end(), 0);
  return ok();
}

wf_status wf_round(wf_handle* h, const wf_plan* plan, const void* d_q, const void* d_k,
                   const void* d_v, void* d_q_rot, void* d_out, void* stream) {
  wf_plan p;
  wf_status s = check_plan(h, plan, &p);
  if (s != WF_OK) return s;
  if (!h->bound) return fail(WF_EINVAL, "handle is not bound (call wf_bind first)");
  if (!d_q || !d_k || !d_v || !d_q_rot || !d_out) return fail(WF_EINVAL, "a tensor pointer is NULL");
  if (!aligned16(d_q) || !aligned16(d_k) || !aligned16(d_v) || !aligned16(d_q_rot) || !aligned16(d_out))
    return fail(WF_EINVAL, "tensors must be 16-byte aligned");
  const size_t per_layer = stage_bytes(h->sh);
  hipStream_t st = static_cast<hipStream_t>(stream);
  for (int l = 0; l < h->sh.L; ++l) {
    s = do_publish(h, p, l, layer_ptr(const_cast<void*>(d_q), per_layer, l),
                   layer_ptr(const_cast<void*>(d_k), per_layer, l),
                   layer_ptr(const_cast<void*>(d_v), per_layer, l), layer_ptr(d_q_rot, per_layer, l), st);
    if (s != WF_OK) return s;
    s = do_attention(h, p, l, layer_ptr(d_q_rot, per_layer, l), layer_ptr(d_out, per_layer, l), st);
    if (s != WF_OK) return s;
  }
  h->next_k += 1;
  std::fill(h->published.begin(), h->published.end(), 0);
  return ok();
}

}  // extern "C"
