// Round scheduler and page allocator: host-only C++, no HIP dependency.
//
// The plan of round k is a pure function of (config, k).  Rules follow
// "Wave Forcing: Towards Speed-of-Light Streaming Video Generation"
// (arXiv 2611.00859): §3.1 Eq. 3 (cells and active set), Eq. 4 (mask),
// Eq. 5 (context order), App. B.2 Eq. 13 (fixed double-buffered slots),
// App. B.3 (store promotion, persistent anchor, store prefix budget).
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>

#include "wf.h"

namespace wf {

// Everything the library derives once from a validated wf_config.
struct Shape {
  int S, W, Ws, Wmax, ring, anchor, n_chunk;
  bool unbounded;              // n_chunk <= 0: a stream, every chunk >= 0 exists
  int max_frames;              // unbounded: frames the stream may reach
  int F, Hh, Ww, H, D, L, N;   // N = tokens per chunk
  int n_slots;                 // 4 + Wmax + 2 S
  int nt, nh, nw;              // RoPE pairs per axis (frame, row, column)
  int dtype, mask;
  double theta, scale;
  size_t elem;                 // bytes per element of q/k/v/q_rot/out
  size_t page_elems;           // 2 H N D
  // Pool page in bytes.  fp32 / bf16: page_elems * elem.  FP8: K [H][Npad][D]
  // and Vt [H][D][Npad] in E4M3, then the per-tile scale codes [H][T][2],
  // rounded up to 256 bytes (Npad = 64 T >= N).  FP8K: the same with Vt in
  // bf16.
  size_t page_bytes;
  size_t anchor_page_bytes;    // raw K + Vt of chunk 0 (bf16 for FP8 pages)
  int Npad, T;
};

// Validates cfg (method-level rules only) and fills `out`.  Returns false
// with a reason in `why` when the config is invalid.
bool derive_shape(const wf_config* cfg, Shape* out, std::string* why);

// FNV-1a over the config fields that change a plan or a launch.
uint64_t config_hash(const wf_config& cfg);

// Round k exists: 0 <= k < n_chunk + S, or F (k + 1) <= max_frames when unbounded.
bool round_in_range(const Shape& sh, int64_t k);

// Builds the plan of round k (caller checked round_in_range).
void build_plan(const Shape& sh, uint64_t hash, int64_t k, wf_plan* out);

// Slot ring (closed form; ring = Wmax + 2):
//   anchor -> k mod 2, clean chunk c -> 2 + c mod ring,
//   denoising stage j of round k -> 2 + ring + (k mod 2) S + j.
inline int slot_anchor(int64_t k) { return static_cast<int>(k & 1); }
inline int slot_clean(const Shape& sh, int64_t c) {
  return 2 + static_cast<int>(c % sh.ring);
}
inline int slot_denoise(const Shape& sh, int64_t k, int j) {
  return 2 + sh.ring + static_cast<int>(k & 1) * sh.S + j;
}

// At most this many query groups of one attention launch are split into two
// parts over their pages (bf16, FP8 and FP8K rounds); the parts' partial
// results live in device scratch after the RoPE tables.
constexpr int kMaxSplit = WF_MAX_SPLIT;

// Bytes of caller buffers.  The table buffer holds the RoPE tables
// (rope_table_bytes, rounded up to 256) and then the split scratch.  The
// RoPE part is the frame-axis frequencies (nt doubles, padded to 16 bytes)
// and the row and column cos/sin tables; rope_hw_offset is where the latter
// start.
size_t pool_bytes(const Shape& sh);
size_t anchor_bytes(const Shape& sh);
size_t rope_table_bytes(const Shape& sh);
size_t rope_hw_offset(const Shape& sh);
size_t split_scratch_bytes(const Shape& sh);
size_t table_bytes(const Shape& sh);
// Byte offsets inside one pool page: Vt after K, then (FP8 / FP8K) the codes.
size_t page_vt_offset(const Shape& sh);
int64_t page_codes_offset(const Shape& sh);   // -1 when the page has none

}  // namespace wf
