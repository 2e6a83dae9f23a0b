// Round scheduler and page allocator (see wf_plan.h for the sources).
#include "wf_plan.h"

#include <cmath>
#include <cstring>

namespace wf {
namespace {

bool mul_ok(size_t a, size_t b, size_t* r) { return !__builtin_mul_overflow(a, b, r); }

bool fail(std::string* why, const char* msg) {
  if (why) *why = msg;
  return false;
}

// Chunk i exists in the request.
inline bool live(const Shape& sh, int64_t i) { return i >= 0 && (sh.unbounded || i < sh.n_chunk); }

}  // namespace

bool derive_shape(const wf_config* c, Shape* o, std::string* why) {
  if (!c) return fail(why, "config is NULL");
  if (c->S < 1 || c->S > WF_MAX_STAGES) return fail(why, "S must be in [1, 8]");
  if (c->W < 0 || c->W > WF_MAX_PAGES) return fail(why, "W must be in [0, 48]");
  if (c->W_store < -1 || c->W_store > WF_MAX_PAGES)
    return fail(why, "W_store must be -1 or in [0, 48]");
  if (c->anchor != 0 && c->anchor != 1) return fail(why, "anchor must be 0 or 1");
  if (c->F < 1 || c->Hh < 1 || c->Ww < 1) return fail(why, "F, Hh, Ww must be >= 1");
  if (c->n_chunk >= 1) {
    if (int64_t(c->n_chunk) * c->F > (int64_t(1) << 30))
      return fail(why, "n_chunk * F must be <= 2^30 (frame positions)");
    if (c->max_frames != 0) return fail(why, "max_frames must be 0 for a bounded request (n_chunk >= 1)");
  } else if (c->max_frames < c->F || c->max_frames > (1 << 30)) {
    return fail(why, "an unbounded request (n_chunk <= 0) needs max_frames in [F, 2^30]");
  }
  const int64_t n = int64_t(c->F) * c->Hh * c->Ww;
  if (n > (1 << 24)) return fail(why, "tokens per chunk F*Hh*Ww must be <= 2^24");
  if (c->n_heads < 1 || c->n_heads > 1024) return fail(why, "n_heads must be in [1, 1024]");
  if (c->head_dim < 6 || c->head_dim > 512 || (c->head_dim & 1))
    return fail(why, "head_dim must be even and in [6, 512]");
  if (c->n_layers < 1 || c->n_layers > 4096) return fail(why, "n_layers must be in [1, 4096]");
  if (c->dtype != WF_F32 && c->dtype != WF_BF16 && c->dtype != WF_FP8 && c->dtype != WF_FP8K)
    return fail(why, "dtype must be WF_F32, WF_BF16, WF_FP8 or WF_FP8K");
  if (c->mask != WF_MASK_WAVE && c->mask != WF_MASK_ROLLING)
    return fail(why, "mask must be WF_MASK_WAVE or WF_MASK_ROLLING");
  if (!(c->rope_theta >= 0.0) || !std::isfinite(c->rope_theta) ||
      (c->rope_theta != 0.0 && c->rope_theta <= 1.0))
    return fail(why, "rope_theta must be 0 (default) or > 1");
  if (!(c->softmax_scale >= 0.0) || !std::isfinite(c->softmax_scale))
    return fail(why, "softmax_scale must be finite and >= 0");

  Shape s{};
  s.S = c->S;
  s.W = c->W;
  s.Ws = c->W_store < 0 ? c->W + c->S : c->W_store;
  s.Wmax = s.W > s.Ws ? s.W : s.Ws;
  s.ring = s.Wmax + 2;
  s.anchor = c->anchor;
  s.unbounded = c->n_chunk <= 0;
  s.n_chunk = s.unbounded ? 0 : c->n_chunk;
  s.max_frames = c->max_frames;
  s.F = c->F;
  s.Hh = c->Hh;
  s.Ww = c->Ww;
  s.H = c->n_heads;
  s.D = c->head_dim;
  s.L = c->n_layers;
  s.N = static_cast<int>(n);
  s.n_slots = 4 + s.Wmax + 2 * s.S;
  // Longest context: anchor + history + store + every denoising chunk.
  const int worst = 1 + s.Wmax + 1 + s.S;
  if (worst > WF_MAX_PAGES) return fail(why, "anchor + max(W, W_store) + 1 + S exceeds 48 pages");
  s.nh = s.D / 6;
  s.nw = s.nh;
  s.nt = s.D / 2 - 2 * s.nh;
  s.dtype = c->dtype;
  s.mask = c->mask;
  s.theta = c->rope_theta == 0.0 ? 10000.0 : c->rope_theta;
  s.scale = c->softmax_scale == 0.0 ? 1.0 / std::sqrt(double(s.D)) : c->softmax_scale;
  s.elem = c->dtype == WF_F32 ? 4 : 2;
  s.T = (s.N + 63) / 64;
  s.Npad = 64 * s.T;
  size_t pe = 0, tmp = 0;
  if (!mul_ok(size_t(2) * s.H, size_t(s.N), &pe) || !mul_ok(pe, size_t(s.D), &pe))
    return fail(why, "page size overflows");
  s.page_elems = pe;
  if (!mul_ok(pe, s.elem, &s.anchor_page_bytes)) return fail(why, "page size overflows");
  if (c->dtype == WF_FP8 || c->dtype == WF_FP8K) {
    // K in one byte per element; V in one (FP8) or two (FP8K: bf16) bytes
    size_t kv = 0;
    const size_t bytes_kv = c->dtype == WF_FP8 ? 2 : 3;
    if (!mul_ok(bytes_kv * s.H, size_t(s.Npad), &kv) || !mul_ok(kv, size_t(s.D), &kv))
      return fail(why, "page size overflows");
    const size_t codes = size_t(2) * s.H * s.T;
    s.page_bytes = (kv + codes + 255) / 256 * 256;
  } else {
    s.page_bytes = s.anchor_page_bytes;
  }
  if (!mul_ok(s.page_bytes, size_t(s.L) * s.n_slots, &tmp)) return fail(why, "pool size overflows");
  *o = s;
  return true;
}

uint64_t config_hash(const wf_config& c) {
  uint64_t h = 1469598103934665603ull;
  auto mix = [&h](const void* p, size_t n) {
    const unsigned char* b = static_cast<const unsigned char*>(p);
    for (size_t i = 0; i < n; ++i) {
      h ^= b[i];
      h *= 1099511628211ull;
    }
  };
  const int32_t ints[] = {c.S, c.W, c.W_store, c.anchor, c.n_chunk <= 0 ? 0 : c.n_chunk, c.F, c.Hh, c.Ww,
                          c.n_heads, c.head_dim, c.n_layers, c.dtype, c.mask, c.max_frames};
  mix(ints, sizeof(ints));
  mix(&c.rope_theta, sizeof(double));
  mix(&c.softmax_scale, sizeof(double));
  return h;
}

size_t pool_bytes(const Shape& sh) { return size_t(sh.L) * sh.n_slots * sh.page_bytes; }
size_t anchor_bytes(const Shape& sh) { return size_t(sh.L) * sh.anchor_page_bytes; }
size_t rope_hw_offset(const Shape& sh) { return (size_t(sh.nt) * sizeof(double) + 15) / 16 * 16; }
size_t rope_table_bytes(const Shape& sh) {
  return rope_hw_offset(sh) + (size_t(sh.Hh) * sh.nh + size_t(sh.Ww) * sh.nw) * 2 * sizeof(float);
}
bool round_in_range(const Shape& sh, int64_t k) {
  if (k < 0) return false;
  if (sh.unbounded) return int64_t(sh.F) * (k + 1) <= sh.max_frames;
  return k < int64_t(sh.n_chunk) + sh.S;
}
// Two halves per split group: O [N][H][D] and (e, l) [N][H] in fp32.
size_t split_scratch_bytes(const Shape& sh) {
  if (sh.dtype == WF_F32) return 0;
  const size_t nh = size_t(sh.N) * size_t(sh.H);
  return size_t(kMaxSplit) * 2 * (nh * size_t(sh.D) + 2 * nh) * sizeof(float);
}
size_t table_bytes(const Shape& sh) {
  return (rope_table_bytes(sh) + 255) / 256 * 256 + split_scratch_bytes(sh);
}

size_t page_vt_offset(const Shape& sh) {
  if (sh.dtype == WF_FP8 || sh.dtype == WF_FP8K) return size_t(sh.H) * sh.Npad * sh.D;
  return size_t(sh.H) * sh.N * sh.D * sh.elem;
}
int64_t page_codes_offset(const Shape& sh) {
  if (sh.dtype == WF_FP8) return int64_t(2) * sh.H * sh.Npad * sh.D;
  if (sh.dtype == WF_FP8K) return int64_t(3) * sh.H * sh.Npad * sh.D;
  return -1;
}

void build_plan(const Shape& sh, uint64_t hash, int64_t k, wf_plan* p) {
  std::memset(p, 0, sizeof(*p));
  p->k = k;
  p->config_hash = hash;
  p->S = sh.S;
  const int S = sh.S;
  const int64_t store_chunk = k - S;
  const bool store_on = live(sh, store_chunk);
  // Anchor: chunk 0, readable once it has been stored (round S), captured
  // from the raw projections in that round (App. B.3).
  const bool anchor_on = sh.anchor == 1 && k >= S + 1;
  p->anchor.present = anchor_on;
  p->anchor.capture = sh.anchor == 1 && k == S;
  p->anchor.slot = anchor_on ? slot_anchor(k) : -1;
  {
    // Placed just before the oldest retained clean page when the window
    // has slid past chunk 1.
    const int64_t shift = k - S - sh.Wmax - 1;
    p->anchor.frame0 = anchor_on ? static_cast<int>(sh.F * (shift > 0 ? shift : 0)) : -1;
  }
  p->evict_chunk = -1;
  if (store_on && store_chunk - sh.Wmax >= sh.anchor) {
    p->evict_chunk = static_cast<int>(store_chunk - sh.Wmax);
  }

  // Cells on the anti-diagonal k = i + s (Eq. 3).
  for (int s = 0; s <= S; ++s) {
    wf_cell& c = p->cells[s];
    const int64_t i = k - s;
    c.stage = s;
    c.active = live(sh, i);
    c.chunk = c.active ? static_cast<int>(i) : -1;
    c.frame0 = c.active ? static_cast<int>(i * sh.F) : -1;
    c.slot = !c.active ? -1 : (s == S ? slot_clean(sh, i) : slot_denoise(sh, k, s));
    p->n_active += c.active;
  }

  // Ordered contexts (Eq. 5).
  int64_t pages_total = 0;
  for (int s = 0; s <= S; ++s) {
    wf_group& g = p->groups[s];
    g.stage = s;
    if (!p->cells[s].active) continue;
    int n = 0;
    auto push = [&](int kind, int64_t chunk, int slot) {
      g.kind[n] = kind;
      g.chunk[n] = static_cast<int>(chunk);
      g.slot[n] = slot;
      ++n;
    };
    if (anchor_on) push(WF_KIND_ANCHOR, 0, slot_anchor(k));
    const int window = s == S ? sh.Ws : sh.W;
    int64_t lo = k - S - window;
    if (lo < sh.anchor) lo = sh.anchor;
    for (int64_t c = lo; c <= k - S - 1; ++c) push(WF_KIND_HISTORY, c, slot_clean(sh, c));
    if (store_on) push(WF_KIND_STORE, store_chunk, slot_clean(sh, store_chunk));
    if (s < S) {
      // Denoising K/V by increasing stage j; WF reads j >= s, the
      // Rolling-Forcing comparison reads every active stage.
      const int j0 = sh.mask == WF_MASK_WAVE ? s : 0;
      for (int j = j0; j < S; ++j) {
        if (live(sh, k - j)) push(WF_KIND_DENOISE, k - j, slot_denoise(sh, k, j));
      }
    }
    g.n_pages = n;
    pages_total += n;
  }

  const double nhd = double(sh.N) * sh.H * sh.D;
  p->kv_tokens = pages_total * sh.N;
  p->flops = double(sh.L) * 4.0 * double(sh.N) * double(p->kv_tokens) * sh.D * sh.H;
  // Publish traffic per layer: read q,k,v and write q_rot, K, Vt per active
  // cell; read anchor_raw K, Vt and write the anchor slot when present;
  // write anchor_raw K, Vt in the capture round.
  double per_layer = 6.0 * p->n_active * nhd;
  if (p->anchor.present) per_layer += 4.0 * nhd;
  if (p->anchor.capture) per_layer += 2.0 * nhd;
  per_layer *= double(sh.elem);
  if (sh.dtype == WF_FP8) {
    // pages hold one byte per element: per cell q,k,v,q_rot stay bf16 and
    // K, Vt shrink to 1 byte; the anchor slot write shrinks likewise
    per_layer -= 2.0 * p->n_active * nhd;
    if (p->anchor.present) per_layer -= 2.0 * nhd;
  } else if (sh.dtype == WF_FP8K) {
    // only K shrinks to 1 byte
    per_layer -= 1.0 * p->n_active * nhd;
    if (p->anchor.present) per_layer -= 1.0 * nhd;
  }
  p->publish_bytes = double(sh.L) * per_layer;
}

}  // namespace wf
