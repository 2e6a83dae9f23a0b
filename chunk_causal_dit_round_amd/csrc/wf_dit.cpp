// Host side of the DiT block around the round (include/wf_dit.h):
// validation, the workspace layout, hipBLASLt products and the row-wise
// kernels, all on the caller's stream.
//
// Per layer, with M = active cells x N token rows (active cells are always
// consecutive stages, so each step is one launch over one row range):
//   norm(ln 0) -> QKV product (bias epilogue, bf16) -> qk norm / split ->
//   publish -> attention -> O product (bias, fp32) -> norm(gate 1, ln 1) ->
//   FFN1 product (bias + tanh-GELU epilogue, bf16) -> FFN2 product (bias,
//   fp32) -> norm(gate 2)
// The products are plain GEMMs (D = W A^T over bf16 operands with fp32
// accumulation); hipBLASLt runs them, with the heuristic's first algorithm
// for each shape, kept for later calls.
#include <hip/hip_runtime.h>
#include <hipblaslt/hipblaslt.h>

#include <string>
#include <vector>

#include "wf_dit.h"
#include "wf_dit_kernels.h"
#include "wf_internal.h"

namespace wf {

struct Gemm {
  int m, n, k;
  hipDataType out;
  hipblasLtEpilogue_t epi;
  hipblasLtMatmulDesc_t desc = nullptr;
  hipblasLtMatrixLayout_t la = nullptr, lb = nullptr, ld = nullptr;
  hipblasLtMatmulAlgo_t algo;
  bool tuned = false;
};

struct DitState {
  hipblasLtHandle_t lt = nullptr;
  std::vector<Gemm> gemms;
};

void dit_release(wf_handle* h) {
  DitState* d = h->dit;
  if (!d) return;
  for (Gemm& g : d->gemms) {
    if (g.la) hipblasLtMatrixLayoutDestroy(g.la);
    if (g.lb) hipblasLtMatrixLayoutDestroy(g.lb);
    if (g.ld) hipblasLtMatrixLayoutDestroy(g.ld);
    if (g.desc) hipblasLtMatmulDescDestroy(g.desc);
  }
  if (d->lt) hipblasLtDestroy(d->lt);
  delete d;
  h->dit = nullptr;
}

namespace {

using namespace rt;

constexpr size_t kLtWorkspace = 64ull << 20;  // largest workspace the heuristic may ask for
constexpr size_t kAlign = 256;

size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Byte offsets inside the caller's work buffer.  Every activation buffer
// spans all S+1 stages so that stage s always sits at row s * N.
struct Layout {
  size_t h, qkv, q, k, v, q_rot, o, y, f, lt, total;
};

Layout layout_of(const Shape& sh, int ffn) {
  const size_t rows = size_t(sh.S + 1) * size_t(sh.N);
  const size_t C = size_t(sh.H) * size_t(sh.D);
  Layout L{};
  size_t at = 0;
  auto take = [&](size_t bytes) {
    const size_t p = at;
    at += round_up(bytes);
    return p;
  };
  L.h = take(rows * C * 2);
  L.qkv = take(rows * 3 * C * 2);
  L.q = take(rows * C * 2);
  L.k = take(rows * C * 2);
  L.v = take(rows * C * 2);
  L.q_rot = take(rows * C * 2);
  L.o = take(rows * C * 2);
  L.y = take(rows * C * 4);
  L.f = take(rows * size_t(ffn) * 2);
  L.lt = take(kLtWorkspace);
  L.total = at;
  return L;
}

wf_status check_dc(const wf_handle* h, const wf_dit_config* dc) {
  if (!h || !dc) return fail(WF_EINVAL, "handle or DiT config is NULL");
  if (dc->ffn_dim <= 0 || dc->ffn_dim % 8 != 0) return fail(WF_EINVAL, "ffn_dim must be > 0 and a multiple of 8");
  if (dc->eps < 0) return fail(WF_EINVAL, "eps must be >= 0");
  const int C = h->sh.H * h->sh.D;
  if (C % 8 != 0 || C > kDitMaxC) return fail(WF_EUNSUPPORTED, "the DiT block needs C % 8 == 0 and C <= 8192");
  return ok();
}

std::string lt_error(const char* what, hipblasStatus_t s) {
  return std::string(what) + " failed (hipblasStatus " + std::to_string(int(s)) + ")";
}

// Product plan for D [m x n] (column-major, ld m) = epi(W^T B + bias) with W
// stored k x m (ld k) and B stored k x n (ld k): in row-major terms
// D_rows = B_rows W_rows^T + bias, the nn.Linear product.
wf_status gemm_plan(DitState* d, int m, int n, int k, hipDataType out, hipblasLtEpilogue_t epi, Gemm** res) {
  for (Gemm& g : d->gemms) {
    if (g.m == m && g.n == n && g.k == k && g.out == out && g.epi == epi) {
      *res = &g;
      return ok();
    }
  }
  Gemm g{};
  g.m = m;
  g.n = n;
  g.k = k;
  g.out = out;
  g.epi = epi;
  hipblasStatus_t s = hipblasLtMatmulDescCreate(&g.desc, HIPBLAS_COMPUTE_32F, HIP_R_32F);
  const hipblasOperation_t opT = HIPBLAS_OP_T, opN = HIPBLAS_OP_N;
  const int32_t bias_type = HIP_R_32F;
  if (s == HIPBLAS_STATUS_SUCCESS)
    s = hipblasLtMatmulDescSetAttribute(g.desc, HIPBLASLT_MATMUL_DESC_TRANSA, &opT, sizeof(opT));
  if (s == HIPBLAS_STATUS_SUCCESS)
    s = hipblasLtMatmulDescSetAttribute(g.desc, HIPBLASLT_MATMUL_DESC_TRANSB, &opN, sizeof(opN));
  if (s == HIPBLAS_STATUS_SUCCESS)
    s = hipblasLtMatmulDescSetAttribute(g.desc, HIPBLASLT_MATMUL_DESC_EPILOGUE, &epi, sizeof(epi));
  if (s == HIPBLAS_STATUS_SUCCESS)
    s = hipblasLtMatmulDescSetAttribute(g.desc, HIPBLASLT_MATMUL_DESC_BIAS_DATA_TYPE, &bias_type,
                                        sizeof(bias_type));
  if (s == HIPBLAS_STATUS_SUCCESS) s = hipblasLtMatrixLayoutCreate(&g.la, HIP_R_16BF, k, m, k);
  if (s == HIPBLAS_STATUS_SUCCESS) s = hipblasLtMatrixLayoutCreate(&g.lb, HIP_R_16BF, k, n, k);
  if (s == HIPBLAS_STATUS_SUCCESS) s = hipblasLtMatrixLayoutCreate(&g.ld, out, m, n, m);
  hipblasLtMatmulPreference_t pref = nullptr;
  if (s == HIPBLAS_STATUS_SUCCESS) s = hipblasLtMatmulPreferenceCreate(&pref);
  const uint64_t ws = kLtWorkspace;
  if (s == HIPBLAS_STATUS_SUCCESS)
    s = hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &ws, sizeof(ws));
  hipblasLtMatmulHeuristicResult_t hr[1];
  int n_res = 0;
  if (s == HIPBLAS_STATUS_SUCCESS)
    s = hipblasLtMatmulAlgoGetHeuristic(d->lt, g.desc, g.la, g.lb, g.ld, g.ld, pref, 1, hr, &n_res);
  if (pref) hipblasLtMatmulPreferenceDestroy(pref);
  if (s != HIPBLAS_STATUS_SUCCESS || n_res < 1) {
    if (g.la) hipblasLtMatrixLayoutDestroy(g.la);
    if (g.lb) hipblasLtMatrixLayoutDestroy(g.lb);
    if (g.ld) hipblasLtMatrixLayoutDestroy(g.ld);
    if (g.desc) hipblasLtMatmulDescDestroy(g.desc);
    if (s != HIPBLAS_STATUS_SUCCESS) return fail(WF_EDEVICE, lt_error("hipBLASLt product setup", s));
    return fail(WF_EUNSUPPORTED, "hipBLASLt has no algorithm for a " + std::to_string(m) + "x" +
                                     std::to_string(n) + "x" + std::to_string(k) + " product");
  }
  g.algo = hr[0].algo;
  d->gemms.push_back(g);
  *res = &d->gemms.back();
  return ok();
}

wf_status gemm(DitState* d, int m, int n, int k, hipDataType out, hipblasLtEpilogue_t epi, const void* W,
               const void* B, void* D, const void* bias, void* ws, hipStream_t st) {
  Gemm* g = nullptr;
  wf_status r = gemm_plan(d, m, n, k, out, epi, &g);
  if (r != WF_OK) return r;
  hipblasStatus_t s =
      hipblasLtMatmulDescSetAttribute(g->desc, HIPBLASLT_MATMUL_DESC_BIAS_POINTER, &bias, sizeof(bias));
  const float alpha = 1.f, beta = 0.f;
  if (s == HIPBLAS_STATUS_SUCCESS)
    s = hipblasLtMatmul(d->lt, g->desc, &alpha, W, g->la, B, g->lb, &beta, D, g->ld, D, g->ld, &g->algo, ws,
                        kLtWorkspace, st);
  if (s != HIPBLAS_STATUS_SUCCESS) return fail(WF_EDEVICE, lt_error("hipBLASLt product", s));
  return ok();
}

// Times the heuristic's first candidates for one product shape on the given
// operands (2 warm-up and 5 timed runs each, HIP events on `st`) and keeps
// the fastest.  Candidates the library rejects at run time are skipped.
wf_status tune_gemm(DitState* d, int m, int n, int k, hipDataType out, hipblasLtEpilogue_t epi, const void* W,
                    const void* B, void* D, const void* bias, void* ws, hipStream_t st) {
  Gemm* g = nullptr;
  wf_status r = gemm_plan(d, m, n, k, out, epi, &g);
  if (r != WF_OK || g->tuned) return r;
  hipblasLtMatmulPreference_t pref = nullptr;
  hipblasStatus_t s = hipblasLtMatmulPreferenceCreate(&pref);
  const uint64_t wsb = kLtWorkspace;
  if (s == HIPBLAS_STATUS_SUCCESS)
    s = hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &wsb, sizeof(wsb));
  hipblasLtMatmulHeuristicResult_t hr[WF_DIT_TUNE_CANDIDATES];
  int n_res = 0;
  if (s == HIPBLAS_STATUS_SUCCESS)
    s = hipblasLtMatmulAlgoGetHeuristic(d->lt, g->desc, g->la, g->lb, g->ld, g->ld, pref, WF_DIT_TUNE_CANDIDATES,
                                        hr, &n_res);
  if (pref) hipblasLtMatmulPreferenceDestroy(pref);
  if (s != HIPBLAS_STATUS_SUCCESS) return fail(WF_EDEVICE, lt_error("hipBLASLt heuristic", s));
  s = hipblasLtMatmulDescSetAttribute(g->desc, HIPBLASLT_MATMUL_DESC_BIAS_POINTER, &bias, sizeof(bias));
  if (s != HIPBLAS_STATUS_SUCCESS) return fail(WF_EDEVICE, lt_error("hipBLASLt bias", s));
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
    if (e0) (void)hipEventDestroy(e0);
    return fail(WF_EDEVICE, "hipEventCreate failed");
  }
  const float alpha = 1.f, beta = 0.f;
  float best_ms = 0.f;
  int best = -1;
  for (int i = 0; i < n_res; ++i) {
    auto run = [&]() {
      return hipblasLtMatmul(d->lt, g->desc, &alpha, W, g->la, B, g->lb, &beta, D, g->ld, D, g->ld, &hr[i].algo,
                             ws, kLtWorkspace, st);
    };
    if (run() != HIPBLAS_STATUS_SUCCESS || run() != HIPBLAS_STATUS_SUCCESS) continue;
    bool ok_run = hipEventRecord(e0, st) == hipSuccess;
    for (int rep = 0; rep < 5 && ok_run; ++rep) ok_run = run() == HIPBLAS_STATUS_SUCCESS;
    float ms = 0.f;
    ok_run = ok_run && hipEventRecord(e1, st) == hipSuccess && hipEventSynchronize(e1) == hipSuccess &&
             hipEventElapsedTime(&ms, e0, e1) == hipSuccess;
    if (ok_run && (best < 0 || ms < best_ms)) {
      best = i;
      best_ms = ms;
    }
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (best >= 0) g->algo = hr[best].algo;
  g->tuned = true;
  return ok();
}

wf_status kernel_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(WF_EDEVICE, std::string(what) + ": " + hipGetErrorString(e));
  return ok();
}

wf_status check_call(wf_handle* h, const wf_dit_config* dc, const wf_dit_weights* w, int n_weights,
                     const void* mod, void* x, void* work, size_t work_bytes) {
  wf_status s = check_dc(h, dc);
  if (s != WF_OK) return s;
  if (!h->bound) return fail(WF_EINVAL, "handle is not bound (call wf_bind first)");
  // bf16 activations and weights; the pages may be bf16, FP8 or FP8 keys
  // with bf16 values (their q/k/v/q_rot/out tensors are bf16 in all three)
  if (h->sh.dtype == WF_F32) return fail(WF_EUNSUPPORTED, "the DiT block runs bf16 activations, not fp32 rounds");
  if (!w || !mod || !x || !work) return fail(WF_EINVAL, "weights, mod, x or work is NULL");
  if (!aligned16(mod) || !aligned16(x) || !aligned16(work))
    return fail(WF_EINVAL, "mod, x and work must be 16-byte aligned");
  for (int l = 0; l < n_weights; ++l) {
    const void* p[10] = {w[l].w_qkv, w[l].b_qkv, w[l].g_q, w[l].g_k, w[l].w_o,
                         w[l].b_o,   w[l].w_1,   w[l].b_1, w[l].w_2, w[l].b_2};
    for (const void* q : p) {
      if (!q) return fail(WF_EINVAL, "layer " + std::to_string(l) + ": a weight pointer is NULL");
      if (!aligned16(q)) return fail(WF_EINVAL, "layer " + std::to_string(l) + ": weights must be 16-byte aligned");
    }
  }
  if (work_bytes < layout_of(h->sh, dc->ffn_dim).total) return fail(WF_ESMALL, "work smaller than wf_dit_workspace_bytes");
  if (!h->dit) {
    DitState* d = new (std::nothrow) DitState();
    if (!d) return fail(WF_EINVAL, "out of host memory");
    const hipblasStatus_t e = hipblasLtCreate(&d->lt);
    if (e != HIPBLAS_STATUS_SUCCESS) {
      delete d;
      return fail(WF_EDEVICE, lt_error("hipblasLtCreate", e));
    }
    h->dit = d;
  }
  return ok();
}

wf_status dit_layer(wf_handle* h, const wf_plan& p, int layer, const wf_dit_config& dc,
                    const wf_dit_weights& w, const float* mod, float* x, char* work, hipStream_t st) {
  const Shape& sh = h->sh;
  const int N = sh.N, C = sh.H * sh.D, F = dc.ffn_dim;
  int s_lo = -1, s_hi = -1;
  for (int s = 0; s <= sh.S; ++s) {
    if (!p.cells[s].active) continue;
    if (s_lo < 0) s_lo = s;
    s_hi = s;
  }
  if (s_lo < 0) return fail(WF_EINVAL, "round has no active cell");
  for (int s = s_lo; s <= s_hi; ++s)
    if (!p.cells[s].active) return fail(WF_EINVAL, "active cells are not consecutive stages");
  const int rows = (s_hi - s_lo + 1) * N;
  const size_t r0 = size_t(s_lo) * size_t(N);
  const Layout L = layout_of(sh, F);
  __bf16* hb = reinterpret_cast<__bf16*>(work + L.h);
  __bf16* qkv = reinterpret_cast<__bf16*>(work + L.qkv);
  __bf16* q = reinterpret_cast<__bf16*>(work + L.q);
  __bf16* k = reinterpret_cast<__bf16*>(work + L.k);
  __bf16* v = reinterpret_cast<__bf16*>(work + L.v);
  __bf16* q_rot = reinterpret_cast<__bf16*>(work + L.q_rot);
  __bf16* o = reinterpret_cast<__bf16*>(work + L.o);
  float* y = reinterpret_cast<float*>(work + L.y);
  __bf16* f = reinterpret_cast<__bf16*>(work + L.f);
  void* ws = work + L.lt;
  const float eps = static_cast<float>(dc.eps > 0 ? dc.eps : 1e-6);
  DitState* d = h->dit;
  (void)hipGetLastError();

  NormArgs na{};
  na.x = x + r0 * C;
  na.mod = mod;
  na.h = hb + r0 * C;
  na.rows = rows;
  na.C = C;
  na.N = N;
  na.s_lo = s_lo;
  na.gate = 2;
  na.ln = 0;
  na.eps = eps;
  wf_status s = kernel_status(launch_norm(na, st), "norm launch");
  if (s != WF_OK) return s;
  s = gemm(d, 3 * C, rows, C, HIP_R_16BF, HIPBLASLT_EPILOGUE_BIAS, w.w_qkv, hb + r0 * C, qkv + r0 * 3 * C,
           w.b_qkv, ws, st);
  if (s != WF_OK) return s;
  QkNormArgs qa{};
  qa.qkv = qkv + r0 * 3 * C;
  qa.g_q = static_cast<const float*>(w.g_q);
  qa.g_k = static_cast<const float*>(w.g_k);
  qa.q = q + r0 * C;
  qa.k = k + r0 * C;
  qa.v = v + r0 * C;
  qa.rows = rows;
  qa.C = C;
  qa.eps = eps;
  if ((s = kernel_status(launch_qk_norm(qa, st), "qk norm launch")) != WF_OK) return s;
  if ((s = do_publish(h, p, layer, q, k, v, q_rot, st)) != WF_OK) return s;
  if ((s = do_attention(h, p, layer, q_rot, o, st)) != WF_OK) return s;
  s = gemm(d, C, rows, C, HIP_R_32F, HIPBLASLT_EPILOGUE_BIAS, w.w_o, o + r0 * C, y + r0 * C, w.b_o, ws, st);
  if (s != WF_OK) return s;
  na.y = y + r0 * C;
  na.gate = 2;
  na.ln = 1;
  if ((s = kernel_status(launch_norm(na, st), "norm launch")) != WF_OK) return s;
  s = gemm(d, F, rows, C, HIP_R_16BF, HIPBLASLT_EPILOGUE_GELU_BIAS, w.w_1, hb + r0 * C, f + r0 * F, w.b_1, ws,
           st);
  if (s != WF_OK) return s;
  s = gemm(d, C, rows, F, HIP_R_32F, HIPBLASLT_EPILOGUE_BIAS, w.w_2, f + r0 * F, y + r0 * C, w.b_2, ws, st);
  if (s != WF_OK) return s;
  na.gate = 5;
  na.ln = -1;
  na.h = nullptr;
  return kernel_status(launch_norm(na, st), "norm launch");
}

}  // namespace
}  // namespace wf

using namespace wf::rt;

extern "C" {

wf_status wf_dit_workspace_bytes(const wf_handle* h, const wf_dit_config* dc, size_t* bytes) {
  if (!bytes) return fail(WF_EINVAL, "bytes is NULL");
  const wf_status s = wf::check_dc(h, dc);
  if (s != WF_OK) return s;
  *bytes = wf::layout_of(h->sh, dc->ffn_dim).total;
  return ok();
}

wf_status wf_dit_layer(wf_handle* h, const wf_plan* plan, int32_t layer, const wf_dit_config* dc,
                       const wf_dit_weights* w, const void* d_mod, void* d_x, void* d_work, size_t work_bytes,
                       void* stream) {
  wf_plan p;
  wf_status s = check_plan(h, plan, &p);
  if (s != WF_OK) return s;
  if ((s = check_layer_call(h, layer)) != WF_OK) return s;
  if ((s = wf::check_call(h, dc, w, 1, d_mod, d_x, d_work, work_bytes)) != WF_OK) return s;
  return wf::dit_layer(h, p, layer, *dc, *w, static_cast<const float*>(d_mod), static_cast<float*>(d_x),
                       static_cast<char*>(d_work), static_cast<hipStream_t>(stream));
}

wf_status wf_dit_tune(wf_handle* h, const wf_dit_config* dc, const wf_dit_weights* w, void* d_work,
                      size_t work_bytes, void* stream) {
  if (!h) return fail(WF_EINVAL, "handle is NULL");
  if (!h->bound) return fail(WF_EINVAL, "handle is not bound (call wf_bind first)");
  // the block's checks with the work buffer standing in for mod and x
  wf_status s = wf::check_call(h, dc, w, 1, d_work, d_work, d_work, work_bytes);
  if (s != WF_OK) return s;
  const wf::Shape& sh = h->sh;
  const int rows = (sh.S + 1) * sh.N, C = sh.H * sh.D, F = dc->ffn_dim;
  const wf::Layout L = wf::layout_of(sh, F);
  char* work = static_cast<char*>(d_work);
  void* ws = work + L.lt;
  hipStream_t st = static_cast<hipStream_t>(stream);
  wf::DitState* d = h->dit;
  s = wf::tune_gemm(d, 3 * C, rows, C, HIP_R_16BF, HIPBLASLT_EPILOGUE_BIAS, w->w_qkv, work + L.h, work + L.qkv,
                    w->b_qkv, ws, st);
  if (s == WF_OK)
    s = wf::tune_gemm(d, C, rows, C, HIP_R_32F, HIPBLASLT_EPILOGUE_BIAS, w->w_o, work + L.o, work + L.y, w->b_o,
                      ws, st);
  if (s == WF_OK)
    s = wf::tune_gemm(d, F, rows, C, HIP_R_16BF, HIPBLASLT_EPILOGUE_GELU_BIAS, w->w_1, work + L.h, work + L.f,
                      w->b_1, ws, st);
  if (s == WF_OK)
    s = wf::tune_gemm(d, C, rows, F, HIP_R_32F, HIPBLASLT_EPILOGUE_BIAS, w->w_2, work + L.f, work + L.y, w->b_2,
                      ws, st);
  return s;
}

wf_status wf_dit_round(wf_handle* h, const wf_plan* plan, const wf_dit_config* dc, const wf_dit_weights* w,
                       const void* d_mod, void* d_x, void* d_work, size_t work_bytes, void* stream) {
  wf_plan p;
  wf_status s = check_plan(h, plan, &p);
  if (s != WF_OK) return s;
  if (!h->bound) return fail(WF_EINVAL, "handle is not bound (call wf_bind first)");
  if ((s = wf::check_call(h, dc, w, h->sh.L, d_mod, d_x, d_work, work_bytes)) != WF_OK) return s;
  const size_t mod_layer = size_t(h->sh.S + 1) * 6 * size_t(h->sh.H) * size_t(h->sh.D);
  for (int l = 0; l < h->sh.L; ++l) {
    s = wf::dit_layer(h, p, l, *dc, w[l], static_cast<const float*>(d_mod) + mod_layer * l,
                      static_cast<float*>(d_x), static_cast<char*>(d_work), static_cast<hipStream_t>(stream));
    if (s != WF_OK) return s;
  }
  return wf_round_commit(h, plan);
}

}  // extern "C"
