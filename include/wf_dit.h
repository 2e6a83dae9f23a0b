/*
 * wf_dit.h -- C ABI of the Wan-shaped DiT block around the wavefront round.
 *
 * WF ("Wave Forcing: Towards Speed-of-Light Streaming Video Generation")
 * splits every layer of a cell into a producer step P_{s,l} (Q/K/V
 * projection and RoPE) and a consumer step C_{s,l} (attention and the rest of
 * the block), §4.1 Eq. 8; its runtime hooks in right after the QKV
 * projection and RoPE (App. B.1).  The model is Wan2.1-T2V with random-init
 * weights (§5.3).  The pages do not spell out the block; this library takes
 * the Wan2.1 block (text cross-attention left out), for each active cell s:
 *
 *   a   = LN(x) (1 + scale1_s) + shift1_s                  (LN: no affine)
 *   qkv = a W_qkv^T + b_qkv;  q = RMSNorm(q) g_q;  k = RMSNorm(k) g_k
 *   o   = the round's attention of layer l (wf_kv_publish + wf_wave_attention)
 *   x  += gate1_s (o W_o^T + b_o)
 *   a2  = LN(x) (1 + scale2_s) + shift2_s
 *   x  += gate2_s (GELU_tanh(a2 W_1^T + b_1) W_2^T + b_2)
 *
 * with C = n_heads * head_dim channels, F = ffn_dim, both norms over all C
 * channels with the same epsilon.
 *
 * Numerics: x stays fp32; a, a2, qkv, q, k, v, o and the FFN hidden
 * activation are rounded to bf16 (round to nearest even) where they are
 * stored; every product accumulates in fp32 on the matrix cores.
 *
 * Layouts (row-major; "row" = one token of one cell, cells by stage):
 *   x       [S+1][N][C] fp32, in/out; rows of inactive stages untouched
 *   mod     per layer [S+1][6][C] fp32: shift1, scale1, gate1, shift2,
 *           scale2, gate2 of the cell at each stage
 *   weights per layer, nn.Linear convention (W is [out][in], y = x W^T + b):
 *           w_qkv [3C][C] bf16 (rows: q channels, then k, then v),
 *           b_qkv [3C] fp32, g_q, g_k [C] fp32, w_o [C][C] bf16, b_o [C]
 *           fp32, w_1 [F][C] bf16, b_1 [F] fp32, w_2 [C][F] bf16, b_2 [C] fp32
 *   work    caller-owned device scratch of wf_dit_workspace_bytes() bytes
 *           (activations of one layer plus the GEMM library's workspace)
 *
 * Pages: any page type of a bf16-activation round -- WF_BF16, WF_FP8 (FP8
 * keys and values, App. C.6) or WF_FP8K (FP8 keys, bf16 values: the 8-bit
 * Q K^T tier, App. B.1 / App. C.2 Tab. 4, whose "Sage" configuration keeps
 * the linear layers in bf16 as this block does).  The attention then runs
 * that page type's kernel; everything else is unchanged.
 *
 * Ownership and errors follow wf.h.  One difference: the first call on a
 * handle creates a hipBLASLt handle (its own small host and device state,
 * freed by wf_destroy); the products run through hipBLASLt, every other step
 * through this library's kernels.  fp32 rounds have no block
 * (WF_EUNSUPPORTED); C must be a multiple of 8 and at most 8192.
 */
#ifndef WF_DIT_H
#define WF_DIT_H

#include "wf.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int32_t ffn_dim;   /* FFN hidden width F (> 0, multiple of 8) */
  int32_t reserved;
  double eps;        /* LN and RMSNorm epsilon; 0 selects 1e-6 */
} wf_dit_config;

typedef struct {     /* one layer's weights: device pointers, layouts above */
  const void* w_qkv;
  const void* b_qkv;
  const void* g_q;
  const void* g_k;
  const void* w_o;
  const void* b_o;
  const void* w_1;
  const void* b_1;
  const void* w_2;
  const void* b_2;
} wf_dit_weights;

/* Bytes of the `work` buffer wf_dit_layer / wf_dit_round need for this
 * handle's config and `dc`.  WF_EINVAL for a NULL pointer or a bad dc. */
wf_status wf_dit_workspace_bytes(const wf_handle* h, const wf_dit_config* dc, size_t* bytes);

/* Layer `layer` of the round's DiT forward for every active cell, in place
 * on x (the block above).  Runs this layer's wf_kv_publish and
 * wf_wave_attention internally, so the same ordering rules apply: the plan
 * must be the handle's next round (WF_EORDER), wf_round_commit ends the
 * round after every layer has run, and calls on one handle must run one
 * after another on the device (one stream, or ordered by events), because
 * their attention shares the handle's split scratch and their products the
 * one work buffer.  `mod` is this layer's [S+1][6][C].
 * Everything is enqueued on `stream`.  WF_ESMALL if work_bytes is below
 * wf_dit_workspace_bytes; WF_EINVAL for NULL or misaligned (16-byte)
 * pointers; WF_EDEVICE if a launch or a hipBLASLt call fails. */
wf_status wf_dit_layer(wf_handle* h, const wf_plan* plan, int32_t layer,
                       const wf_dit_config* dc, const wf_dit_weights* w,
                       const void* d_mod, void* d_x, void* d_work, size_t work_bytes,
                       void* stream);

/* The whole round: wf_dit_layer for l = 0..L-1 (weights w[l], modulation
 * d_mod + l [S+1][6][C]), then wf_round_commit. */
wf_status wf_dit_round(wf_handle* h, const wf_plan* plan, const wf_dit_config* dc,
                       const wf_dit_weights* w, const void* d_mod, void* d_x,
                       void* d_work, size_t work_bytes, void* stream);

/* For callers that time the block or run it for long (benchmarks, serving
 * warm-up): times the hipBLASLt heuristic's first WF_DIT_TUNE_CANDIDATES
 * algorithms for each of the block's four products (QKV, output, FFN1,
 * FFN2) at the full-width shape, (S + 1) N rows, on the caller's buffers
 * (layer 0's weights w[0]; the work buffer's contents are overwritten), and
 * keeps the fastest for later products of that shape on this handle; other
 * shapes (fill and drain rounds) keep the heuristic's first choice.  Unlike
 * every other call it synchronises `stream` (it reads HIP events).  Outputs
 * then differ from the untuned block only by the products' rounding order.
 * Errors as wf_dit_layer; WF_EDEVICE if a product or an event fails. */
#define WF_DIT_TUNE_CANDIDATES 8
wf_status wf_dit_tune(wf_handle* h, const wf_dit_config* dc, const wf_dit_weights* w,
                      void* d_work, size_t work_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* WF_DIT_H */
