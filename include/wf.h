/*
 * wf.h -- C ABI of the MI355X (gfx950) wavefront-round library.
 *
 * One call sequence runs one round of Wave Forcing's chunk-wise causal
 * attention ("Wave Forcing: Towards Speed-of-Light Streaming Video
 * Generation", arXiv 2611.00859; cited below as WF):
 *
 *   wf_round_plan      which cells are active, which key pages each query
 *                      group reads and in which order, which slot every page
 *                      lives in                      (WF §3.1 Eq. 3-5, App. B.3)
 *   wf_kv_publish      per layer: 3D-RoPE on q and k, K/V written straight into
 *                      their fixed attention slots  (WF §4.1 Eq. 8, App. B.2 Eq. 13)
 *   wf_wave_attention  per layer: every active group attends to its ordered
 *                      context under M_WF(s,j) = 1[j >= s] in one launch
 *                                                    (WF §3.1 Eq. 4-5, §4.2 Eq. 10)
 *   wf_round_commit    store page promoted to history, round counter advanced
 *                                                    (WF App. B.3)
 *   wf_round           all layers (publish, attention) then commit
 *
 * Conventions
 *   - Every call returns a wf_status; 0 is success, negative is an error.
 *     Nothing is thrown across the ABI.  wf_last_error() gives a
 *     thread-local human-readable detail for the last failing call.
 *   - All validation happens before any device work; a failing call has
 *     launched nothing.  Errors of asynchronous device execution surface at
 *     the caller's next synchronisation.
 *   - The caller owns all device memory (inputs, outputs, the slot pool,
 *     the anchor store and the RoPE tables) and the stream.  The library
 *     never allocates device memory and never synchronises the stream.  The
 *     handle holds host state only.  Device pointers must stay valid until
 *     the stream work that uses them has completed.
 *   - Streams are passed as `void*` holding a hipStream_t (NULL = the null
 *     stream), so this header needs no HIP headers.
 *   - Chunk, stage and layer indices are zero-based (WF numbers layers from
 *     one; App. B.8 "Index conventions").
 *   - Stage S is the store cell (k - S, S); stages 0..S-1 are denoising.
 *
 * Device layouts (element type = dtype: fp32 or bf16, bf16 for FP8; D = head_dim,
 * H = n_heads, N = tokens per chunk = F * Hh * Ww, token n at frame
 * n / (Hh Ww), row (n / Ww) % Hh, column n % Ww):
 *   q, k, v, q_rot, out   per layer [S+1][N][H][D], indexed by stage; the
 *                         store is stage S; rows of inactive stages are
 *                         neither read nor written.  wf_round takes
 *                         [L][S+1][N][H][D].
 *   page                  one chunk's keys and values for one layer:
 *                         K  [H][N][D]   (RoPE applied)
 *                         Vt [H][D][N]   (values, transposed: keys contiguous)
 *                         page_elems = 2 * H * N * D.
 *   pool                  [L][n_slots] pages, n_slots = 4 + max(W, W_store) + 2 S.
 *   anchor_raw            [L] pages holding chunk 0's unrotated K and its Vt.
 *   tables                written by wf_bind: the frame-axis frequencies
 *                         theta^(-m/nt) in fp64, then fp32 cos/sin pairs of
 *                         the row and column axes, rounded up to 256 bytes
 *                         (the frame-axis angles are computed on the device
 *                         from the absolute frame, so no table grows with the
 *                         request), then (bf16, FP8, FP8K) the attention's
 *                         split scratch: 4 x ([N][H][D] + [N][H][2]) fp32,
 *                         the partial results of at most two split groups.
 *
 * FP8 pages (dtype WF_FP8; WF App. C.6 Eq. 20-21: K/V in 8 bits halve the
 * payload).  q, k, v, q_rot, out and anchor_raw are bf16 as above; a pool
 * page holds, with Npad = 64 T, T = ceil(N / 64):
 *                         K8  [H][Npad][D]  E4M3 codes of RoPE(k) / 2^eK
 *                         Vt8 [H][D][Npad]  E4M3 codes of v / 2^eV
 *                         codes [H][T][2]   per 64-token tile: eK + 127, eV + 127
 *                         rounded up to 256 bytes.  E4M3 is the OCP format
 *                         (bias 7, max 448, no infinities), rounded to
 *                         nearest even; e is the smallest integer with
 *                         amax(tile) <= 448 * 2^e (0 for an all-zero tile).
 *                         Tokens N..Npad-1 are zero and never attended.
 *                         Attention quantises each bf16 q_rot row times
 *                         c = scale * log2(e) (fp32 product) the same way
 *                         (one exponent per row) and multiplies on the FP8
 *                         matrix cores; the softmax weights are
 *                         rounded to E4M3 for the PV product and the row
 *                         sum adds the same rounded weights.
 *
 * 8-bit QK^T pages (dtype WF_FP8K; WF App. B.1 and App. C.2 Tab. 4: an
 * approximate compute mode swaps self-attention for SageAttention, which
 * multiplies Q K^T in 8 bits and P V in higher precision): the FP8 page
 * layout with the values kept in bf16:
 *                         K8  [H][Npad][D]  E4M3 codes of RoPE(k) / 2^eK
 *                         Vt  [H][D][Npad]  bf16 values, keys padded with 0
 *                         codes [H][T][2]   eK + 127, 127 (values unscaled)
 *                         rounded up to 256 bytes.  Attention quantises the
 *                         query rows as for FP8 pages and multiplies Q K^T on
 *                         the FP8 matrix cores, P V on the bf16 matrix cores
 *                         (softmax weights rounded to bf16, row sum of the
 *                         same rounded weights).
 */
#ifndef WF_H
#define WF_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define WF_MAX_STAGES 8                     /* S <= 8 denoising stages     */
#define WF_MAX_GROUPS (WF_MAX_STAGES + 1)   /* + the store                 */
#define WF_MAX_PAGES 48                     /* key pages per query group   */
#define WF_MAX_SPLIT 2                      /* split query groups per launch */

typedef enum {
  WF_OK = 0,
  WF_EINVAL = -1,       /* bad argument, config or pointer                  */
  WF_ERANGE = -2,       /* round index outside [0, n_chunk + S) (unbounded:
                           F (k + 1) > max_frames)                          */
  WF_EORDER = -3,       /* plan not for this handle / not the next round /
                           attention before publish / commit before publish */
  WF_ESMALL = -4,       /* a caller buffer is smaller than required         */
  WF_EDEVICE = -5,      /* a HIP call or kernel launch failed               */
  WF_EUNSUPPORTED = -6  /* valid config without a kernel instance           */
} wf_status;

typedef enum {
  WF_F32 = 0,   /* everything fp32                                           */
  WF_BF16 = 1,  /* everything bf16 (fp32 accumulation)                       */
  WF_FP8 = 2,   /* bf16 tensors, FP8 E4M3 pages (see "FP8 pages" above)      */
  WF_FP8K = 3   /* bf16 tensors, FP8 keys and bf16 values (8-bit QK^T tier)  */
} wf_dtype;

typedef enum {
  WF_MASK_WAVE = 0,    /* M_WF(s,j) = 1[j >= s]                 (WF §3.1 Eq. 4) */
  WF_MASK_ROLLING = 1  /* every active denoising chunk reads every other one
                          (Rolling Forcing's window, WF §3.1; comparison only) */
} wf_mask;

typedef enum {
  WF_SPLIT_AUTO = 0,   /* split groups when the launch's modelled time drops  */
  WF_SPLIT_OFF = 1,    /* every group is one run over its whole context       */
  WF_SPLIT_FORCE = 2   /* always split the two longest groups (>= 2 pages)    */
} wf_split_mode;

typedef enum {
  WF_KIND_ANCHOR = 0,  /* first clean chunk, persistent            (App. B.3) */
  WF_KIND_HISTORY = 1, /* bounded clean history                    (Eq. 5)    */
  WF_KIND_STORE = 2,   /* live store page of this round            (Eq. 5)    */
  WF_KIND_DENOISE = 3  /* denoising chunk of this round            (Eq. 5)    */
} wf_kind;

/* Round shape.  All fields are read by wf_create; the handle keeps a copy. */
typedef struct {
  int32_t S;          /* denoising steps; round width is S + 1 (WF §2 Eq. 2)  */
  int32_t W;          /* clean-history pages a denoising query reads           */
  int32_t W_store;    /* history pages the store reads; -1 = W + S, i.e. the
                         same (W + S + 2)-chunk context budget as stage 0      */
  int32_t anchor;     /* 1 = keep chunk 0 as persistent anchor, 0 = none       */
  int32_t n_chunk;    /* chunks in the request (>= 1); rounds = n_chunk + S.
                         <= 0: an unbounded request (a stream, WF §1 and
                         App. B.8): every chunk k >= 0 is admitted in round k,
                         no drain until wf_finish_stream                      */
  int32_t F, Hh, Ww;  /* latent frames per chunk, token rows, token columns    */
  int32_t n_heads;    /* H                                                    */
  int32_t head_dim;   /* D (even, >= 6)                                       */
  int32_t n_layers;   /* L                                                    */
  int32_t dtype;      /* wf_dtype of q/k/v/q_rot/out and of the pages          */
  int32_t mask;       /* wf_mask                                              */
  int32_t max_frames; /* unbounded requests: the latent frames the stream may
                         reach, in [F, 2^30] (round k needs F (k + 1) <=
                         max_frames); bounded requests: 0.  No buffer depends
                         on it: attention storage is the same slot ring.     */
  double rope_theta;  /* RoPE base; 0 selects 10000                            */
  double softmax_scale; /* 0 selects 1/sqrt(head_dim)                          */
} wf_config;

/* One cell (k - stage, stage) of the round. */
typedef struct {
  int32_t stage;
  int32_t chunk;   /* k - stage, or -1 when inactive                           */
  int32_t active;  /* 1 if 0 <= chunk < n_chunk                                */
  int32_t slot;    /* slot its K/V page is published into, or -1              */
  int32_t frame0;  /* first latent-frame position F * chunk, or -1            */
} wf_cell;

/* Ordered context of the query group of one stage (WF §3.1 Eq. 5). */
typedef struct {
  int32_t stage;
  int32_t n_pages;                 /* 0 when the cell is inactive            */
  int32_t slot[WF_MAX_PAGES];      /* pool slot of each page, context order  */
  int32_t chunk[WF_MAX_PAGES];     /* logical chunk id of each page          */
  int32_t kind[WF_MAX_PAGES];      /* wf_kind of each page                   */
} wf_group;

typedef struct {
  int32_t present;  /* anchor page is read this round (k > S, anchor on)      */
  int32_t slot;     /* k mod 2 when present, else -1                          */
  int32_t frame0;   /* frame position the anchor key is rotated to, or -1     */
  int32_t capture;  /* 1 in round S: chunk 0's raw K/V is saved               */
} wf_anchor;

/* Plain-old-data plan of one round; a pure function of (config, k). */
typedef struct {
  int64_t k;
  uint64_t config_hash;            /* identifies the config it was made for  */
  int32_t S;
  int32_t n_active;                /* active cells, store included           */
  wf_cell cells[WF_MAX_GROUPS];    /* index = stage                          */
  wf_group groups[WF_MAX_GROUPS];  /* index = query stage                    */
  wf_anchor anchor;
  int32_t evict_chunk;             /* leaves the retained window after the
                                      round's store is promoted, or -1       */
  int32_t reserved;
  int64_t kv_tokens;               /* key tokens summed over groups, 1 layer */
  double flops;                    /* attention flops, all layers: 4 N D H
                                      per key token (QK^T and PV)            */
  double publish_bytes;            /* publish HBM bytes, all layers          */
} wf_plan;

/* Where a config's data lives in the caller's buffers (sizes in bytes).
 * The slot ring (WF App. B.2 Eq. 13: fixed, double-buffered attention slots)
 * and the page formats are the library's; callers that look inside pages
 * (tests, debuggers) read the numbers here instead of re-deriving them. */
typedef struct {
  int64_t n_slots;               /* pool slots per layer                     */
  int64_t page_bytes;            /* one slot of one layer                    */
  int64_t pool_bytes;            /* n_layers * n_slots * page_bytes          */
  int64_t anchor_page_bytes;     /* one layer's raw anchor K and Vt          */
  int64_t anchor_bytes;          /* n_layers * anchor_page_bytes             */
  int64_t tokens;                /* N = F * Hh * Ww                          */
  int64_t tokens_padded;         /* token rows per page head: 64 * tiles on
                                    FP8 / FP8K pages, N otherwise           */
  int64_t tiles;                 /* ceil(N / 64): scale-code tiles per head  */
  int64_t vt_offset;             /* Vt inside a page (K starts at 0)         */
  int64_t codes_offset;          /* scale codes inside a page, -1 if none    */
  int64_t table_bytes;           /* RoPE tables + split scratch              */
  int64_t split_scratch_offset;  /* split scratch inside the table buffer    */
  int64_t split_scratch_bytes;   /* 0 for fp32 configs (they never split)    */
} wf_layout;

typedef struct wf_handle wf_handle;

/* Text for a status code (static storage); any int32 is accepted. */
const char* wf_strerror(int32_t status);

/* Detail of the last failing call on this thread ("" if none). */
const char* wf_last_error(void);

/* Validate `cfg` and create a handle (host memory only; no device calls).
 * WF_EINVAL for an invalid config or a NULL pointer. */
wf_status wf_create(const wf_config* cfg, wf_handle** out);

/* Free a handle (NULL is ignored).  Device memory stays the caller's. */
void wf_destroy(wf_handle* h);

/* Bytes the caller must allocate for the slot pool, the anchor store and
 * the RoPE tables of `cfg` (the table buffer also holds the attention's
 * split scratch, see "tables" above).  Any output pointer may be NULL. */
wf_status wf_pool_bytes(const wf_config* cfg, size_t* pool_bytes,
                        size_t* anchor_bytes, size_t* table_bytes);

/* The layout of `cfg`'s buffers and pages (host only, no device calls).
 * WF_EINVAL for an invalid config or a NULL pointer. */
wf_status wf_page_layout(const wf_config* cfg, wf_layout* out);

/* Attach caller-owned device buffers and upload the RoPE tables (computed
 * on the host in fp64, stored as fp32) with a synchronous copy.  Sizes are
 * checked first (WF_ESMALL), then kernel support for the config
 * (WF_EUNSUPPORTED: bf16 needs head_dim 64 or 128, N % 8 == 0, N >= 64 and
 * one layer's slots below 4 GiB; FP8 and FP8K need head_dim 128, N % 8 == 0,
 * one layer's slots below 4 GiB and (1 + max(W, W_store) + 1 + S) * T <= 4096;
 * fp32 needs head_dim % 4 == 0, head_dim <= 128 and N % 4 == 0).  Buffers
 * must be 16-byte aligned.  The handle keeps the pointers, not the memory. */
wf_status wf_bind(wf_handle* h, void* d_pool, size_t pool_bytes,
                  void* d_anchor_raw, size_t anchor_bytes,
                  void* d_tables, size_t table_bytes);

/* Plan round k (host only, no device calls; valid before wf_bind).
 * WF_ERANGE if k is outside [0, n_chunk + S), or for an unbounded request if
 * F (k + 1) > max_frames.  An unbounded request's plan of round k equals the
 * plan of a bounded request of any n_chunk > k (its config hash aside). */
wf_status wf_round_plan(const wf_handle* h, int64_t k, wf_plan* out);

/* Round index the handle expects next (0 after create / reset). */
wf_status wf_next_round(const wf_handle* h, int64_t* k);

/* End an unbounded request (WF §1: the stream stops): it becomes the
 * bounded request of n_chunk chunks, whose rounds next..n_chunk + S - 1
 * admit the remaining chunks and drain the pipeline (App. B.3).  n_chunk
 * must be at least the next round (every chunk admitted so far stays) and
 * F n_chunk <= 2^30; the handle's config then has n_chunk set and
 * max_frames 0, so plans of the following rounds are those of that bounded
 * request, hash included (plans made before the call are rejected).  Call it
 * between rounds (WF_EORDER once a layer of the next round is published).
 * Buffers stay bound: their sizes do not depend on n_chunk.  WF_EINVAL for a
 * bounded handle or an n_chunk out of range.  Host only. */
wf_status wf_finish_stream(wf_handle* h, int64_t n_chunk);

/* Start a new request at round 0.  Page contents become meaningless. */
wf_status wf_reset(wf_handle* h);

/* Layer `layer` of the round's producer step (WF §4.1 Eq. 8 P_{s,l}, App.
 * B.2 Eq. 13): for every active cell, q_rot = RoPE3D(q), the cell's page
 * slot gets K = RoPE3D(k) and Vt = v^T.  In round S the store cell's raw k
 * and v^T are also kept in anchor_raw; when the anchor is present its slot
 * gets RoPE3D(anchor K, anchor position) and the anchor Vt.
 * d_q/d_k/d_v: this layer's [S+1][N][H][D] inputs (read only);
 * d_q_rot: this layer's [S+1][N][H][D] output.  Enqueued on `stream`.
 * WF_EORDER if the plan is not the handle's next round or was made for
 * another config; WF_EINVAL if unbound or a pointer is NULL. */
wf_status wf_kv_publish(wf_handle* h, const wf_plan* plan, int32_t layer,
                        const void* d_q, const void* d_k, const void* d_v,
                        void* d_q_rot, void* stream);

/* Layer `layer` of the round's attention (WF §3.1 Eq. 4-5): for every
 * active query group g and head, out = softmax(scale * Q K^T) V over the
 * group's key pages concatenated in plan order.  One launch covers all
 * groups, followed by one merge launch when groups are split (see
 * wf_set_attention_split).  d_q_rot: [S+1][N][H][D] from wf_kv_publish;
 * d_out: [S+1][N][H][D].
 * WF_EORDER if this layer was not published in this round.
 * Numerics (bf16): the kernel multiplies each bf16 q_rot row by
 * scale * log2(e) and rounds the product to bf16 again (the scores then come
 * out in base-2 units), so every score carries two bf16 roundings of q and
 * one of K: its error grows with the score's magnitude (about 2^-8 of it per
 * rounding), not only with the output's.  fp32 accumulation; the softmax
 * weights are rounded to bf16 for the P V product and the row sum alike.
 * Stream order: every attention call of a handle (of any layer and round,
 * and wf_dit_layer's, which calls this) uses the one split scratch of the
 * handle's table buffer unless the handle's split mode is WF_SPLIT_OFF or
 * its dtype is WF_F32.  Such calls must therefore run one after another on
 * the device: enqueue them on one stream, or order them with events.  Two
 * of them in flight at once on different streams overwrite each other's
 * partial results.  Publishes need no such order among themselves. */
wf_status wf_wave_attention(wf_handle* h, const wf_plan* plan, int32_t layer,
                            const void* d_q_rot, void* d_out, void* stream);

/* Bytes of the library's static split scratch (wf_wave_attention_noalloc). */
#define WF_STATIC_SCRATCH_BYTES (128u << 20)

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * wf_wave_attention with the split groups' partial results kept in a static
 * device array of the library (WF_STATIC_SCRATCH_BYTES = 128 MiB, held by
 * every GPU the library runs on until the process ends) instead of the
 * handle's table buffer.  Arguments, results, validation and stream-order
 * rules are those of wf_wave_attention; the call allocates nothing (the
 * array's device address is looked up once per device, on the first call
 * with that device current).  Every call on one GPU, from any handle,
 * shares that GPU's one array and leaves its partial results there, so two
 * such calls in flight at once on one GPU (different streams, handles or
 * threads) race: order them.  Split groups need 2 (N H D + 2 N H) * 4
 * bytes each: under WF_SPLIT_AUTO the choice is made among the splits whose
 * partial results fit the array (none at the 14B class), so it can differ
 * from wf_wave_attention's; WF_ESMALL, before any launch, when a forced
 * split (WF_SPLIT_FORCE) needs more than WF_STATIC_SCRATCH_BYTES.
 * WF_SPLIT_OFF needs none.  WF_EDEVICE if the array's address cannot be
 * found. */
wf_status wf_wave_attention_noalloc(wf_handle* h, const wf_plan* plan, int32_t layer,
                                    const void* d_q_rot, void* d_out, void* stream);

/* How wf_wave_attention divides its work (bf16, FP8 and FP8K rounds; fp32
 * rounds never split).  A launch runs one work-group per (group, head, 256
 * query rows), each over the group's whole context, so the launch ends with
 * a tail in which the shortest groups' work-groups leave compute units idle.
 * A split group instead runs as two halves over pages [0, n/2) and [n/2, n)
 * of its context; each half leaves its unnormalised output, exponent offset
 * and weight sum in the split scratch (see "tables" above), and a second
 * launch merges the two softmax partials exactly (WF §4.2 gives the per-
 * stage key counts that make the groups' lengths unequal).  WF_SPLIT_AUTO
 * (the default) models the launch as work-groups taken longest first by
 * the device's compute units and splits the at most WF_MAX_SPLIT groups
 * that minimise that model's end time plus the merge; the choice is cached
 * per list of group lengths.  WF_SPLIT_FORCE splits the two longest groups
 * (>= 2 pages).  Results of the modes agree up to rounding.
 * WF_EINVAL for a NULL handle or an unknown mode.  Host only. */
wf_status wf_set_attention_split(wf_handle* h, int32_t mode);

/* The split wf_wave_attention makes for `plan` under the handle's split
 * mode (see wf_set_attention_split; wf_wave_attention_noalloc chooses among
 * the splits its static array holds): *n_split groups (0..WF_MAX_SPLIT);
 * group i is query stage stage[i], run as pages [0, at[i]) and
 * [at[i], n) of its context (at[i] = n/2).  stage and at have room for
 * WF_MAX_SPLIT entries; entries past *n_split are left untouched.  The
 * model uses the compute-unit count of the device current at wf_bind (256
 * before).
 * WF_EINVAL for a NULL argument or a modified plan; WF_EORDER for a plan
 * of another config; WF_ERANGE for a round outside the request.  Host only
 * (needs no bound pool). */
wf_status wf_attention_split_choice(wf_handle* h, const wf_plan* plan, int32_t* n_split,
                                    int32_t* stage, int32_t* at);

/* End the round (WF App. B.3): requires every layer published; advances
 * the expected round.  Host only: the store page is promoted in place. */
wf_status wf_round_commit(wf_handle* h, const wf_plan* plan);

/* Whole round: for l = 0..L-1 publish(l) then attention(l), then commit.
 * d_q/d_k/d_v/d_q_rot/d_out are [L][S+1][N][H][D]. */
wf_status wf_round(wf_handle* h, const wf_plan* plan,
                   const void* d_q, const void* d_k, const void* d_v,
                   void* d_q_rot, void* d_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* WF_H */
