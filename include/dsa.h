/*
 * dsa.h - C ABI of the MI355X (gfx950) DeepSeek Sparse Attention layer hot path.
 *
 * The layer, per query row t of request b that sees the candidates s in [0, n_t):
 *   1. lightning-indexer scores  I(t,s) = index_scale * sum_j w[t,j] * max(0, q_idx[t,j,:] . k[s,:])
 *      (the scoring stage of tokenspeed PR 627 "Add gluon kernel for DSA"; the pages name the
 *      stage and its index_k_cache input but print no formula, so this is the DeepSeek
 *      lightning indexer read plainly);
 *   2. per-row top-k: the min(topk, n_t) best positions, -1 padding, and a lens count (the
 *      (out, lens_out) pair of the decode top-k wrapper in the review of PR 627);
 *   3. sparse absorbed-MLA attention over the selected latent rows (512 latent + 64 RoPE bf16
 *      rows of tokenspeed PR 664 "gfx950 Gluon bf16 MLA decode and prefill kernels"; fp8 rows
 *      of aiter PR 4382 "Paged Sparse Attention Gluon Kernel"), with -1 entries masked
 *      (radixark/miles PR 3608, section "What", padding bullet).
 *
 * Conventions shared by every entry point:
 *  - Every data pointer is DEVICE memory owned by the caller (descriptor structs themselves are
 *    host memory, read during the call). The library never allocates, frees or synchronises;
 *    it never reads device data on the host, so calls can be captured in a HIP graph.
 *  - `stream` is a hipStream_t passed as void*. Every call enqueues its kernels on it and
 *    returns; a non-OK status means nothing was enqueued (except DSA_ERR_HIP, raised after a
 *    failed launch).
 *  - Argument checks run on the host before any HIP call: null pointers, non-positive sizes,
 *    strides smaller than a row, pointers or row strides that break 16-byte alignment give
 *    DSA_ERR_ARG; shapes outside the compiled envelope give DSA_ERR_UNSUPPORTED (never a
 *    fallback to another implementation).
 *  - Strides (ld_*) are in ELEMENTS between consecutive query rows; inner dimensions are dense.
 *  - Device-side contract (not checkable on the host without a sync): row_len[t] <= n_max,
 *    row_req[t] < n_req, every listed position < n_t's request length, every page id addresses
 *    a page inside the cache. Kernels clamp page ids and slots into the cache, so a broken
 *    contract gives wrong numbers, never an out-of-bounds access.
 *  - Workspace: entries that need scratch take (workspace, ws_bytes). Size it with
 *    dsa_workspace_size() and initialise it ONCE with dsa_workspace_init(); each entry leaves
 *    its control words zeroed on return, so the same buffer can be reused by any entry, but
 *    calls that overlap in time on one workspace race. After DSA_ERR_HIP, initialise again.
 */
#ifndef DSA_MI355X_H
#define DSA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dsa_status {
  DSA_OK = 0,
  DSA_ERR_ARG = -1,          /* null pointer, bad shape, bad stride or alignment */
  DSA_ERR_UNSUPPORTED = -2,  /* valid, but outside the compiled envelope; never a fallback */
  DSA_ERR_WORKSPACE = -3,    /* workspace missing or smaller than dsa_workspace_size() */
  DSA_ERR_HIP = -4,          /* a HIP launch failed */
  DSA_ERR_SCRATCH_LIMIT = -5 /* dsa_decode_static: the problem needs more than its static scratch */
} dsa_status;

typedef enum dsa_key_dtype {
  DSA_KEY_BF16 = 0,          /* index keys bf16 [n_slots, di] */
  DSA_KEY_FP8 = 1            /* index keys OCP fp8 e4m3 [n_slots, di] + fp32 scale [n_slots] */
} dsa_key_dtype;

typedef enum dsa_kv_format {
  /* bf16 rows [n_slots, d_nope + d_rope] (GLM: 512 latent + 64 RoPE), PR 664 */
  DSA_KV_BF16 = 0,
  /* fp8 e4m3 rows [n_slots, D] + fp32 scales [n_slots, D/64]; x = fp8 * scale[slot, c/64];
     PR 4382, section "Uniform fp8 pool - 2D" (page_size 1 there: a slot is a token) */
  DSA_KV_FP8_UNIFORM = 1,
  /* packed pages [n_slots/page_size, page_size * 584] bytes, block-planar: page_size x 576
     data bytes (448 NoPE fp8 + 64 RoPE bf16) then page_size x 8 scale bytes (7 UE8M0
     exponents + 1 pad); NoPE x = fp8 * 2^(e-127); PR 4382, "Packed fp8 fp8_ds_mla - 3D" */
  DSA_KV_FP8_DS_MLA = 2,
  /* the uniform layout with fnuz e4m3 bytes (exponent bias 8, largest magnitude 240, 0x80 is
     NaN and is never written); PR 4382, section "fp8 flavors": no native gfx950 conversion,
     so the bytes are decoded by bit placement (exact) */
  DSA_KV_FP8_UNIFORM_FNUZ = 3
} dsa_kv_format;

/* Logical position s of request b -> cache slot.
 * block_table != NULL: slot = block_table[b * bt_stride + s / page_size] * page_size + s % page_size
 *                      (paged cache; page 64 in PR 664, 256 for fp8_ds_mla in PR 4382)
 * block_table == NULL: slot = req_base[b] + s (packed sequences back to back). */
typedef struct dsa_paging {
  int32_t page_size;
  int32_t _pad0;
  const int32_t* block_table;  /* device int32, or NULL */
  int64_t bt_stride;           /* elements between requests' table rows (>= pages used) */
  const int32_t* req_base;     /* device int32 [n_req]; used when block_table == NULL */
} dsa_paging;

typedef struct dsa_key_cache {
  int32_t dtype;               /* dsa_key_dtype */
  int32_t _pad0;
  const void* data;            /* device [n_slots, di] */
  const float* scale;          /* device fp32 [n_slots] (DSA_KEY_FP8 only, else NULL) */
  int64_t n_slots;
  dsa_paging paging;
} dsa_key_cache;

typedef struct dsa_kv_cache {
  int32_t format;              /* dsa_kv_format */
  int32_t d_nope;              /* bf16: 512; fp8 formats: NoPE width (448 for fp8_ds_mla) */
  int32_t d_rope;              /* 64 */
  int32_t _pad0;
  const void* data;            /* device, layout per format (see dsa_kv_format) */
  const float* scales;         /* device fp32 [n_slots, D/64] for DSA_KV_FP8_UNIFORM, else NULL */
  int64_t n_slots;             /* tokens the cache holds (pages * page_size for paged caches) */
  dsa_paging paging;
} dsa_kv_cache;

/* Query rows. Row t belongs to request row_req[t] (row_req == NULL: request t) and sees
 * positions [0, row_len[t]). Decode: one row per request, row_len = context length.
 * Causal prefill of packed segments: the row at segment position p has row_len = p + 1
 * (diagonal included) and never sees another segment (PR 3608, "Correctness": packed
 * sequences end to end, 1-token segments). */
typedef struct dsa_rows {
  int32_t T;                   /* number of rows (>= 0) */
  int32_t n_req;               /* number of requests (rows of block_table / req_base) */
  const int32_t* row_req;      /* device int32 [T] or NULL */
  const int32_t* row_len;      /* device int32 [T] */
  int32_t n_max;               /* host: an upper bound of row_len[t] (sizes grids and buffers) */
  int32_t _pad0;
} dsa_rows;

/* ---------------------------------------------------------------- step 1: indexer scores
 * q_idx: bf16 [T, Hi, di], row stride ld_q_idx elements (>= Hi*di, multiple of 8).
 * w:     fp32 [T, Hi], row stride ld_w (>= Hi); any sign.
 * logits: fp32 [T, ld_logits], ld_logits >= n_max; writes logits[t, 0:n_t],
 *         leaves [n_t, ld_logits) untouched.
 * Envelope: 1 <= Hi <= 64, di in {64, 128}. */
dsa_status dsa_index_scores(const void* q_idx, int64_t ld_q_idx, const float* w, int64_t ld_w,
                            const dsa_key_cache* keys, const dsa_rows* rows, int32_t Hi,
                            int32_t di, float index_scale, float* logits, int64_t ld_logits,
                            void* stream);

/* ---------------------------------------------------------------- step 2: top-k
 * Reads logits[t, 0:n_t]. Writes indices[t, 0:topk] (int32, stride ld_idx >= topk): the
 * positions of the min(topk, n_t) largest scores (ties: smaller position first, so the set is
 * deterministic), in unspecified order, then -1 padding; lens[t] = min(topk, n_t).
 * Envelope: 1 <= topk <= 65536. Uses the workspace. */
dsa_status dsa_topk(const float* logits, int64_t ld_logits, const dsa_rows* rows, int32_t topk,
                    int32_t* indices, int64_t ld_idx, int32_t* lens, void* workspace,
                    size_t ws_bytes, void* stream);

/* Attention options (NULL everywhere means: no sink, natural-log lse). DeepSeek-V4's forward
 * hands its backward an lse in base 2 with an attention sink folded in (radixark/miles PR
 * 3608, section "What", forward bullet). The sink is one logit per head, in the units of
 * softmax_scale * q . c, that joins the softmax denominator and carries no value row:
 *   out[t,h] = sum_i e^(l_i) c_i[0:d_v] / (e^(sink[h]) + sum_i e^(l_i)),
 *   lse[t,h] = ln(e^(sink[h]) + sum_i e^(l_i))   (a row with no listed entry: out 0, lse sink[h]).
 * sink: device fp32 [H] or NULL (a -inf entry is no sink for that head).
 * lse_log2: 0 = natural log, 1 = base 2 (lse / ln 2; -inf stays -inf). Other values: DSA_ERR_ARG. */
typedef struct dsa_attn_opts {
  const float* sink;
  int32_t lse_log2;
  int32_t _pad0;
} dsa_attn_opts;

/* ---------------------------------------------------------------- step 3: sparse MLA
 * q:   bf16 [T, H, d_qk], row stride ld_q (>= H*d_qk, multiple of 8).
 * idx: int32 [T, n_idx] positions (stride ld_idx) into `kv` for the row's request; -1 = none.
 * extra_kv/extra_idx (may be NULL, n_extra = 0): a second list into a second cache; the row's
 *      softmax runs over the union of both lists (PR 4382, two-loop SWA + top-k layout).
 * out: bf16 [T, H, d_v], row stride ld_out (>= H*d_v, multiple of 8):
 *      out[t,h] = sum_i softmax_i(softmax_scale * q[t,h] . c_i) * c_i[0:d_v]; rows with no
 *      listed entry give out = 0.
 * lse: fp32 [T, H] natural-log logsumexp of the scaled logits (-inf for empty rows); may be NULL.
 * opts: sink and lse base (see dsa_attn_opts); may be NULL.
 * Envelope: H >= 1 (heads run in tiles of 16; in a partial tile the missing heads are read
 * as zero and nothing is written for them, so H = 8, a TP=8 share of 64 heads, costs one tile);
 * d_qk = d_nope + d_rope in {512, 576}; d_v = 512; both caches of the same format. The decode entry splits each row's list over workgroups and merges the
 * partials (PR 664 split-KV + LSE merge); the prefill entry gives each row one workgroup. */
dsa_status dsa_sparse_mla_decode(const void* q, int64_t ld_q, const dsa_kv_cache* kv,
                                 const int32_t* idx, int64_t ld_idx, int32_t n_idx,
                                 const dsa_kv_cache* extra_kv, const int32_t* extra_idx,
                                 int64_t ld_extra, int32_t n_extra, int32_t B, int32_t H,
                                 int32_t d_qk, int32_t d_v, float softmax_scale, void* out,
                                 int64_t ld_out, float* lse, const dsa_attn_opts* opts,
                                 void* workspace, size_t ws_bytes, void* stream);

dsa_status dsa_sparse_mla_prefill(const void* q, int64_t ld_q, const dsa_kv_cache* kv,
                                  const int32_t* idx, int64_t ld_idx, int32_t n_idx,
                                  const dsa_kv_cache* extra_kv, const int32_t* extra_idx,
                                  int64_t ld_extra, int32_t n_extra, const dsa_rows* rows,
                                  int32_t H, int32_t d_qk, int32_t d_v, float softmax_scale,
                                  void* out, int64_t ld_out, float* lse,
                                  const dsa_attn_opts* opts, void* workspace, size_t ws_bytes,
                                  void* stream);

/* ---------------------------------------------------------------- backward of step 3
 * The gradient of step 3 for training (radixark/miles PR 3608, section "What": dq, and dKV
 * added atomically through the listed indices; the backward takes the forward's lse with the
 * sink folded in). One list into one bf16 cache. With l_i = softmax_scale * q[t,h] . c_i,
 * p_i = e^(l_i - lse[t,h]) and D = dout[t,h] . out[t,h]:
 *   dq[t,h]      = softmax_scale * sum_i p_i (dout[t,h] . c_i[0:d_v] - D) c_i[0:d_qk]
 *   dkv[slot_i] += softmax_scale * p_i (dout[t,h] . c_i[0:d_v] - D) q[t,h]   (columns 0:d_qk)
 *                + p_i dout[t,h]                                             (columns 0:d_v)
 *   dsink[h]    += -e^(sink[h] - lse[t,h]) D
 * summed over heads and rows; -1 entries contribute nothing, an entry listed twice twice.
 * q, kv, idx, rows: as in dsa_sparse_mla_prefill (rows names each row's request; row_len is
 *      not read). out, lse: the forward's outputs for the same inputs and opts (lse base per
 *      opts->lse_log2; its values are taken as given, so P is recomputed from them).
 * dout: bf16 [T, H, d_v], row stride ld_dout (>= H*d_v, multiple of 8).
 * dq:  fp32 [T, H, d_qk], row stride ld_dq (>= H*d_qk, multiple of 4), 16-byte aligned;
 *      written.
 * dkv: fp32 [kv->n_slots, d_qk] indexed by cache slot; ADDED TO (the caller zeroes it first).
 *      A slot that several entries of the call name (over all rows, or twice in one row)
 *      takes fp32 atomics in no fixed order, so its last bits vary between runs; with the
 *      owner map below, a slot that exactly one entry names takes one plain load and store.
 * dsink: fp32 [H] added to by atomics, or NULL; needs opts->sink.
 * Kernels: per (row, 32 heads, part of the row's list) dq, and P and dZ into the workspace
 * (bf16, 4 bytes per (row, entry, head), plus the entries' slots, and the list parts' dq sums
 * when a row's list is split to fill the GPU); then per row dKV over all heads, so that an
 * entry costs one add per column whatever H is (H <= 16: one kernel, the workspace unused).
 * For 17 <= H <= 64 and a workspace sized with n_slots = kv->n_slots, an owner map (one word
 * per slot, marked by a kernel between the two, cleared again by the dKV kernel) tells the dKV
 * kernel which slots one entry alone names; words found non-zero (a workspace that held other
 * data) only make their slots take atomics. Workspace: dsa_workspace_size(
 * DSA_ENTRY_MLA_BACKWARD, {T, H, n_idx, n_slots}); n_slots = 0 sizes it without the map (every
 * dKV add atomic).
 * Envelope: DSA_KV_BF16 cache; 1 <= H <= 128 (heads padded to 16, 32, 64 or 128 inside, the
 * padding heads reading as zero); d_qk in {512, 576}; d_v = 512.
 * Errors: DSA_ERR_ARG for null pointers, bad strides or alignment, dsink without a sink;
 * DSA_ERR_WORKSPACE for a missing or small workspace; DSA_ERR_UNSUPPORTED outside the envelope. */
dsa_status dsa_sparse_mla_backward(const void* q, int64_t ld_q, const dsa_kv_cache* kv,
                                   const int32_t* idx, int64_t ld_idx, int32_t n_idx,
                                   const dsa_rows* rows, int32_t H, int32_t d_qk, int32_t d_v,
                                   float softmax_scale, const void* out, int64_t ld_out,
                                   const float* lse, const void* dout, int64_t ld_dout,
                                   const dsa_attn_opts* opts, float* dq, int64_t ld_dq,
                                   float* dkv, float* dsink, void* workspace, size_t ws_bytes,
                                   void* stream);

/* ---------------------------------------------------------------- fused layer
 * Steps 1-3 on one stream with no host sync: scores into the workspace, top-k, attention
 * over the selected positions. idx_out / lens_out (nullable) receive the selection as
 * dsa_topk writes it. Same envelopes as the three steps. */
dsa_status dsa_decode(const void* q, int64_t ld_q, const void* q_idx, int64_t ld_q_idx,
                      const float* w, int64_t ld_w, const dsa_key_cache* keys,
                      const dsa_kv_cache* kv, const dsa_rows* rows, int32_t H, int32_t d_qk,
                      int32_t d_v, int32_t Hi, int32_t di, int32_t topk, float index_scale,
                      float softmax_scale, void* out, int64_t ld_out, float* lse,
                      const dsa_attn_opts* opts, int32_t* idx_out, int64_t ld_idx_out,
                      int32_t* lens_out, void* workspace, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- fused layer, no allocation
 * For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): dsa_decode with the same arguments and results,
 * minus the workspace. Its scratch is one static device array of DSA_STATIC_SCRATCH_BYTES
 * that every GPU the library runs on holds until the process ends; the entry never calls
 * hipMalloc, hipFree or any allocating routine. The first call on a device looks up that
 * device's copy of the array and zeroes its control words with a kernel (no memset node);
 * every call leaves them zero, so later calls need no clearing (after DSA_ERR_HIP the next
 * call clears them again).
 * Limits: a problem whose dsa_workspace_size(DSA_ENTRY_DECODE, ...) exceeds
 * DSA_STATIC_SCRATCH_BYTES is rejected with DSA_ERR_SCRATCH_LIMIT before anything is enqueued
 * (64 MiB holds, e.g., one row of 1M candidates, or 64 rows of 32K at topk 2048 and 64 heads).
 * Every call on a GPU shares that GPU's array: calls that overlap in time on one GPU (two
 * streams, two host threads) race and must be serialised by the caller. The device is the
 * stream's (hipStreamGetDevice; the current device for the null stream). */
#define DSA_STATIC_SCRATCH_BYTES (64u << 20)

dsa_status dsa_decode_static(const void* q, int64_t ld_q, const void* q_idx, int64_t ld_q_idx,
                             const float* w, int64_t ld_w, const dsa_key_cache* keys,
                             const dsa_kv_cache* kv, const dsa_rows* rows, int32_t H,
                             int32_t d_qk, int32_t d_v, int32_t Hi, int32_t di, int32_t topk,
                             float index_scale, float softmax_scale, void* out, int64_t ld_out,
                             float* lse, const dsa_attn_opts* opts, int32_t* idx_out,
                             int64_t ld_idx_out, int32_t* lens_out, void* stream);

/* ---------------------------------------------------------------- workspace and errors */
typedef enum dsa_entry {
  DSA_ENTRY_TOPK = 1,
  DSA_ENTRY_MLA_DECODE = 2,
  DSA_ENTRY_MLA_PREFILL = 3,
  DSA_ENTRY_DECODE = 4,
  DSA_ENTRY_MLA_BACKWARD = 5
} dsa_entry;

/* Problem sizes the workspace depends on (unused fields may be 0). */
typedef struct dsa_problem {
  int32_t T;        /* query rows */
  int32_t n_max;    /* max candidates per row */
  int32_t topk;
  int32_t H;        /* attention heads */
  int32_t n_idx;    /* attention list length (main + extra) */
  int32_t n_slots;  /* backward: the cache's slot count for the owner map (0: no map) */
} dsa_problem;

/* Bytes of workspace `entry` needs for problem `p` (0 if it needs none; SIZE_MAX on bad input). */
size_t dsa_workspace_size(int32_t entry, const dsa_problem* p);

/* Zero the workspace once after allocating it (enqueued on `stream`, no memset node). */
dsa_status dsa_workspace_init(void* workspace, size_t ws_bytes, void* stream);

/* Static message for a status code. */
const char* dsa_status_string(int32_t status);

/* ---------------------------------------------------------------- cache writes
 * The step just before the layer: new tokens' rows enter the caches in the layer's formats
 * (aiter PR 4382 "Paged Sparse Attention Gluon Kernel", section "Supported formats &
 * dtypes": the uniform fp8 pool and the packed fp8_ds_mla token; and fp8 index keys with one
 * fp32 scale per token).
 * src:   bf16 rows [n_tok, ld_src], ld_src >= row width and a multiple of 8, 16-byte aligned.
 * slots: device int32 [n_tok], the cache slot of each row (the caller's block-table mapping of
 *        (request, position)); -1 or a slot outside [0, n_slots) skips that row.
 * The cache's data (and scales) must be writable device memory (the descriptors' const is for
 * the read path). Rows with distinct slots may be written by one call; two rows with the same
 * slot race. Rounding (the pages give the layouts only): e4m3 to nearest even after
 * saturating to +-448; fp32 scales = amax / 448 in fp32 (1 for an all-zero group), each value
 * divided by its scale with IEEE division (fnuz pool: 240 in place of 448, and zero of either
 * sign is byte 0x00); fp8_ds_mla exponent byte = k + 127 for the smallest
 * integer k with 448 * 2^k >= amax, clamped to [1, 254] (127 for an all-zero group), values
 * multiplied by 2^-k exactly.
 * dsa_kv_cache_write: DSA_KV_BF16 copies d_nope + d_rope channels; DSA_KV_FP8_UNIFORM takes
 *   D = d_nope + d_rope (a multiple of 64) channels, one scale per 64 (DSA_KV_FP8_UNIFORM_FNUZ
 *   likewise); DSA_KV_FP8_DS_MLA needs
 *   d_nope = 448, d_rope = 64 (exponent pad byte written 0).
 * dsa_key_cache_write: di in {64, 128}; DSA_KEY_BF16 copies, DSA_KEY_FP8 writes e4m3 bytes and
 *   one scale per token.
 * Errors: DSA_ERR_ARG for null pointers, bad strides or alignment, n_tok < 0;
 * DSA_ERR_UNSUPPORTED for shapes outside the list above. */
dsa_status dsa_kv_cache_write(const void* src, int64_t ld_src, int32_t n_tok, const int32_t* slots,
                              const dsa_kv_cache* kv, void* stream);
dsa_status dsa_key_cache_write(const void* src, int64_t ld_src, int32_t n_tok, const int32_t* slots,
                               const dsa_key_cache* keys, int32_t di, void* stream);

/* ABI version (bumped on any signature or struct change). */
int32_t dsa_abi_version(void);

/* ---------------------------------------------------------------- kernel timing
 * Profiling aid (the per-stage timings the pages report, e.g. the scores / top-k / sparse
 * attention columns of PR 627's benchmark tables). While enabled, every kernel the library
 * launches records two HIP events from its own dispatch on the caller's stream, at the
 * kernel's start and end (host-side event objects from a pool; no device memory), so a
 * duration is the kernel's alone. dsa_profile_collect() waits for the recorded events,
 * aggregates them by kernel name into `out` (at most max_entries rows), clears the record
 * and returns the number of rows written (or a negative dsa_status). Not thread-safe;
 * disabled by default. */
typedef struct dsa_kernel_time {
  char name[40];
  int32_t count;
  float total_ms;
  float min_ms;
  float max_ms;
} dsa_kernel_time;

dsa_status dsa_profile_enable(int32_t on);
int32_t dsa_profile_collect(dsa_kernel_time* out, int32_t max_entries);

/* ---------------------------------------------------------------- launch override
 * Tuning aid: force the sparse-attention launch plan of every later call in this process
 * (dsa_sparse_mla_decode, dsa_sparse_mla_prefill, dsa_decode, and dsa_workspace_size for
 * those entries) instead of the compiled-in launch table, for sweeps without a rebuild.
 * head_tiles: 16-head tiles per workgroup, 1, 2 or 4 (0 = the table's choice); it must divide
 *             the padded head count ceil(H / 16), or the affected calls return
 *             DSA_ERR_UNSUPPORTED.
 * n_split:    splits of each row's list for the split-KV entries (decode and the fused
 *             layer), clamped to [1, the list's 32-row blocks]; 0 = the table's choice.
 *             Prefill rows never split.
 * Size the workspace after setting it. (0, 0) restores the table. DSA_ERR_ARG for other
 * values. Not thread-safe against calls in flight on other threads. DSA_LOG=1 shows the plan
 * each launch takes. */
dsa_status dsa_launch_override(int32_t head_tiles, int32_t n_split);

#ifdef __cplusplus
}
#endif
#endif /* DSA_MI355X_H */
