/*
 * paged_attn.h -- C ABI of the MI355X (gfx950) paged-KV attention library.
 *
 * The library computes attention forward over a paged KV cache:
 *
 *   out[i, h, :] = sum_t softmax_t(scale * q[i, h, :] . k[t, kvh, :] + mask(i, t)) v[t, kvh, :]
 *
 * as defined by boostr 0.2.0-beta.2, attention/flash_standard.rs
 * (`standard_attention_fwd`: softmax(Q K^T * scale + mask) V, natural-log
 * logsumexp per query row in f32; `build_attention_mask`: causal and
 * sliding-window masking; `expand_kv`: query head h uses KV head
 * h / (Hq / Hkv)), over the paged layout and absolute positions of ruDNN
 * 0.1.107, paged_attention/mod.rs (`DevicePlan::attention`: packed Q
 * [queries, Hq, D], K [pages, page_size, Hkv, D], V [pages, page_size, Hkv,
 * Dv]; causal masking compares absolute positions from the plan, prefill
 * chunks included, so packed decode queries and chunked-prefill queries run
 * in one launch).
 *
 * Masking, for a query at absolute position p of a sequence holding L keys:
 * key position t is visible iff t < L, (causal == 0 or t <= p) and
 * (window == 0 or t > p - window).  Logical key t of sequence s lives in pool
 * page block_table[s * table_width + t / page_size], slot t % page_size.
 *
 * Conventions for every entry point:
 *   - Return value: PA_OK (0) or a negative pa_status.  On failure nothing
 *     was launched, allocated or written (ruDNN `execute_attention_into` and
 *     `execute_backward_into` validate everything before any launch or
 *     allocation); pa_last_error() then gives a detail message for the
 *     calling thread.
 *   - Device pointers are HIP device addresses on the plan's device; tensors
 *     are dense row-major with the shapes stated.  The caller owns every
 *     tensor, the workspace included; the library owns only the plan.
 *   - `stream` is a hipStream_t (NULL = the null stream).  A plan belongs to
 *     the device and the stream it was made on, and so does any workspace
 *     used with it (ruDNN: metadata and split workspaces belong to one device
 *     queue): every call with a plan must pass that stream, else
 *     PA_ERR_DEVICE.  The forward calls only enqueue kernels: no host
 *     synchronisation, no device-to-host readback (ruDNN
 *     `attention_into_split`).
 *   - Calls with different plans that share an output or a workspace must be
 *     ordered by the caller (same stream, or events); concurrent calls on
 *     them race.
 */
#ifndef PAGED_ATTN_H
#define PAGED_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes.  Each error case of ruDNN's `PagedAttentionError` falls in
 * one of these classes; pa_status_string() describes a class. */
typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_INVALID = -1,     /* null pointer, unknown dtype, flag out of range */
  PA_ERR_SHAPE = -2,       /* tensor sizes, head counts or scale that do not fit together */
  PA_ERR_PLAN = -3,        /* malformed schedule: offsets, positions, block table */
  PA_ERR_UNSUPPORTED = -4, /* valid request with no kernel specialisation in this build */
  PA_ERR_WORKSPACE = -5,   /* split workspace missing or too small */
  PA_ERR_OVERLAP = -6,     /* an output overlaps an input or another output */
  PA_ERR_RANGE = -7,       /* a size exceeds the 32-bit index range */
  PA_ERR_HIP = -8,         /* HIP runtime failure (allocation, copy or launch) */
  PA_ERR_DEVICE = -9       /* plan used on a device or stream other than the one it was made on, or built on
                              the host only */
} pa_status;

typedef enum pa_dtype {
  PA_F32 = 0, /* IEEE binary32 */
  PA_BF16 = 1, /* bfloat16, raw 16-bit patterns; outputs rounded to nearest even */
  PA_F16 = 2   /* IEEE binary16; outputs rounded to nearest even */
} pa_dtype;

/*
 * Schedule of one batch (host memory; copied, not retained).
 *
 * ruDNN `DevicePlan` (its doc comment sits, garbled, above the backward
 * structs): immutable metadata uploaded once and reusable for every call while
 * the schedule is unchanged; cache data are supplied separately.  The query
 * packing follows alice-llm 2.0.0, sparse_attention/llama3_bridge.rs
 * (`CuSeqlensQ` offsets and per-sequence `BlockTables`).
 *
 *   num_seqs         S >= 0
 *   seq_lens[S]      L_s >= 0 keys held by sequence s (its new tokens included)
 *   cu_q[S+1]        packed query offsets: queries of s are cu_q[s] .. cu_q[s+1]-1;
 *                    cu_q[0] == 0, non-decreasing
 *   q_pos[Q]         absolute position of each packed query, 0 <= q_pos < L_s
 *                    (Q = cu_q[S]); a query's own key is in the cache
 *   block_table[S*W] pool page of logical page j of sequence s at [s * W + j];
 *                    entries j < ceil(L_s / page_size) must be in [0, num_pages);
 *                    later entries are ignored
 *   table_width      W >= 1
 *   page_size        keys per page; a power of two in [1, 1024]
 *   num_pages        pages in the K/V pools
 *   num_q_heads      Hq (MLA: H)
 *   num_kv_heads     Hkv, divides Hq (MLA: must be 1)
 *   causal           0 or 1
 *   window           0 = unlimited, else the number of visible keys ending at the
 *                    query position (boostr `StandardAttnConfig::window_size`)
 *   max_splits       1..64: cap on the key ranges one decode query row is split
 *                    into (1 = never split; no workspace needed)
 *   mla              0 = GQA/MHA plan (pa_attention_fwd); 1 = absorbed-MLA plan
 *                    (pa_mla_fwd)
 *   split_tokens     0 = library default; else target keys per decode split
 *                    (rounded to a multiple of 64)
 */
typedef struct pa_plan_desc {
  int32_t num_seqs;
  const int32_t* seq_lens;
  const int32_t* cu_q;
  const int32_t* q_pos;
  const int32_t* block_table;
  int32_t table_width;
  int32_t page_size;
  int32_t num_pages;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t causal;
  int32_t window;
  int32_t max_splits;
  int32_t mla;
  int32_t split_tokens;
} pa_plan_desc;

typedef struct pa_plan pa_plan;

/* Counts of the work a plan schedules (host-side, no synchronisation). */
typedef struct pa_plan_info {
  int32_t num_queries;   /* Q */
  int32_t decode_items;  /* (query, KV head, key range) workgroups */
  int32_t prefill_items; /* (query tile, KV head) workgroups */
  int32_t split_rows;    /* (query, KV head) rows split into >1 ranges */
  int32_t split_slots;   /* partial-statistics slots those rows use */
  int32_t launches;      /* kernels one forward call enqueues (0, 1 or 2) */
  int32_t workgroups;    /* workgroups of the main launch */
  int32_t heads_per_item; /* KV heads one decode item covers (decode-only plans: a power of two) */
  int32_t bwd_dq_items;   /* backward: (query, KV head) workgroups of the dQ pass (GQA plans) */
  int32_t bwd_kv_items;   /* backward: (128-key block, KV head) workgroups of the dK/dV pass */
  int32_t bwd_shared_pages; /* backward: 1 when a referenced pool page holds two key positions (f32 atomic sums) */
} pa_plan_info;

/*
 * Validate a schedule, build the work list on the host and upload it with one
 * asynchronous host-to-device copy on `stream` (on the current HIP device),
 * into device memory allocated in stream order on that stream.  The plan
 * keeps its host copy and is bound to that device and stream.  Errors:
 * PA_ERR_INVALID, PA_ERR_PLAN, PA_ERR_UNSUPPORTED (e.g. page_size not a power of
 * two), PA_ERR_RANGE, PA_ERR_HIP.  *out_plan is set only on success.
 */
int pa_plan_create(const pa_plan_desc* desc, void* stream, pa_plan** out_plan);

/* Free a plan (NULL is allowed).  The device buffer is released in stream
 * order on the plan's stream, after every call already enqueued there; the
 * host does not wait for the device (only, if still pending, for the upload
 * copy).  Destroy a plan before destroying its stream. */
int pa_plan_destroy(pa_plan* plan);

/* Fill *info with the plan's work counts. */
int pa_plan_get_info(const pa_plan* plan, pa_plan_info* info);

/*
 * Build the work lists pa_plan_create would build on a device with `num_cus`
 * compute units, on the host only: no HIP call, no device memory.  For
 * inspecting and testing the planner (pa_plan_get_info, pa_plan_get_work);
 * forward calls reject such a plan with PA_ERR_DEVICE.  Release it with
 * pa_plan_destroy.  Errors: as pa_plan_create, PA_ERR_INVALID for num_cus
 * outside [1, 65536].
 */
int pa_plan_create_host(const pa_plan_desc* desc, int32_t num_cus, pa_plan** out_plan);

/*
 * Copy a plan's work lists (host copy; any plan).  *n_items, *n_wg and
 * *n_merges receive the counts; each array may be NULL to skip it, else it
 * must hold:
 *   items     8 * n_items int32: per work item (kind: 0 decode, 1 prefill,
 *             2 empty; first KV head; sequence; first packed query; query
 *             count; first key; end key (exclusive); partial slot of the
 *             first head, -1 when the row is not split).  A decode item of a
 *             decode-only plan covers 2^s consecutive KV heads
 *             (pa_plan_info.heads_per_item), head kvh + i using slot + i.
 *   wg_first  n_wg + 1 int32: workgroup b of the main launch runs items
 *             wg_first[b] .. wg_first[b + 1] - 1.
 *   merges    5 * n_merges int32: per split (query, KV head) row (query; KV
 *             head; first slot; number of pieces; slot stride).
 */
int pa_plan_get_work(const pa_plan* plan, int32_t* items, int32_t* n_items, int32_t* wg_first, int32_t* n_wg,
                     int32_t* merges, int32_t* n_merges);

/*
 * Bytes of f32 split workspace a forward call with value width `v_head_dim`
 * needs (0 when no query row is split).  The workspace holds, per split slot
 * and query head of the group, the unnormalised output sums and (max, sum)
 * statistics (ruDNN `SplitWorkspace`: f32 partials matched to queries, heads,
 * value width and splits); a second, small kernel merges them.
 */
int pa_plan_workspace_bytes(const pa_plan* plan, int32_t v_head_dim, size_t* bytes);

/*
 * Paged GQA/MHA attention forward (ruDNN `DevicePlan::attention_into` /
 * `attention_into_split`).
 *
 *   dtype        PA_F32, PA_BF16 or PA_F16, the type of q, k_pool, v_pool and out
 *   q            [Q, Hq, head_dim]
 *   k_pool       [num_pages, page_size, Hkv, head_dim]
 *   v_pool       [num_pages, page_size, Hkv, v_head_dim]
 *   out          [Q, Hq, v_head_dim], written (must not overlap any input)
 *   lse          NULL or f32 [Q, Hq]: natural-log logsumexp of the scaled,
 *                masked scores of each row
 *   head_dim     D, 1..1024; v_head_dim Dv, 1..1024, any group size
 *                Hq / Hkv.  D = Dv in {64, 128, 256} and D = 192 with
 *                Dv = 128 at group sizes {1, 2, 3, 4, 5, 6, 7, 8, 12, 16}
 *                run on the specialised decode and MFMA kernels; every
 *                other shape runs on a vector-ALU kernel (fp32), which takes
 *                the query heads of a KV head in groups of 16
 *   scale        finite and > 0 (e.g. 1/sqrt(D))
 *   workspace    f32 scratch of >= pa_plan_workspace_bytes(plan, v_head_dim)
 *                bytes, 256-byte aligned; may be NULL when that size is 0
 *   main_events  NULL, or an array of two hipEvent_t (timing enabled) that
 *                receive the start and the end of the main attention
 *                kernel's own execution (hipExtLaunchKernel), so a caller can
 *                time that kernel apart from the split merge
 *
 * Tensors other than lse and the workspace must be 16-byte aligned
 * (PA_ERR_INVALID otherwise); the kernels move rows in 16-byte pieces.
 *
 * The plan must be a GQA plan (mla == 0) made on the current device.
 * Q == 0 returns PA_OK without launching anything; q and out (empty then)
 * may be NULL.
 */
int pa_attention_fwd(const pa_plan* plan, int32_t dtype, const void* q, const void* k_pool,
                     const void* v_pool, void* out, float* lse, int32_t head_dim,
                     int32_t v_head_dim, float scale, void* workspace, size_t workspace_bytes,
                     void* const* main_events, void* stream);

/* Bytes of the fixed device array that pa_attention_fwd_noalloc keeps the
 * split partials in (per GPU, held until the process ends). */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/*
 * pa_attention_fwd without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  It runs the same kernels as
 * pa_attention_fwd; the split partials live in one file-scope device array
 * of PA_NOALLOC_SCRATCH_BYTES bytes per GPU instead of a caller workspace.
 * The call allocates nothing (no hipMalloc, no host heap in its checks).
 *
 * Every call on one GPU shares that array, which keeps the last call's
 * contents (nothing in it needs clearing: each partial the merge reads is
 * written earlier in the same call).  Calls that overlap in time on one GPU
 * -- on different streams, or from plans whose calls are not ordered --
 * race on it; order them.
 *
 * Arguments, layouts and errors as for pa_attention_fwd (no main_events),
 * plus PA_ERR_WORKSPACE when pa_plan_workspace_bytes(plan, v_head_dim)
 * exceeds PA_NOALLOC_SCRATCH_BYTES (checked before anything is launched).
 */
int pa_attention_fwd_noalloc(const pa_plan* plan, int32_t dtype, const void* q, const void* k_pool,
                             const void* v_pool, void* out, float* lse, int32_t head_dim,
                             int32_t v_head_dim, float scale, void* stream);

/*
 * Absorbed multi-head latent attention forward (ruDNN `DevicePlan::mla`): one
 * shared latent head serves as both key and value; a rotated position cache
 * adds a second dot product to every score:
 *
 *   score(i, h, t) = scale * (q_abs[i, h, :] . latent[t, :] + q_rope[i, h, :] . kpos[t, :])
 *   out[i, h, :]   = sum_t softmax_t(score + mask) latent[t, :]
 *
 *   q_abs   [Q, H, rank]        q_rope [Q, H, rope_dim]
 *   latent  [num_pages, page_size, 1, rank]
 *   kpos    [num_pages, page_size, 1, rope_dim]
 *   out     [Q, H, rank]        lse NULL or f32 [Q, H]
 *   rank    1..1024, rope_dim 1..256, any H >= 1, dtype PA_F32, PA_BF16 or
 *           PA_F16.  16-bit data with rank 512 and rope_dim 64 runs on MFMA
 *           (the heads in groups of 16, so H = 16 n uses every MFMA column);
 *           every other shape and f32 run on a vector-ALU kernel (fp32)
 *   scale   from the model's original query/key head size, not the latent
 *           rank (e.g. 1/sqrt(rank + rope_dim))
 *
 * The plan must be an MLA plan (mla == 1, num_kv_heads == 1).  The remaining
 * arguments are as for pa_attention_fwd.
 */
int pa_mla_fwd(const pa_plan* plan, int32_t dtype, const void* q_abs, const void* q_rope,
               const void* latent, const void* kpos, void* out, float* lse, int32_t rank,
               int32_t rope_dim, float scale, void* workspace, size_t workspace_bytes,
               void* const* main_events, void* stream);

/* Static name of a status code. */
const char* pa_status_string(int status);

/*
 * Paged K/V append (ruDNN 0.1.107 paged_attention `DevicePlan::append`: the
 * cache write that precedes attention in a decode or prefill step): for every
 * packed query i of sequence s at position p = q_pos[i], the new rows go to
 * pool page block_table[s][p / page_size], slot p % page_size:
 *
 *   k_pool[page, slot, h, :] = k_new[i, h, :]   v_pool[page, slot, h, :] = v_new[i, h, :]
 *
 *   dtype     PA_F32, PA_BF16 or PA_F16 (of all four tensors; rows are copied bit
 *             for bit)
 *   k_new     [Q, heads, head_dim]       v_new [Q, heads, v_head_dim]
 *   k_pool    [num_pages, page_size, heads, head_dim], written in place
 *   v_pool    [num_pages, page_size, heads, v_head_dim], written in place
 *   heads     the plan's num_kv_heads (1 for an MLA plan: k_new / k_pool are
 *             the latent rows and pool, v_new / v_pool the rotary ones)
 *
 * Rows of the pools that no query's position names are left as they are.
 * Copy-on-write of caches shared between sequences is the caller's (the
 * library never allocates).  Errors: PA_ERR_PLAN when two queries of the plan
 * name the same pool slot (their writes would race); PA_ERR_UNSUPPORTED for
 * rows that are not whole 16-byte chunks; PA_ERR_OVERLAP when a new-row
 * tensor overlaps a pool or the pools overlap; otherwise as pa_attention_fwd.
 * Q == 0 returns PA_OK without launching anything (k_new and v_new may then
 * be NULL).
 */
int pa_append_kv(const pa_plan* plan, int32_t dtype, const void* k_new, const void* v_new, void* k_pool,
                 void* v_pool, int32_t head_dim, int32_t v_head_dim, void* stream);

/*
 * Bytes of f32 workspace pa_attention_bwd needs for this plan, data type and
 * head sizes: one value per (query, head) row (D = dO . O), 256-byte aligned;
 * when the plan has queries and a pool page holding two key positions
 * (pa_plan_info.bwd_shared_pages) and the data are 16-bit, also f32 sums of
 * the whole dK and dV pools (num_pages * page_size * Hkv * (D + Dv) values;
 * ruDNN's backward keeps low-precision history gradients in f32 scratch the
 * same way).  0 when the plan has no queries.  Errors: PA_ERR_INVALID for a
 * NULL argument or an unknown dtype, PA_ERR_SHAPE for head sizes outside
 * [1, 1024].
 */
int pa_plan_bwd_workspace_bytes(const pa_plan* plan, int32_t dtype, int32_t head_dim, int32_t v_head_dim,
                                size_t* bytes);

/*
 * Paged GQA/MHA backward (ruDNN 0.1.107 paged_attention
 * `attention_backward_into`: first-order gradients, scores recomputed from Q
 * and K; formulas of boostr `standard_attention_bwd`).  With P the softmax
 * weights of a row and dO its output gradient:
 *
 *   D = dO . O   dS_t = P_t (dO . V_t - D)   dQ = scale sum_t dS_t K_t
 *   dK_t = scale sum_rows dS_t Q             dV_t = sum_rows P_t dO
 *
 * summed over the G query heads of each KV head.  When every referenced pool
 * page holds key positions of one sequence, every pool row has a single
 * writer (ruDNN's ordered, atomic-free variant) and results repeat bit for
 * bit.  When a page is shared (prefix sharing between sequences, or one page
 * at two positions of a sequence), the contributions to its rows are added
 * up in f32 with atomic adds (ruDNN's atomic variant), in the pools for f32
 * data and in workspace sums rounded into the pools once for 16-bit data;
 * the order of the additions, and so the last bits of those rows, may then
 * change from call to call.
 *
 *   dtype        of q, k_pool, v_pool, out, dout, dq, dk_pool, dv_pool
 *   q, k_pool, v_pool  as for pa_attention_fwd with the same plan
 *   out, lse     the forward's output [Q, Hq, Dv] and f32 logsumexp [Q, Hq]
 *   dout         output gradient [Q, Hq, Dv]
 *   dq           [Q, Hq, D], written
 *   dk_pool, dv_pool  pool shaped like k_pool / v_pool, written in full: rows
 *                no visible key of any query lands on are zero
 *   workspace    >= pa_plan_bwd_workspace_bytes bytes, 256-byte aligned
 *
 * Head sizes and group sizes as for pa_attention_fwd: D = Dv in {64, 128, 256}
 * and 192 / 128 at group sizes 1, 2, 4, 8, 16 run on the specialised kernels
 * (16-bit MFMA, f32 vector), every other shape on vector-ALU kernels (fp32).
 * Errors:
 * PA_ERR_INVALID for MLA plans (pa_mla_bwd);
 * PA_ERR_WORKSPACE,
 * PA_ERR_OVERLAP, PA_ERR_SHAPE, PA_ERR_DEVICE, PA_ERR_HIP as for
 * pa_attention_fwd.  Q == 0 zeroes dk_pool and dv_pool and touches nothing
 * else.
 */
int pa_attention_bwd(const pa_plan* plan, int32_t dtype, const void* q, const void* k_pool, const void* v_pool,
                     const void* out, const float* lse, const void* dout, void* dq, void* dk_pool, void* dv_pool,
                     int32_t head_dim, int32_t v_head_dim, float scale, void* workspace, size_t workspace_bytes,
                     void* stream);

/*
 * Block-sparse top-k attention (alice-llm 2.0.0, sparse_attention/
 * llama3_bridge.rs, `llama3_sparse_attention`), on a GQA plan.  Key
 * positions are grouped in blocks of `block_size` (a multiple of the plan's
 * page size: block r holds positions [r * block_size, (r + 1) *
 * block_size)).  For each query and KV head:
 *
 *   1. candidates: the blocks that hold a key the query sees (mask as for
 *      pa_attention_fwd);
 *   2. proxy score of a candidate: the largest dot product between the
 *      group's FIRST query head (h = kvh * G) and a visible key of the block,
 *      an f32 sum over dimensions in increasing order, one fused
 *      multiply-add per dimension (`compute_proxy_block_max_scores`);
 *   3. kept blocks: all candidates when topk == 0 or topk >= their number
 *      (the page's dense fallback), else the topk best scores, a tie going
 *      to the lower block index (`sparse_topk_select_batch`);
 *   4. every query head of the group attends to the visible keys of the kept
 *      blocks only: one partial per block, merged by log-sum-exp weights
 *      (`kvouter_forward`, `lse_combine`).
 *
 *   block_size  > 0, a multiple of the plan's page size; a query row may
 *               span at most 8192 blocks
 *   topk        >= 0 (0 = keep every block)
 *   selection   NULL, or int32 [Q, Hkv, width] receiving each row's kept
 *               blocks in increasing order, -1 padded (width from
 *               pa_sparse_workspace_bytes)
 *   workspace   >= pa_sparse_workspace_bytes bytes, 256-byte aligned
 *
 * Other arguments, layouts and errors as for pa_attention_fwd (the plan's
 * own split settings are not used: each kept block is one split piece);
 * PA_ERR_SHAPE for a block size that is not a positive multiple of the page
 * size; PA_ERR_UNSUPPORTED for K rows that are not whole 16-byte pieces or
 * rows of more than 8192 blocks.  Four launches when topk > 0 (block
 * scores, selection, block attention, merge), three when topk == 0.
 */
int pa_sparse_attention_fwd(const pa_plan* plan, int32_t dtype, const void* q, const void* k_pool,
                            const void* v_pool, void* out, float* lse, int32_t head_dim,
                            int32_t v_head_dim, float scale, int32_t block_size, int32_t topk,
                            int32_t* selection, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes and selection width (topk, or for topk == 0 the largest
 * candidate count of any row) of pa_sparse_attention_fwd for this plan. */
int pa_sparse_workspace_bytes(const pa_plan* plan, int32_t v_head_dim, int32_t block_size, int32_t topk,
                              size_t* bytes, int32_t* width);

/*
 * Absorbed-MLA backward (ruDNN 0.1.107 paged_attention `mla_backward` /
 * `mla_backward_into`): first-order gradients of pa_mla_fwd, scores
 * recomputed from the queries and the caches.  The latent serves as key and
 * value, so its gradient holds both terms.  With s_t = scale (q_abs . lat_t
 * + q_rope . kpos_t), P the softmax weights of a row (from the forward's
 * lse), dP_t = dO . lat_t, D = dO . O and dS_t = P_t (dP_t - D):
 *
 *   dq_abs = scale sum_t dS_t lat_t        dq_rope = scale sum_t dS_t kpos_t
 *   dlat_t = sum_rows (scale dS_t q_abs + P_t dO)
 *   dkpos_t = sum_rows scale dS_t q_rope
 *
 *   dtype        PA_F32, PA_BF16 or PA_F16; rank and rope_dim as for
 *                pa_mla_fwd, any H (16-bit rank 512 / rope_dim 64 on MFMA,
 *                the rest on vector-ALU kernels)
 *   q_abs, q_rope, latent, kpos, out, lse  as for pa_mla_fwd with the same
 *                plan (out and lse: the forward's results)
 *   dout         [Q, H, rank] output gradient
 *   dq_abs       [Q, H, rank], dq_rope [Q, H, rope_dim], written
 *   dlatent, dkpos  pools shaped like latent / kpos, written in full (rows no
 *                visible key lands on are zero)
 *   workspace    >= pa_plan_bwd_workspace_bytes(plan, dtype, rank, rope_dim)
 *
 * Pool rows have a single writer unless a page is shared (then f32 sums in
 * the workspace, as pa_attention_bwd).  Errors as pa_attention_bwd; a GQA
 * plan gives PA_ERR_INVALID.
 */
int pa_mla_bwd(const pa_plan* plan, int32_t dtype, const void* q_abs, const void* q_rope, const void* latent,
               const void* kpos, const void* out, const float* lse, const void* dout, void* dq_abs, void* dq_rope,
               void* dlatent, void* dkpos, int32_t rank, int32_t rope_dim, float scale, void* workspace,
               size_t workspace_bytes, void* stream);

/* Detail message of the calling thread's last failure ("" if none). */
const char* pa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_ATTN_H */
