/*
 * lbm.h -- C ABI of the two-stream paged-KV streaming-attention library for
 * AMD Instinct MI355X (gfx950).
 *
 * Each new video frame brings P patch tokens and S special tokens.  The
 * frame's queries attend over a two-stream paged KV cache:
 *   - a patch stream: one page per frame (page size P), of which the first
 *     scale_frames frames are kept for the whole stream and, after them, only
 *     the latest sliding_window frames; evicted pages return to a free list
 *     and are reused;
 *   - a special stream: S tokens per frame packed continuously into pages of
 *     special_page_size tokens, append-only, never evicted.
 * Sources (cited by page title and section):
 *   [P1] "How Paged KV Cache Attention Enables ~20 FPS Streaming Inference in LingBot-Map"
 *   [P2] "How the Paged KV Cache Attention Mechanism Enables Long Sequence Inference in LingBot-Map"
 *   [P3] "How LingBot-Map Uses KV Caching for Efficient Streaming Inference"
 *   [P4] "How FlashInfer's Paged KV Cache Attention Outperforms SDPA Fallback in Streaming Inference"
 *
 * Memory ownership.  The caller owns every device buffer: the per-block page
 * pools, the workspace, and q/k/v/out.  The library owns its host-side
 * bookkeeping and a small pinned staging buffer; it never allocates device
 * memory and never synchronises the device.  All device work is enqueued on
 * the hipStream_t passed to the call (NULL = the default stream); calls that
 * touch the same cache must be issued on one stream, or ordered by the caller.
 *
 * Pool layout ([P4] "Physical Memory Layout"; [P2] "Physical Memory Layout":
 * a 5-D tensor [max_num_pages, 2, page_size, H, D] per block, dim 1 = K/V):
 *   patch pool   [max_patch_pages,   2, P,                 H, D]
 *   special pool [max_special_pages, 2, special_page_size, H, D]
 * in the config dtype, row-major, 16-byte aligned.
 *
 * Token layout of a frame: rows [0, P) are its patch tokens, rows [P, P+S)
 * its special tokens ([P3] "Key methods": patch tokens first, then specials).
 *
 * Errors.  Every call returns an lbm_status; out-parameters are written only
 * on LBM_OK; a failed call leaves the cache unchanged.  lbm_last_error()
 * returns a thread-local message for the last failure.  A handle is not
 * thread-safe: the caller serialises calls on one handle.
 */
#ifndef LBM_H
#define LBM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum lbm_dtype {
  LBM_BF16 = 0, /* bf16 storage, bf16 MFMA products, fp32 softmax and accumulation */
  LBM_F32 = 1,  /* fp32 throughout (the force_fp32 path, [P2] "Memory Efficiency Analysis") */
  LBM_F16 = 2   /* fp16 storage, fp16 MFMA products, fp32 softmax and accumulation (the
                   pages' kernels run natively on fp16 or bf16: [P4] "Precision and Hardware
                   Utilization") */
} lbm_dtype;

typedef enum lbm_status {
  LBM_OK = 0,
  LBM_ERR_INVALID_ARG = -1,  /* a null pointer, a size out of range, a bad config */
  LBM_ERR_BAD_STATE = -2,    /* the call is not allowed in the cache's current state */
  LBM_ERR_OUT_OF_PAGES = -3, /* a free list is empty */
  LBM_ERR_UNSUPPORTED = -4,  /* a valid config this build has no kernel for */
  LBM_ERR_HIP = -5           /* a HIP runtime call failed */
} lbm_status;

/* Cache configuration ([P1] "Implementation Examples": the manager's
 * num_blocks, tokens_per_frame, num_heads, head_dim, dtype,
 * num_special_tokens, scale_frames, sliding_window; [P3] "Configuration
 * Parameters"). */
typedef struct lbm_config {
  int32_t num_blocks;          /* transformer blocks sharing the page bookkeeping, >= 1 */
  int32_t num_heads;           /* H >= 1 */
  int32_t head_dim;            /* D: 64 for bf16; 32 or 64 for fp32 */
  int32_t patches_per_frame;   /* P >= 1, also the patch page size (one page per frame) */
  int32_t special_per_frame;   /* S >= 0 */
  int32_t special_page_size;   /* >= 1 (16 in every workload here) */
  int32_t scale_frames;        /* first frames whose patch pages are never evicted, >= 0 */
  int32_t sliding_window;      /* later frames whose patch pages stay resident, >= 0 */
  int32_t max_patch_pages;     /* patch pool pages; >= scale_frames + sliding_window + 1 for streaming */
  int32_t max_special_pages;   /* special pool pages */
  int32_t max_frames_per_step; /* 1..128: frames one append may bring */
  int32_t max_q_tokens;        /* largest num_q_tokens of lbm_plan / lbm_run */
  int32_t dtype;               /* lbm_dtype */
  int32_t num_splits;          /* 0: the planner splits the key range; n > 0: exactly n splits (capped) */
} lbm_config;

/* The stats record of [P3] "Inspecting Cache Statistics". */
typedef struct lbm_stats {
  int32_t frame_count;    /* accepted frames so far, including a provisional one */
  int32_t scale_pages;    /* patch pages of the scale frames */
  int32_t live_pages;     /* patch pages in the live window FIFO */
  int32_t free_pages;     /* patch pages on the free list */
  int32_t special_tokens; /* special tokens written so far */
} lbm_stats;

typedef struct lbm_cache lbm_cache;

/* Sizes, in bytes, of one block's patch pool, one block's special pool, and
 * the workspace the caller must allocate (device memory, 256-byte aligned). */
lbm_status lbm_query_sizes(const lbm_config* cfg, size_t* patch_pool_bytes,
                           size_t* special_pool_bytes, size_t* workspace_bytes);

/* Create a cache over caller-owned device memory.  patch_pools and
 * special_pools are host arrays of num_blocks device pointers; workspace is a
 * device buffer of the queried size.  Patch and special free lists start in
 * ascending id order
 * ([P4] "Two-Stream Design": pages are allocated from free lists). */
lbm_status lbm_cache_create(const lbm_config* cfg, void* const* patch_pools,
                            void* const* special_pools, void* workspace, lbm_cache** out);

/* Destroy the handle.  Waits only for the library's own pending staging
 * copies; caller-owned device memory is untouched. */
void lbm_cache_destroy(lbm_cache* cache);

/* Empty the cache for a new video: all pages free, counters zero, the free
 * lists back in their initial order ([P3] "Manual Cache Control for Advanced
 * Use Cases": clean_kv_cache). */
lbm_status lbm_cache_reset(lbm_cache* cache);

/* Test hook: replace the initial free-list orders (permutations of
 * [0, max_patch_pages) and [0, max_special_pages)).  Only on an empty cache;
 * kept across lbm_cache_reset. */
lbm_status lbm_cache_seed_free_lists(lbm_cache* cache, const int32_t* patch_order,
                                     int32_t n_patch, const int32_t* special_order,
                                     int32_t n_special);

/* Append num_frames new frames' K/V of one block ([P2] "Appending New
 * Frames"; called once per block: [P2] "Runtime Flow for Frame Processing").
 * k, v: device [num_frames, P + S, H, D] in the config dtype.
 * block_idx 0 opens a step: it reserves one patch page per frame (popping
 * the patch free list; the first scale_frames frames of the stream become
 * scale pages, later ones join the live FIFO) and special slots packed after
 * the previous specials (taking a special page when the count of special
 * tokens is a multiple of special_page_size).  Every block then enqueues a
 * copy of its rows into that reservation.  Blocks 1..num_blocks-1 must follow
 * block 0 in the same step, each once.  Errors: INVALID_ARG (bad block,
 * null pointer, num_frames out of 1..max_frames_per_step), BAD_STATE (block
 * out of order), OUT_OF_PAGES (a free list too short; nothing changes). */
lbm_status lbm_append_frame(lbm_cache* cache, int32_t block_idx, const void* k, const void* v,
                            int32_t num_frames, void* hip_stream);

/* Evict: while the live FIFO holds more than sliding_window pages, move its
 * oldest page to the tail of the patch free list ([P3] "Sliding-Window
 * Eviction Strategy"; [P2] "Evicting Stale Frames").  Scale and special pages
 * are never evicted; nothing is copied.  Host only, idempotent; also commits a
 * provisional frame ([P3] "Flow-Based Keyframe Selection": deferred eviction
 * runs when the frame is kept).  evicted_ids (nullable) receives up to cap
 * evicted page ids, n_evicted (nullable) their count. */
lbm_status lbm_evict_frames(lbm_cache* cache, int32_t* evicted_ids, int32_t cap,
                            int32_t* n_evicted);

/* Undo the last append when it brought one frame and no evict has run since
 * ([P3] "Key methods": rollback_last_frame discards a rejected frame's KV).
 * Restores page tables, free lists (the page back at the head) and counters
 * exactly; page contents are left as they are (no longer visible).
 * Errors: BAD_STATE. */
lbm_status lbm_rollback_last_frame(lbm_cache* cache);

/* Build the visible page table once per frame step ([P4] "Plan-Run Execution
 * Workflow": plan at the first block, reused by every block): the scale
 * pages, the latest sliding_window live pages, then every special page, plus
 * last_page_len, the valid tokens on the final page ([P2] "Building the
 * Visible Page Table").  Host work plus one asynchronous host-to-device copy
 * of the table into the workspace on hip_stream.  num_q_tokens is the query
 * count every lbm_run of this plan will use (1..max_q_tokens).
 * Errors: INVALID_ARG, BAD_STATE (empty cache). */
lbm_status lbm_plan(lbm_cache* cache, int32_t num_q_tokens, void* hip_stream);

/* Paged attention of one block over the planned table ([P4] "Plan-Run
 * Execution Workflow": run once per block; [P1] "FlashInfer Paged-Kernel
 * Integration"): for every query row i and head h,
 *   out[i,h,:] = sum_j softmax_j(q[i,h,:] . k[j,h,:] / sqrt(D)) v[j,h,:]
 * over the visible tokens j, read straight from the pages.  No mask inside a
 * step.  q, out: device [num_q_tokens, H, D] in the config dtype (out
 * rounded to nearest even for bf16).  Enqueues the attention kernel, and a
 * merge kernel when the plan splits the key range.  Errors: INVALID_ARG, BAD_STATE (no
 * plan, a plan made before the last append/evict/rollback, a different
 * num_q_tokens, or block_idx not yet appended in the open step). */
lbm_status lbm_run(lbm_cache* cache, int32_t block_idx, const void* q, void* out,
                   int32_t num_q_tokens, void* hip_stream);

/* Skip-append step: a frame processed without storing its K/V ([P1]
 * "Implementation Examples": non-key frames skip the append; [P3] "Manual
 * Cache Control for Advanced Use Cases": a frame processed without storing
 * its KV).  Plans the visible set of the cache as it stands followed by
 * num_own_tokens rows of the frame itself (1..max_q_tokens), which
 * lbm_run_transient reads from the caller's k/v instead of the pools.  The
 * bookkeeping is unchanged: no page is reserved, nothing is written, the stats
 * and the next frame's visible set are as if the frame never came.  That the
 * frame attends to its own tokens is the plain reading of a block computing
 * attention over the cache and the current tokens (the pages do not say).
 * Same preconditions as lbm_plan; with a step open, every block must have
 * appended it.  Errors: INVALID_ARG, BAD_STATE. */
lbm_status lbm_plan_transient(lbm_cache* cache, int32_t num_q_tokens, int32_t num_own_tokens,
                              void* hip_stream);

/* Attention of one block for a skip-append plan: out = softmax(q K^T/sqrt(D)) V
 * over the visible tokens then the frame's own rows k, v (device
 * [num_own_tokens, H, D] in the config dtype, 16-byte aligned; read only, never
 * stored).  q, out as for lbm_run.  Errors: INVALID_ARG, BAD_STATE (no plan, a
 * stale plan, a normal plan, a different num_q_tokens).  lbm_run refuses a
 * skip-append plan. */
lbm_status lbm_run_transient(lbm_cache* cache, int32_t block_idx, const void* q, const void* k,
                             const void* v, void* out, int32_t num_q_tokens, void* hip_stream);

/* One block's append and attention of a frame step in one call: the append
 * of [P2] "Appending New Frames" and the run of [P4] "Plan-Run Execution
 * Workflow", for callers that make both calls per block back to back.
 * k, v: device [num_frames, P + S, H, D] as for lbm_append_frame; q, out:
 * device [num_q_tokens, H, D] as for lbm_run.  block_idx 0 opens the step: it
 * reserves the pages (as lbm_append_frame), plans (num_q_tokens queries), and
 * evicts (as lbm_evict_frames; the ids are not reported).  Every block's call
 * then enqueues the append kernel (the rows into the reserved pages) and the
 * attention over the visible set, the step's own rows read back from those
 * pages (and the merge).  The result is the same attention as
 * lbm_append_frame + lbm_plan + lbm_run (the keys taken in another order).
 * Blocks 1..num_blocks-1 follow
 * block 0 in the same step, each once, with the same num_frames and
 * num_q_tokens.  k and v must stay unchanged until the append has run.
 * Requires num_frames <= sliding_window (every frame of the step stays
 * visible).  Errors: INVALID_ARG, BAD_STATE (block out of order, the open step
 * opened by lbm_append_frame), OUT_OF_PAGES (nothing changes); a plan refused
 * after block 0's reservation undoes a one-frame reservation, and leaves the
 * cache unusable (BAD_STATE until lbm_cache_reset) after a longer one. */
lbm_status lbm_append_run(lbm_cache* cache, int32_t block_idx, const void* q, const void* k,
                          const void* v, void* out, int32_t num_frames, int32_t num_q_tokens,
                          void* hip_stream);

/* Most streams in one batched run. */
#define LBM_MAX_BATCH 8

/* Batched run: block block_idx of n independent streams (caches), 1..LBM_MAX_BATCH, in one
 * attention launch (and one merge launch per split stream) -- the pages'
 * kernel is a batch prefill over the pages of several requests ([P1]
 * "FlashInfer Paged-Kernel Integration": BatchPrefillWithPagedKVCacheWrapper).
 * Each cache must hold a current plan made by lbm_plan (not a skip-append
 * plan); q[i], out[i]: device [that plan's num_q_tokens, H, D].  All caches
 * share num_heads, head_dim and dtype; they may differ in page sizes, frames
 * and key lengths.  The key-range split count is chosen for the combined work
 * (one count for the launch).  Results equal lbm_run of each cache with that
 * split count.  Errors: INVALID_ARG (n, null or misaligned pointers, mismatched
 * caches, a cache listed twice -- its workspace holds one stream's partials),
 * BAD_STATE (as for lbm_run, per cache). */
lbm_status lbm_run_batch(lbm_cache* const* caches, int32_t n, int32_t block_idx,
                         const void* const* q, void* const* out, void* hip_stream);

/* A whole frame step as one HIP graph ([P1] "Implementation Examples": the
 * block compiles its operations into CUDA graphs).  lbm_graph_create captures,
 * over fixed caller buffers -- per block b: k[b], v[b] (the step's num_frames
 * frames, [num_frames*T, H, D]), q[b] and out[b] ([num_frames*T, H, D]) --
 * one step: every block's append scatter, the row table, every block's
 * attention (and merge), all reading the step's page tables and lengths from
 * the workspace.  k, v, q, out: host arrays of num_blocks device pointers,
 * 16-byte aligned; the buffers must stay valid while the graph lives.  The
 * key-range split count is fixed at capture (cfg.num_splits, else the
 * planner's choice for the full window); splits a step leaves without keys
 * contribute nothing.  Destroy graphs before their cache.  Errors: INVALID_ARG,
 * HIP. */
typedef struct lbm_graph lbm_graph;
lbm_status lbm_graph_create(lbm_cache* cache, int32_t num_frames, const void* const* k,
                            const void* const* v, const void* const* q, void* const* out,
                            lbm_graph** out_graph);

/* One frame step through the graph: on the host, the bookkeeping of append
 * (page reservation), eviction and the plan; then one graph launch on
 * hip_stream that copies the step's tables and runs every block.  Results and
 * cache state equal those of the call sequence append (every block), evict,
 * plan, run (every block) with the graph's split count.  The caller fills
 * k/v/q before the launch (in stream order) and reads out after it.  The host
 * may run at most two steps ahead of the device (pinned staging in two
 * slots).  The eviction is committed once the launch is enqueued.  Errors:
 * OUT_OF_PAGES, BAD_STATE (a step open and not every block appended, or the
 * cache left unusable by an earlier failure), HIP.  When the launch itself
 * fails, a one-frame step's reservation is undone (the cache is as before the
 * call); after a failed multi-frame step, or a failure once the step is
 * queued, every step call (append, evict, rollback, plan, run, graph launch)
 * returns BAD_STATE until lbm_cache_reset. */
lbm_status lbm_graph_launch(lbm_graph* graph, void* hip_stream);

/* The split count fixed at capture (0 for a null graph). */
int32_t lbm_graph_num_splits(const lbm_graph* graph);

/* Waits for the graph's pending launches, then frees it. */
void lbm_graph_destroy(lbm_graph* graph);

/* Stateless paged attention over caller-given tables (device int32 arrays):
 * the visible keys are the n_patch_pages patch pages listed in patch_ids
 * (each P tokens) followed by the first n_special_tokens tokens of the
 * special pages listed in special_ids.  Pools, q, out as above (16-byte
 * aligned); the workspace is a 256-byte aligned device buffer sized by
 * lbm_query_sizes(cfg) (scratch for the row table and split partials; no
 * initial contents required).  Every id must lie below max_patch_pages or
 * max_special_pages: the ids live on the device and are not checked here.
 * Enqueues two to three kernels on hip_stream. */
lbm_status lbm_paged_attention(const lbm_config* cfg, const void* q, void* out,
                               int32_t num_q_tokens, const void* patch_pool,
                               const void* special_pool, const int32_t* patch_ids,
                               int32_t n_patch_pages, const int32_t* special_ids,
                               int32_t n_special_tokens, void* workspace, void* hip_stream);

/* lbm_paged_attention without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  The row table and the split partials live
 * in a static scratch array of 64 MiB in the library's device code, one copy
 * per GPU, held from module load until the process ends; its device address
 * is looked up once per device (hipGetSymbolAddress) on the first call there.
 * The call allocates nothing (no hipMalloc, hipFree or allocating library
 * routine).  Limits: the row table takes 4 bytes per visible key, in whole
 * 64-key tiles, and the scratch holds it for the largest visible set a valid
 * config allows (2^24 keys); a visible set beyond the config's own maximum
 * (scale_frames + sliding_window patch pages, max_special_pages special pages,
 * max_q_tokens own rows) is refused with INVALID_ARG, as lbm_paged_attention
 * refuses it.  The split count is capped to the partials that fit beside the
 * row table (a single split needs none): 9 splits for 1375 query rows of 16
 * heads, so a large run may split less than lbm_paged_attention would.  Every call on one GPU shares that
 * GPU's scratch and leaves its contents behind (nothing in it needs to start
 * at zero): calls that overlap on one GPU -- on different streams, or from
 * different host threads without ordering -- race and give wrong results; the
 * caller orders them.  Other arguments, results and errors as for
 * lbm_paged_attention. */
lbm_status lbm_paged_attention_static(const lbm_config* cfg, const void* q, void* out,
                                      int32_t num_q_tokens, const void* patch_pool,
                                      const void* special_pool, const int32_t* patch_ids,
                                      int32_t n_patch_pages, const int32_t* special_ids,
                                      int32_t n_special_tokens, void* hip_stream);

/* The stats record ([P3] "Inspecting Cache Statistics"). */
lbm_status lbm_get_stats(const lbm_cache* cache, lbm_stats* out);

/* State record for tests: [frame_count, special_tokens, |scale|, scale ids...,
 * |live|, live ids..., |patch free|, ids..., |special|, special ids...,
 * |special free|, ids...].  Writes min(cap, len) entries; *len = full length. */
lbm_status lbm_dump_state(const lbm_cache* cache, int32_t* buf, int64_t cap, int64_t* len);

/* Current table for tests: [kv_len, n_patch_pages, n_special_pages,
 * special_tokens, last_page_len, patch ids..., special ids...], computed from
 * the current state.  Writes min(cap, len) entries; *len = full length. */
lbm_status lbm_get_plan(const lbm_cache* cache, int32_t* buf, int64_t cap, int64_t* len);

/* Number of key-range splits the last lbm_plan chose (0 if none). */
int32_t lbm_plan_num_splits(const lbm_cache* cache);

/* Thread-local message of the last failed call ("" if none). */
const char* lbm_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LBM_H */
