/*
 * lbm_core.h -- host-only view of the page bookkeeping and planner, for
 * testing without a GPU.
 *
 * The same C++ sources that run inside liblbm (lbm.h) are also built, with no
 * HIP, into liblbm_core.  These entry points drive that bookkeeping directly:
 * no device memory, no kernels.  Semantics, the record formats and the error
 * model are those of the lbm_* calls of the same name in lbm.h
 * (lbmcore_append = the block-0 reservation of lbm_append_frame,
 * lbmcore_evict = lbm_evict_frames, lbmcore_rollback =
 * lbm_rollback_last_frame, lbmcore_plan = lbm_get_plan, lbmcore_dump =
 * lbm_dump_state, lbmcore_stats = lbm_get_stats).
 */
#ifndef LBM_CORE_H
#define LBM_CORE_H

#include "lbm.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct lbmcore lbmcore;

lbm_status lbmcore_create(const lbm_config* cfg, lbmcore** out);
void lbmcore_destroy(lbmcore* core);
lbm_status lbmcore_reset(lbmcore* core);
lbm_status lbmcore_seed_free_lists(lbmcore* core, const int32_t* patch_order, int32_t n_patch,
                                   const int32_t* special_order, int32_t n_special);
lbm_status lbmcore_append(lbmcore* core, int32_t num_frames);
/* Write map of the last append: [nf, patch page per frame..., first special
 * token index, index in the special page list of the page holding it,
 * n special pages touched, those page ids...]. */
lbm_status lbmcore_write_map(const lbmcore* core, int32_t* buf, int64_t cap, int64_t* len);
lbm_status lbmcore_evict(lbmcore* core, int32_t* evicted_ids, int32_t cap, int32_t* n_evicted);
lbm_status lbmcore_rollback(lbmcore* core);
lbm_status lbmcore_plan(const lbmcore* core, int32_t* buf, int64_t cap, int64_t* len);
lbm_status lbmcore_dump(const lbmcore* core, int32_t* buf, int64_t cap, int64_t* len);
lbm_status lbmcore_stats(const lbmcore* core, lbm_stats* out);

/* The planner's key-range split choice for a run of num_q_tokens queries
 * over kv_len keys by a kernel whose workgroups hold rows_per_wg query rows
 * (0: 256; the 16-bit kernel's hold 512, the fp32 kernel's 128), with the
 * fewest query groups that hold the rows: returns the split count (>= 1), or
 * a negative status. */
int32_t lbmcore_choose_splits(int32_t num_q_tokens, int32_t kv_len, int32_t num_heads,
                              int32_t num_cu, int32_t wg_per_cu, int32_t split_cap,
                              int32_t forced, int32_t rows_per_wg);

/* The same choice with the number of query groups chosen as well (the fewest
 * that hold the rows, or one more; the 16-bit kernel's launches): returns the
 * split count and writes the groups to *groups (non-null), or returns a
 * negative status. */
int32_t lbmcore_choose_launch(int32_t num_q_tokens, int32_t kv_len, int32_t num_heads,
                              int32_t num_cu, int32_t wg_per_cu, int32_t split_cap,
                              int32_t forced, int32_t rows_per_wg, int32_t* groups);

const char* lbmcore_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LBM_CORE_H */
