// C entry points of the host-only bookkeeping (lbm_core.h).
#include <new>
#include <vector>

#include "bookkeeping.h"
#include "lbm_core.h"

struct lbmcore {
  explicit lbmcore(const lbm_config& c) : cfg(c), bk(c) {}
  lbm_config cfg;
  lbm::Bookkeeping bk;
};

namespace {
lbm_status copy_out(const std::vector<int32_t>& v, int32_t* buf, int64_t cap, int64_t* len) {
  if (!len) return lbm::fail(LBM_ERR_INVALID_ARG, "len is null");
  if (cap > 0 && !buf) return lbm::fail(LBM_ERR_INVALID_ARG, "buf is null");
  const int64_t n = int64_t(v.size());
  for (int64_t i = 0; i < n && i < cap; ++i) buf[i] = v[size_t(i)];
  *len = n;
  return LBM_OK;
}
}  // namespace

extern "C" {

lbm_status lbmcore_create(const lbm_config* cfg, lbmcore** out) {
  lbm::clear_error();
  if (!cfg || !out) return lbm::fail(LBM_ERR_INVALID_ARG, "null argument");
  const lbm_status st = lbm::validate_config(*cfg);
  if (st != LBM_OK) return st;
  lbmcore* c = new (std::nothrow) lbmcore(*cfg);
  if (!c) return lbm::fail(LBM_ERR_INVALID_ARG, "out of host memory");
  *out = c;
  return LBM_OK;
}

void lbmcore_destroy(lbmcore* core) { delete core; }

lbm_status lbmcore_reset(lbmcore* core) {
  lbm::clear_error();
  if (!core) return lbm::fail(LBM_ERR_INVALID_ARG, "null core");
  core->bk.reset();
  return LBM_OK;
}

lbm_status lbmcore_seed_free_lists(lbmcore* core, const int32_t* patch_order, int32_t n_patch,
                                   const int32_t* special_order, int32_t n_special) {
  lbm::clear_error();
  if (!core) return lbm::fail(LBM_ERR_INVALID_ARG, "null core");
  return core->bk.seed_free_lists(patch_order, n_patch, special_order, n_special);
}

lbm_status lbmcore_append(lbmcore* core, int32_t num_frames) {
  lbm::clear_error();
  if (!core) return lbm::fail(LBM_ERR_INVALID_ARG, "null core");
  return core->bk.reserve(num_frames);
}

lbm_status lbmcore_write_map(const lbmcore* core, int32_t* buf, int64_t cap, int64_t* len) {
  lbm::clear_error();
  if (!core) return lbm::fail(LBM_ERR_INVALID_ARG, "null core");
  const lbm::WriteMap& w = core->bk.write_map();
  std::vector<int32_t> v;
  v.push_back(w.nf);
  v.insert(v.end(), w.patch_pages, w.patch_pages + w.nf);
  v.push_back(w.st0);
  v.push_back(w.sp_first);
  v.push_back(w.n_sp);
  v.insert(v.end(), w.spages, w.spages + w.n_sp);
  return copy_out(v, buf, cap, len);
}

lbm_status lbmcore_evict(lbmcore* core, int32_t* evicted_ids, int32_t cap, int32_t* n_evicted) {
  lbm::clear_error();
  if (!core) return lbm::fail(LBM_ERR_INVALID_ARG, "null core");
  if (cap > 0 && !evicted_ids) return lbm::fail(LBM_ERR_INVALID_ARG, "evicted_ids is null");
  std::vector<int32_t> ev;
  const lbm_status st = core->bk.evict(&ev);
  if (st != LBM_OK) return st;
  for (size_t i = 0; i < ev.size() && int64_t(i) < cap; ++i) evicted_ids[i] = ev[i];
  if (n_evicted) *n_evicted = int32_t(ev.size());
  return LBM_OK;
}

lbm_status lbmcore_rollback(lbmcore* core) {
  lbm::clear_error();
  if (!core) return lbm::fail(LBM_ERR_INVALID_ARG, "null core");
  return core->bk.rollback();
}

lbm_status lbmcore_plan(const lbmcore* core, int32_t* buf, int64_t cap, int64_t* len) {
  lbm::clear_error();
  if (!core) return lbm::fail(LBM_ERR_INVALID_ARG, "null core");
  std::vector<int32_t> v;
  core->bk.plan_record(&v);
  return copy_out(v, buf, cap, len);
}

lbm_status lbmcore_dump(const lbmcore* core, int32_t* buf, int64_t cap, int64_t* len) {
  lbm::clear_error();
  if (!core) return lbm::fail(LBM_ERR_INVALID_ARG, "null core");
  std::vector<int32_t> v;
  core->bk.dump(&v);
  return copy_out(v, buf, cap, len);
}

lbm_status lbmcore_stats(const lbmcore* core, lbm_stats* out) {
  lbm::clear_error();
  if (!core || !out) return lbm::fail(LBM_ERR_INVALID_ARG, "null argument");
  *out = core->bk.stats();
  return LBM_OK;
}

int32_t lbmcore_choose_splits(int32_t num_q_tokens, int32_t kv_len, int32_t num_heads,
                              int32_t num_cu, int32_t wg_per_cu, int32_t split_cap,
                              int32_t forced, int32_t rows_per_wg) {
  return lbm::choose_splits(num_q_tokens, kv_len, num_heads, num_cu, wg_per_cu, split_cap, forced,
                            rows_per_wg > 0 ? rows_per_wg : lbm::kRowsPerGroup);
}

int32_t lbmcore_choose_launch(int32_t num_q_tokens, int32_t kv_len, int32_t num_heads,
                              int32_t num_cu, int32_t wg_per_cu, int32_t split_cap,
                              int32_t forced, int32_t rows_per_wg, int32_t* groups) {
  if (!groups) return LBM_ERR_INVALID_ARG;
  return lbm::choose_splits(num_q_tokens, kv_len, num_heads, num_cu, wg_per_cu, split_cap, forced,
                            rows_per_wg > 0 ? rows_per_wg : lbm::kRowsPerGroup, groups);
}

const char* lbmcore_last_error(void) { return lbm::last_error(); }

}  // extern "C"
