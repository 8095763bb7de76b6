// Host-side page bookkeeping and planner (see bookkeeping.h for the policy).
#include "bookkeeping.h"

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <limits>

namespace lbm {

namespace {
thread_local std::string g_error;

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
int32_t ceil_div(int32_t a, int32_t b) { return (a + b - 1) / b; }

bool is_permutation_of_iota(const int32_t* p, int32_t n) {
  std::vector<char> seen(static_cast<size_t>(n), 0);
  for (int32_t i = 0; i < n; ++i) {
    if (p[i] < 0 || p[i] >= n || seen[p[i]]) return false;
    seen[p[i]] = 1;
  }
  return true;
}
}  // namespace

lbm_status fail(lbm_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_error = buf;
  return st;
}

void clear_error() { g_error.clear(); }
const char* last_error() { return g_error.c_str(); }

size_t dtype_size(int32_t dtype) { return dtype == LBM_F32 ? 4 : 2; }

lbm_status validate_config(const lbm_config& c) {
  if (c.num_blocks < 1) return fail(LBM_ERR_INVALID_ARG, "num_blocks %d < 1", c.num_blocks);
  if (c.num_heads < 1) return fail(LBM_ERR_INVALID_ARG, "num_heads %d < 1", c.num_heads);
  if (c.head_dim < 1) return fail(LBM_ERR_INVALID_ARG, "head_dim %d < 1", c.head_dim);
  if (c.patches_per_frame < 1)
    return fail(LBM_ERR_INVALID_ARG, "patches_per_frame %d < 1", c.patches_per_frame);
  if (c.special_per_frame < 0)
    return fail(LBM_ERR_INVALID_ARG, "special_per_frame %d < 0", c.special_per_frame);
  if (c.special_page_size < 1)
    return fail(LBM_ERR_INVALID_ARG, "special_page_size %d < 1", c.special_page_size);
  if (c.scale_frames < 0 || c.sliding_window < 0)
    return fail(LBM_ERR_INVALID_ARG, "negative scale_frames or sliding_window");
  if (c.max_patch_pages < 1)
    return fail(LBM_ERR_INVALID_ARG, "max_patch_pages %d < 1", c.max_patch_pages);
  if (c.max_special_pages < 0)
    return fail(LBM_ERR_INVALID_ARG, "max_special_pages %d < 0", c.max_special_pages);
  if (c.max_frames_per_step < 1 || c.max_frames_per_step > kMaxStepFrames)
    return fail(LBM_ERR_INVALID_ARG, "max_frames_per_step %d outside 1..%d",
                c.max_frames_per_step, kMaxStepFrames);
  if (c.max_q_tokens < 1) return fail(LBM_ERR_INVALID_ARG, "max_q_tokens %d < 1", c.max_q_tokens);
  if (c.dtype != LBM_BF16 && c.dtype != LBM_F32 && c.dtype != LBM_F16)
    return fail(LBM_ERR_INVALID_ARG, "dtype %d", c.dtype);
  if (c.num_splits < 0) return fail(LBM_ERR_INVALID_ARG, "num_splits %d < 0", c.num_splits);
  // special pages one append can touch must fit the kernel argument block
  const int64_t sp_touch =
      (int64_t(c.max_frames_per_step) * c.special_per_frame + c.special_page_size - 1) /
          c.special_page_size + 1;
  if (sp_touch > kMaxStepSpecialPages)
    return fail(LBM_ERR_UNSUPPORTED, "one append may touch %lld special pages (> %d)",
                (long long)sp_touch, kMaxStepSpecialPages);
  // every visible key position must stay below 2^24
  // visible keys at most, plus the own rows of a skip-append step
  const int64_t max_kv = int64_t(c.scale_frames + c.sliding_window) * c.patches_per_frame +
                         int64_t(c.max_special_pages) * c.special_page_size + c.max_q_tokens;
  if (max_kv >= kMaxKvLen)
    return fail(LBM_ERR_UNSUPPORTED, "visible key range %lld exceeds %d", (long long)max_kv,
                kMaxKvLen);
  const int64_t row_elems = int64_t(c.num_heads) * c.head_dim;
  const int64_t row_bytes = row_elems * int64_t(dtype_size(c.dtype));
  if (row_bytes % 16 != 0)
    return fail(LBM_ERR_UNSUPPORTED, "a token row of H*D elements must be a multiple of 16 bytes");
  // the kernels address a row by a 31-bit byte offset inside its block's pool
  const int64_t pool_max = std::max(int64_t(c.max_patch_pages) * 2 * c.patches_per_frame,
                                    int64_t(c.max_special_pages) * 2 * c.special_page_size) *
                           row_bytes;
  if (pool_max >= (int64_t(1) << 31))
    return fail(LBM_ERR_UNSUPPORTED, "one block's pool exceeds 2 GiB (%lld bytes)",
                (long long)pool_max);
  return LBM_OK;
}

// ---------------------------------------------------------------------------

Bookkeeping::Bookkeeping(const lbm_config& c)
    : P_(c.patches_per_frame),
      S_(c.special_per_frame),
      sps_(c.special_page_size),
      scale_frames_(c.scale_frames),
      window_(c.sliding_window),
      max_patch_(c.max_patch_pages),
      max_special_(c.max_special_pages),
      max_step_(c.max_frames_per_step) {
  patch_order_.resize(max_patch_);
  special_order_.resize(max_special_);
  for (int32_t i = 0; i < max_patch_; ++i) patch_order_[i] = i;
  for (int32_t i = 0; i < max_special_; ++i) special_order_[i] = i;
  reset();
}

lbm_status Bookkeeping::seed_free_lists(const int32_t* po, int32_t np, const int32_t* so,
                                        int32_t ns) {
  if (!empty() || undo_.valid)
    return fail(LBM_ERR_BAD_STATE, "free lists can be seeded only on an empty cache");
  if (np != max_patch_ || ns != max_special_ || (np > 0 && !po) || (ns > 0 && !so))
    return fail(LBM_ERR_INVALID_ARG, "free-list orders must cover every page");
  if (!is_permutation_of_iota(po, np) || !is_permutation_of_iota(so, ns))
    return fail(LBM_ERR_INVALID_ARG, "free-list order is not a permutation");
  patch_order_.assign(po, po + np);
  special_order_.assign(so, so + ns);
  reset();
  return LBM_OK;
}

void Bookkeeping::reset() {
  patch_free_.assign(patch_order_.begin(), patch_order_.end());
  special_free_.assign(special_order_.begin(), special_order_.end());
  live_.clear();
  scale_.clear();
  all_special_.clear();
  frame_count_ = 0;
  special_tokens_ = 0;
  undo_ = Undo();
  wm_ = WriteMap();
  ++epoch_;
}

lbm_status Bookkeeping::reserve(int32_t nf) {
  if (nf < 1 || nf > max_step_)
    return fail(LBM_ERR_INVALID_ARG, "num_frames %d outside 1..%d", nf, max_step_);
  if (int32_t(patch_free_.size()) < nf)
    return fail(LBM_ERR_OUT_OF_PAGES, "patch free list holds %zu pages, append needs %d",
                patch_free_.size(), nf);
  // special pages needed: one per multiple of the page size crossed
  const int64_t t0 = special_tokens_;
  const int64_t t1 = t0 + int64_t(nf) * S_;
  const int64_t need_sp = (t1 + sps_ - 1) / sps_ - (t0 + sps_ - 1) / sps_;
  if (int64_t(special_free_.size()) < need_sp)
    return fail(LBM_ERR_OUT_OF_PAGES, "special free list holds %zu pages, append needs %lld",
                special_free_.size(), (long long)need_sp);
  if (t1 > std::numeric_limits<int32_t>::max())
    return fail(LBM_ERR_INVALID_ARG, "special token count overflows");

  Undo u;
  u.valid = true;
  u.nf = nf;
  u.frame_count = frame_count_;
  u.special_tokens = special_tokens_;
  WriteMap wm;
  wm.nf = nf;
  wm.st0 = special_tokens_;
  wm.sp_first = special_tokens_ / sps_;
  for (int32_t f = 0; f < nf; ++f) {
    const int32_t page = patch_free_.front();
    patch_free_.pop_front();
    const bool to_scale = frame_count_ < scale_frames_;
    if (to_scale)
      scale_.push_back(page);
    else
      live_.push_back(page);
    if (f == 0) {
      u.page = page;
      u.to_scale = to_scale;
    }
    wm.patch_pages[f] = page;
    ++frame_count_;
    for (int32_t s = 0; s < S_; ++s) {
      if (special_tokens_ % sps_ == 0) {
        const int32_t sp = special_free_.front();
        special_free_.pop_front();
        all_special_.push_back(sp);
        u.special.push_back(sp);
      }
      ++special_tokens_;
    }
  }
  const int32_t last_page = special_tokens_ > 0 ? (special_tokens_ - 1) / sps_ : -1;
  wm.n_sp = (nf * S_ > 0) ? last_page - wm.sp_first + 1 : 0;
  for (int32_t i = 0; i < wm.n_sp; ++i) wm.spages[i] = all_special_[wm.sp_first + i];
  wm_ = wm;
  undo_ = std::move(u);
  ++epoch_;
  return LBM_OK;
}

lbm_status Bookkeeping::evict(std::vector<int32_t>* evicted) {
  if (evicted) evicted->clear();
  bool changed = false;
  while (int32_t(live_.size()) > window_) {
    const int32_t page = live_.front();
    live_.pop_front();
    patch_free_.push_back(page);
    if (evicted) evicted->push_back(page);
    changed = true;
  }
  undo_.valid = false;  // evict commits the step
  if (changed) ++epoch_;
  return LBM_OK;
}

lbm_status Bookkeeping::rollback() {
  if (!undo_.valid) return fail(LBM_ERR_BAD_STATE, "no append to roll back (or already committed)");
  if (undo_.nf != 1)
    return fail(LBM_ERR_BAD_STATE, "rollback undoes a single-frame append only (last had %d)",
                undo_.nf);
  if (undo_.to_scale) {
    scale_.pop_back();
  } else {
    live_.pop_back();
  }
  patch_free_.push_front(undo_.page);
  for (auto it = undo_.special.rbegin(); it != undo_.special.rend(); ++it) {
    all_special_.pop_back();
    special_free_.push_front(*it);
  }
  special_tokens_ = undo_.special_tokens;
  frame_count_ = undo_.frame_count;
  undo_ = Undo();
  wm_ = WriteMap();
  ++epoch_;
  return LBM_OK;
}

void Bookkeeping::visible_patch_pages(std::vector<int32_t>* out) const {
  out->assign(scale_.begin(), scale_.end());
  const int32_t n_live = int32_t(live_.size());
  const int32_t take = std::min(n_live, window_);
  for (int32_t i = n_live - take; i < n_live; ++i) out->push_back(live_[i]);
}

PlanInfo Bookkeeping::plan_info() const {
  PlanInfo p;
  p.n_patch_pages = int32_t(scale_.size()) + std::min(int32_t(live_.size()), window_);
  p.patch_tokens = p.n_patch_pages * P_;
  p.n_special_pages = int32_t(all_special_.size());
  p.special_tokens = special_tokens_;
  p.last_page_len = special_tokens_ > 0 ? (special_tokens_ - 1) % sps_ + 1 : 0;
  p.kv_len = p.patch_tokens + special_tokens_;
  return p;
}

lbm_stats Bookkeeping::stats() const {
  lbm_stats s;
  s.frame_count = frame_count_;
  s.scale_pages = int32_t(scale_.size());
  s.live_pages = int32_t(live_.size());
  s.free_pages = int32_t(patch_free_.size());
  s.special_tokens = special_tokens_;
  return s;
}

void Bookkeeping::dump(std::vector<int32_t>* out) const {
  out->clear();
  out->push_back(frame_count_);
  out->push_back(special_tokens_);
  out->push_back(int32_t(scale_.size()));
  out->insert(out->end(), scale_.begin(), scale_.end());
  out->push_back(int32_t(live_.size()));
  out->insert(out->end(), live_.begin(), live_.end());
  out->push_back(int32_t(patch_free_.size()));
  out->insert(out->end(), patch_free_.begin(), patch_free_.end());
  out->push_back(int32_t(all_special_.size()));
  out->insert(out->end(), all_special_.begin(), all_special_.end());
  out->push_back(int32_t(special_free_.size()));
  out->insert(out->end(), special_free_.begin(), special_free_.end());
}

void Bookkeeping::plan_record(std::vector<int32_t>* out) const {
  const PlanInfo p = plan_info();
  std::vector<int32_t> pp;
  visible_patch_pages(&pp);
  out->clear();
  out->push_back(p.kv_len);
  out->push_back(p.n_patch_pages);
  out->push_back(p.n_special_pages);
  out->push_back(p.special_tokens);
  out->push_back(p.last_page_len);
  out->insert(out->end(), pp.begin(), pp.end());
  out->insert(out->end(), all_special_.begin(), all_special_.end());
}

// ---------------------------------------------------------------------------

int32_t choose_splits(int32_t num_q_tokens, int32_t kv_len, int32_t num_heads, int32_t num_cu,
                      int32_t wg_per_cu, int32_t split_cap, int32_t forced, int32_t rows_per_wg,
                      int32_t* groups) {
  if (num_q_tokens < 1 || kv_len < 1 || num_heads < 1 || num_cu < 1 || wg_per_cu < 1 ||
      split_cap < 1 || rows_per_wg < 1)
    return LBM_ERR_INVALID_ARG;
  const int32_t n_tiles = ceil_div(kv_len, kKeysPerTile);
  const int32_t cap = std::min({split_cap, kSplitMax, n_tiles});
  auto normalise = [&](int32_t ns) {
    const int32_t tps = ceil_div(n_tiles, ns);
    return ceil_div(n_tiles, tps);  // no empty split
  };
  const int32_t q_min = ceil_div(num_q_tokens, rows_per_wg);
  const int32_t n_half = ceil_div(num_q_tokens, 32);
  const int32_t q_max = groups ? std::min(q_min + 1, std::max(n_half, q_min)) : q_min;
  if (groups) *groups = q_min;
  if (forced > 0) return normalise(std::min(forced, cap));
  // Cost model, in tile-times of one full workgroup alone on a CU, fitted to
  // the 16-bit kernel (256 query rows per workgroup) on MI355X and applied to
  // either kernel's workgroups (the fp32 kernel's hold 128 rows): k workgroups
  // sharing a CU each take 1 + 0.85 (k - 1) per tile (a second workgroup
  // mostly hides latency; the CU's throughput grows little); every workgroup
  // pays a start/finish cost of about 2 tiles; splitting adds a merge pass (a
  // launch, ~13 tiles, plus ~4 tiles per split of partials).  Equal
  // workgroups are dispatched in rounds of num_cu * wg_per_cu; the last,
  // partial round spreads its workgroups over the CUs.  Choosing groups, a
  // group of g halves takes ceil(g / 4) / ceil(g_full / 4) of a full group's
  // tile time (its busiest SIMD's share; g_full = rows_per_wg / 32).
  constexpr double kShare = 0.85, kFixed = 2.0, kMergeLaunch = 13.0, kMergePerSplit = 4.0;
  const int64_t slots = int64_t(num_cu) * wg_per_cu;
  const int32_t simd_full = std::max(1, ceil_div(rows_per_wg / 32, 4));
  auto per_tile = [&](int64_t k) { return 1.0 + kShare * double(k - 1); };
  int32_t best = 1, best_q = q_min;
  double best_cost = std::numeric_limits<double>::infinity();
  for (int32_t nq = q_min; nq <= q_max; ++nq) {
    const double load =
        groups ? double(ceil_div(ceil_div(n_half, nq), 4)) / double(simd_full) : 1.0;
    const int64_t units = int64_t(nq) * num_heads;
    for (int32_t ns = 1; ns <= cap; ++ns) {
      const int32_t n = normalise(ns);
      if (n != ns) continue;
      const double len = (double(ceil_div(n_tiles, n)) + kFixed) * std::min(1.0, load);
      const int64_t wgs = units * n;
      const int64_t full = wgs / slots, rest = wgs % slots;
      double cost = double(full) * len * per_tile(wg_per_cu);
      if (rest > 0) cost += len * per_tile((rest + num_cu - 1) / num_cu);
      if (n > 1) cost += kMergeLaunch + kMergePerSplit * n;
      if (cost < best_cost - 1e-9) {
        best_cost = cost;
        best = n;
        best_q = nq;
      }
    }
  }
  if (groups) *groups = best_q;
  return best;
}

WorkspaceLayout workspace_layout(const lbm_config& c) {
  WorkspaceLayout w;
  size_t off = 0;
  w.desc_off = off;
  off = align_up(off + sizeof(StepDesc), 256);
  w.patch_ids_off = off;
  off = align_up(off + sizeof(int32_t) * size_t(std::max(1, c.scale_frames + c.sliding_window)), 256);
  w.special_ids_off = off;
  off = align_up(off + sizeof(int32_t) * size_t(std::max(1, c.max_special_pages)), 256);
  // visible keys at most, plus the own rows of a skip-append step
  const int64_t max_kv = int64_t(c.scale_frames + c.sliding_window) * c.patches_per_frame +
                         int64_t(c.max_special_pages) * c.special_page_size + c.max_q_tokens;
  w.rowtab_len = int32_t((max_kv + kKeysPerTile - 1) / kKeysPerTile * kKeysPerTile);
  if (w.rowtab_len < kKeysPerTile) w.rowtab_len = kKeysPerTile;
  w.rowtab_off = off;
  off = align_up(off + sizeof(uint32_t) * size_t(w.rowtab_len), 256);
  const int32_t rows = ceil_div(std::min(c.max_q_tokens, kSplitRowCap), kRowsPerGroup) * kRowsPerGroup;
  w.split_rows = rows;
  w.part_ml_off = off;
  off = align_up(off + sizeof(float) * size_t(kSplitMax) * rows * c.num_heads * 2, 256);
  w.part_o_off = off;
  off = align_up(off + sizeof(float) * size_t(kSplitMax) * rows * c.num_heads * c.head_dim, 256);
  w.total = off;
  return w;
}

int32_t split_capacity(const WorkspaceLayout& w, int32_t num_q_tokens) {
  const int64_t rows_pad = int64_t(ceil_div(num_q_tokens, kRowsPerGroup)) * kRowsPerGroup;
  const int64_t cap = int64_t(kSplitMax) * w.split_rows / rows_pad;
  return int32_t(std::max<int64_t>(1, std::min<int64_t>(cap, kSplitMax)));
}

}  // namespace lbm
