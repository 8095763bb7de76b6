// Stress driver for the host bookkeeping through its C API (lbm_core.h),
// built with AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_core_sanitizers.py.  It streams seeded random schedules (multi-
// and single-frame appends, evictions, deferred evictions with rollbacks,
// resets, re-seeded free lists) and drives every error path it can reach from
// the host, checking after each step:
//   - the page count is conserved (free + scale + live = max_patch_pages,
//     live <= sliding_window after an eviction, +1 inside a deferred window);
//   - a rollback restores the state record exactly;
//   - a failed call leaves the state record unchanged;
//   - records fit the lengths the calls report.
// Prints "ok" and exits 0 when every check holds; a sanitizer report aborts
// the run with a non-zero status.
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <utility>
#include <vector>

#include "lbm_core.h"

namespace {

int g_failures = 0;
// how often the schedules reached the paths they are meant to reach
int g_rollbacks = 0, g_full_refusals = 0, g_resets = 0, g_seeds = 0, g_evicted = 0;

#define CHECK(cond, ...)                                        \
  do {                                                          \
    if (!(cond)) {                                              \
      std::fprintf(stderr, "check failed at line %d: ", __LINE__); \
      std::fprintf(stderr, __VA_ARGS__);                        \
      std::fprintf(stderr, "\n");                               \
      ++g_failures;                                             \
    }                                                           \
  } while (0)

// splitmix64: a seeded source of schedule decisions
struct Rng {
  uint64_t s;
  uint64_t next() {
    uint64_t z = (s += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  }
  int32_t below(int32_t n) { return int32_t(next() % uint64_t(n)); }
};

std::vector<int32_t> record(lbm_status (*fn)(const lbmcore*, int32_t*, int64_t, int64_t*),
                            const lbmcore* c) {
  int64_t len = 0;
  lbm_status st = fn(c, nullptr, 0, &len);
  CHECK(st == LBM_OK && len >= 0, "record length query failed (%d)", int(st));
  std::vector<int32_t> v(size_t(len) + 4, -7);
  int64_t len2 = 0;
  st = fn(c, v.data(), int64_t(v.size()), &len2);
  CHECK(st == LBM_OK && len2 == len, "record read failed (%d, %lld vs %lld)", int(st),
        (long long)len2, (long long)len);
  for (size_t i = size_t(len); i < v.size(); ++i)
    CHECK(v[i] == -7, "record wrote past its reported length");
  v.resize(size_t(len));
  return v;
}

std::vector<int32_t> dump(const lbmcore* c) { return record(lbmcore_dump, c); }

void check_counts(const lbmcore* c, const lbm_config& cfg, bool deferred) {
  lbm_stats s;
  CHECK(lbmcore_stats(c, &s) == LBM_OK, "stats failed");
  CHECK(s.free_pages + s.scale_pages + s.live_pages == cfg.max_patch_pages,
        "pages not conserved: %d + %d + %d != %d", s.free_pages, s.scale_pages, s.live_pages,
        cfg.max_patch_pages);
  CHECK(s.scale_pages <= cfg.scale_frames, "scale pages %d > %d", s.scale_pages, cfg.scale_frames);
  CHECK(s.live_pages <= cfg.sliding_window + (deferred ? 1 : 0), "live pages %d", s.live_pages);
  CHECK(s.special_tokens == s.frame_count * cfg.special_per_frame, "special tokens %d for %d frames",
        s.special_tokens, s.frame_count);
}

lbm_config make_config(int32_t P, int32_t S, int32_t sps, int32_t scale, int32_t window,
                       int32_t max_frames, int32_t max_step) {
  lbm_config c{};
  c.num_blocks = 2;
  c.num_heads = 2;
  c.head_dim = 64;
  c.patches_per_frame = P;
  c.special_per_frame = S;
  c.special_page_size = sps;
  c.scale_frames = scale;
  c.sliding_window = window;
  c.max_patch_pages = scale + window + max_step;
  c.max_special_pages = (S * max_frames + sps - 1) / sps + 1;
  c.max_frames_per_step = max_step;
  c.max_q_tokens = max_step * (P + S);
  c.dtype = LBM_BF16;
  c.num_splits = 0;
  return c;
}

// A random schedule of `steps` steps over `cfg`.
void stream(const lbm_config& cfg, uint64_t seed, int32_t steps) {
  lbmcore* c = nullptr;
  CHECK(lbmcore_create(&cfg, &c) == LBM_OK && c, "create failed: %s", lbmcore_last_error());
  if (!c) return;
  Rng rng{seed};
  int32_t frames = 0;
  for (int32_t s = 0; s < steps; ++s) {
    if (rng.below(97) == 0) {  // a new video
      CHECK(lbmcore_reset(c) == LBM_OK, "reset failed");
      frames = 0;
      ++g_resets;
    }
    if (rng.below(61) == 0 && frames == 0) {
      ++g_seeds;  // free lists in a permuted order
      std::vector<int32_t> p(size_t(cfg.max_patch_pages)), q(size_t(cfg.max_special_pages));
      for (size_t i = 0; i < p.size(); ++i) p[i] = int32_t(i);
      for (size_t i = 0; i < q.size(); ++i) q[i] = int32_t(i);
      for (size_t i = p.size(); i > 1; --i) std::swap(p[i - 1], p[size_t(rng.below(int32_t(i)))]);
      for (size_t i = q.size(); i > 1; --i) std::swap(q[i - 1], q[size_t(rng.below(int32_t(i)))]);
      CHECK(lbmcore_seed_free_lists(c, p.data(), int32_t(p.size()), q.data(), int32_t(q.size())) ==
                LBM_OK, "seed failed: %s", lbmcore_last_error());
    }
    const int32_t room = cfg.max_special_pages * cfg.special_page_size / std::max(1, cfg.special_per_frame);
    const int32_t nf = frames == 0 ? 1 + rng.below(cfg.max_frames_per_step) : 1;
    if (cfg.special_per_frame > 0 && frames + nf > room - 1) {
      // the special stream is full: the append must fail and change nothing
      const std::vector<int32_t> before = dump(c);
      const lbm_status st = lbmcore_append(c, nf);
      if (st != LBM_OK) {
        CHECK(st == LBM_ERR_OUT_OF_PAGES, "full special pool gave %d", int(st));
        ++g_full_refusals;
        CHECK(dump(c) == before, "failed append changed the state");
        CHECK(lbmcore_reset(c) == LBM_OK, "reset failed");
        frames = 0;
        continue;
      }
      frames += nf;
      int32_t ev[64], n_ev = -1;
      CHECK(lbmcore_evict(c, ev, 64, &n_ev) == LBM_OK, "evict failed");
      continue;
    }
    const bool deferred = nf == 1 && rng.below(3) == 0;
    const std::vector<int32_t> before = dump(c);
    lbm_status st = lbmcore_append(c, nf);
    CHECK(st == LBM_OK, "append %d failed: %s", nf, lbmcore_last_error());
    if (st != LBM_OK) break;
    const std::vector<int32_t> wm = record(lbmcore_write_map, c);
    CHECK(!wm.empty() && wm[0] == nf, "write map names %d frames", wm.empty() ? -1 : wm[0]);
    (void)record(lbmcore_plan, c);
    if (deferred) {
      check_counts(c, cfg, true);
      if (rng.below(10) < 3) {
        CHECK(lbmcore_rollback(c) == LBM_OK, "rollback failed: %s", lbmcore_last_error());
        ++g_rollbacks;
        CHECK(dump(c) == before, "rollback did not restore the state");
        // a second rollback has nothing to undo and must change nothing
        const std::vector<int32_t> after = dump(c);
        CHECK(lbmcore_rollback(c) != LBM_OK, "second rollback accepted");
        CHECK(dump(c) == after, "refused rollback changed the state");
        check_counts(c, cfg, false);
        continue;
      }
    }
    frames += nf;
    // an undersized eviction buffer: the count is reported in full
    int32_t ev[1] = {-1};
    int32_t n_ev = -1;
    st = lbmcore_evict(c, ev, rng.below(2), &n_ev);
    CHECK(st == LBM_OK && n_ev >= 0, "evict failed: %s", lbmcore_last_error());
    g_evicted += n_ev;
    // evict is idempotent; rollback after evict is refused and changes nothing
    int32_t n2 = -1;
    CHECK(lbmcore_evict(c, nullptr, 0, &n2) == LBM_OK && n2 == 0, "second evict freed %d", n2);
    if (nf == 1) {
      const std::vector<int32_t> after = dump(c);
      CHECK(lbmcore_rollback(c) == LBM_ERR_BAD_STATE, "rollback after evict accepted");
      CHECK(dump(c) == after, "refused rollback changed the state");
    }
    check_counts(c, cfg, false);
    (void)record(lbmcore_plan, c);
  }
  lbmcore_destroy(c);
}

void error_paths() {
  lbm_config cfg = make_config(16, 6, 16, 2, 4, 40, 3);
  lbmcore* c = nullptr;
  CHECK(lbmcore_create(nullptr, &c) == LBM_ERR_INVALID_ARG, "null config accepted");
  CHECK(lbmcore_create(&cfg, nullptr) == LBM_ERR_INVALID_ARG, "null out accepted");
  lbm_config bad = cfg;
  bad.max_patch_pages = 0;
  CHECK(lbmcore_create(&bad, &c) != LBM_OK, "zero patch pages accepted");
  bad = cfg;
  bad.special_page_size = 0;
  CHECK(lbmcore_create(&bad, &c) != LBM_OK, "zero special page size accepted");
  bad = cfg;
  bad.max_frames_per_step = 0;
  CHECK(lbmcore_create(&bad, &c) != LBM_OK, "zero frames per step accepted");
  bad = cfg;
  bad.patches_per_frame = 1 << 30;  // one block's pool past 2 GiB
  CHECK(lbmcore_create(&bad, &c) != LBM_OK, "oversized pool accepted");

  CHECK(lbmcore_create(&cfg, &c) == LBM_OK, "create failed");
  if (!c) return;
  const std::vector<int32_t> empty = dump(c);
  CHECK(lbmcore_append(c, 0) == LBM_ERR_INVALID_ARG, "zero frames accepted");
  CHECK(lbmcore_append(c, cfg.max_frames_per_step + 1) == LBM_ERR_INVALID_ARG, "too many frames");
  CHECK(lbmcore_rollback(c) != LBM_OK, "rollback of an empty cache accepted");
  CHECK(dump(c) == empty, "failed calls changed an empty cache");
  int64_t len = -1;
  CHECK(lbmcore_dump(c, nullptr, 4, &len) == LBM_ERR_INVALID_ARG, "null buffer with capacity");
  CHECK(lbmcore_dump(c, nullptr, 0, nullptr) == LBM_ERR_INVALID_ARG, "null length accepted");
  CHECK(lbmcore_stats(c, nullptr) == LBM_ERR_INVALID_ARG, "null stats accepted");
  std::vector<int32_t> dup(size_t(cfg.max_patch_pages), 0);
  CHECK(lbmcore_seed_free_lists(c, dup.data(), int32_t(dup.size()), nullptr, 0) != LBM_OK,
        "duplicate page ids accepted");
  // multi-frame step, then a rollback (single-frame only) is refused
  CHECK(lbmcore_append(c, 3) == LBM_OK, "append failed");
  const std::vector<int32_t> three = dump(c);
  CHECK(lbmcore_rollback(c) == LBM_ERR_BAD_STATE, "rollback of a 3-frame step accepted");
  CHECK(dump(c) == three, "refused rollback changed the state");
  // exhaust the patch pages without evicting: the append that finds the list
  // empty fails and changes nothing
  lbm_status st = LBM_OK;
  for (int i = 0; i < cfg.max_patch_pages + 2 && st == LBM_OK; ++i) {
    const std::vector<int32_t> before = dump(c);
    st = lbmcore_append(c, 1);
    if (st != LBM_OK) {
      CHECK(st == LBM_ERR_OUT_OF_PAGES, "empty free list gave %d", int(st));
      CHECK(dump(c) == before, "failed append changed the state");
    }
  }
  CHECK(st == LBM_ERR_OUT_OF_PAGES, "patch pages never ran out");
  lbmcore_destroy(c);
  lbmcore_destroy(nullptr);

  // the planner's split choice over edge arguments
  CHECK(lbmcore_choose_splits(0, 100, 16, 256, 2, 16, 0, 0) < 0, "zero queries accepted");
  CHECK(lbmcore_choose_splits(100, 0, 16, 256, 2, 16, 0, 0) < 0, "zero keys accepted");
  CHECK(lbmcore_choose_splits(1, 1, 1, 1, 1, 1, 0, 0) == 1, "one key, one split");
  for (int32_t kv = 1; kv < 200000; kv = kv * 3 + 7)
    for (int32_t q = 1; q < 20000; q = q * 5 + 3) {
      const int32_t n = lbmcore_choose_splits(q, kv, 16, 256, 2, 16, 0, (q & 1) ? 128 : 0);
      const int32_t tiles = (kv + 63) / 64;
      CHECK(n >= 1 && n <= 16 && n <= tiles, "splits %d for q %d kv %d", n, q, kv);
      const int32_t f = lbmcore_choose_splits(q, kv, 16, 256, 2, 16, 1000, 0);
      CHECK(f >= 1 && f <= 16 && f <= tiles, "forced splits %d for kv %d", f, kv);
    }
}

}  // namespace

int main() {
  error_paths();
  // the tiny workload's shape, a ViT-L-shaped frame, and degenerate settings
  const lbm_config cfgs[] = {
      make_config(16, 6, 16, 2, 4, 400, 3),
      make_config(1369, 6, 16, 8, 64, 3000, 8),
      make_config(37, 3, 8, 0, 3, 400, 4),   // no scale frames
      make_config(100, 0, 16, 2, 3, 400, 3), // no special tokens
      make_config(100, 6, 16, 2, 0, 400, 3), // no window
  };
  uint64_t seed = 1;
  for (const lbm_config& cfg : cfgs)
    for (int rep = 0; rep < 3; ++rep) stream(cfg, seed++, 1500);
  if (g_failures) {
    std::printf("%d checks failed\n", g_failures);
    return 1;
  }
  std::printf("ok: %d rollbacks, %d full-pool refusals, %d resets, %d seeded orders, %d evictions\n",
              g_rollbacks, g_full_refusals, g_resets, g_seeds, g_evicted);
  return 0;
}
