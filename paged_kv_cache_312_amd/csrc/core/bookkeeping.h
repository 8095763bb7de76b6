// Host-side page bookkeeping and planner of the two-stream paged KV cache.
//
// Pure C++17, no HIP: built into liblbm (with the kernels) and, alone, into
// liblbm_core for tests on machines without a GPU.
//
// Page policy.  From the pages: a recyclable patch stream with one page per
// frame and an append-only special stream packed across pages ("How FlashInfer's
// Paged KV Cache Attention Outperforms SDPA Fallback in Streaming Inference",
// section "Two-Stream Design"); eviction pops the oldest live-window page into
// the free list while the window is over-full, scale and special pages are never
// evicted ("How LingBot-Map Uses KV Caching for Efficient Streaming Inference",
// section "Sliding-Window Eviction Strategy"); the visible table is scale pages,
// then the latest window, then the special pages, with the valid-token count of
// the last page ("How the Paged KV Cache Attention Mechanism Enables Long
// Sequence Inference in LingBot-Map", section "Building the Visible Page Table").
// Conventions the pages leave open: free lists start ascending, allocation pops
// the head, eviction pushes to the tail, rollback pushes back to the head; a
// special page is taken when the special-token count is a multiple of the page
// size; evict commits a provisional frame.
#pragma once

#include <cstdint>
#include <deque>
#include <string>
#include <vector>

#include "lbm.h"

namespace lbm {

constexpr int32_t kMaxStepFrames = 128;        // frames one append may bring
constexpr int32_t kMaxStepSpecialPages = 256;  // special pages one append may touch
constexpr int32_t kRowsPerGroup = 256;         // query rows per 16-bit attention workgroup (and
                                               // the padding of partial-result rows)
constexpr int32_t kKeysPerTile = 64;           // keys per attention tile
constexpr int32_t kSplitMax = 16;              // most key-range splits of one run
constexpr int32_t kSplitRowCap = 2048;         // partial-result rows budgeted per split
constexpr int32_t kMaxKvLen = 1 << 24;         // key positions addressable by the kernels

// Thread-local error message; `fail` records it and returns the status.
lbm_status fail(lbm_status st, const char* fmt, ...);
void clear_error();
const char* last_error();

// Checks of a config that every path needs (not whether a kernel exists).
lbm_status validate_config(const lbm_config& c);

// Where one append writes: one patch page per frame, and the special pages
// covering special-token indices [st0, st0 + nf * S).
struct WriteMap {
  int32_t nf = 0;
  int32_t patch_pages[kMaxStepFrames] = {};
  int32_t st0 = 0;       // special tokens written before this append
  int32_t sp_first = 0;  // index, in the special page list, of the page holding token st0
  int32_t n_sp = 0;      // special pages touched
  int32_t spages[kMaxStepSpecialPages] = {};
};

// Visible table summary for one frame step.
struct PlanInfo {
  int32_t kv_len = 0;
  int32_t n_patch_pages = 0;
  int32_t patch_tokens = 0;
  int32_t n_special_pages = 0;
  int32_t special_tokens = 0;
  int32_t last_page_len = 0;
};

class Bookkeeping {
 public:
  explicit Bookkeeping(const lbm_config& cfg);

  lbm_status seed_free_lists(const int32_t* patch_order, int32_t n_patch,
                             const int32_t* special_order, int32_t n_special);
  void reset();

  lbm_status reserve(int32_t nf);  // the block-0 part of append
  lbm_status evict(std::vector<int32_t>* evicted);
  lbm_status rollback();

  const WriteMap& write_map() const { return wm_; }
  bool empty() const { return frame_count_ == 0; }
  uint64_t epoch() const { return epoch_; }

  // Visible patch page ids (scale pages, then the latest sliding_window live
  // pages) and the summary of the whole table.
  void visible_patch_pages(std::vector<int32_t>* out) const;
  const std::vector<int32_t>& special_pages() const { return all_special_; }
  PlanInfo plan_info() const;

  lbm_stats stats() const;
  void dump(std::vector<int32_t>* out) const;         // state record
  void plan_record(std::vector<int32_t>* out) const;  // table record

 private:
  struct Undo {
    bool valid = false;
    int32_t nf = 0;
    int32_t frame_count = 0;
    int32_t special_tokens = 0;
    int32_t page = -1;
    bool to_scale = false;
    std::vector<int32_t> special;  // special pages taken, in order
  };

  int32_t P_, S_, sps_, scale_frames_, window_, max_patch_, max_special_, max_step_;
  std::vector<int32_t> patch_order_, special_order_;
  std::deque<int32_t> patch_free_, special_free_, live_;
  std::vector<int32_t> scale_, all_special_;
  int32_t frame_count_ = 0;
  int32_t special_tokens_ = 0;
  Undo undo_;
  WriteMap wm_;
  uint64_t epoch_ = 1;
};

// Split count for one run: how many key ranges each (query group, head) is
// cut into so that the launch fills the chip (>= 1).  `forced` > 0 asks for
// that many (capped); `split_cap` bounds the choice; `rows_per_wg` is the
// query rows of one workgroup of the kernel that will run.  With `groups`,
// the query groups are chosen too (the fewest that hold the rows, or one
// more), written there: a workgroup's step time is taken to follow its
// busiest SIMD, which holds ceil(halves / 4) of the group's 32-row halves
// (four SIMDs per CU); without it the groups are the fewest.
int32_t choose_splits(int32_t num_q_tokens, int32_t kv_len, int32_t num_heads, int32_t num_cu,
                      int32_t wg_per_cu, int32_t split_cap, int32_t forced,
                      int32_t rows_per_wg = kRowsPerGroup, int32_t* groups = nullptr);

// Workspace layout (byte offsets from the workspace base).
// Per-step values of a frame step that graph-replayed launches read from
// device memory (their own arguments stay those of the capture): the host
// writes it, with the step's page tables, into pinned staging that the graph's
// first node copies to the workspace.
struct StepDesc {
  int32_t kv_len = 0;           // visible keys
  int32_t patch_tokens = 0;     // visible patch pages * P
  int32_t n_tiles = 0;          // ceil(kv_len / 64)
  int32_t tiles_per_split = 0;  // for the graph's split count (later splits may be empty)
  int32_t st0 = 0;              // append: special tokens before the step
  int32_t sp_first = 0;         // append: index of the page holding token st0
  int32_t pad[2] = {};
  int32_t patch_pages[kMaxStepFrames] = {};
  int32_t spages[kMaxStepSpecialPages] = {};
};

struct WorkspaceLayout {
  size_t desc_off = 0;        // StepDesc (graph-replayed steps)
  size_t patch_ids_off = 0;   // int32 [scale_frames + sliding_window]
  size_t special_ids_off = 0; // int32 [max_special_pages]
  size_t rowtab_off = 0;      // uint32 [rowtab_len]: per key position, the pool and row
  size_t part_ml_off = 0;     // float [kSplitMax * split_rows * H * 2]
  size_t part_o_off = 0;      // float [kSplitMax * split_rows * H * D]
  size_t total = 0;
  int32_t rowtab_len = 0;     // longest visible key range, rounded up to whole tiles
  int32_t split_rows = 0;     // partial-result rows per split slot
};
WorkspaceLayout workspace_layout(const lbm_config& c);

// Largest split count the workspace holds for a run of num_q_tokens rows.
int32_t split_capacity(const WorkspaceLayout& w, int32_t num_q_tokens);

size_t dtype_size(int32_t dtype);

}  // namespace lbm
