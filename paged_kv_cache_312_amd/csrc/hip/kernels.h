// Device-side argument blocks and launchers of the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "../core/bookkeeping.h"

namespace lbm {

// Append scatter: copy a step's K and V token rows into the reserved patch
// page of each frame and the packed special slots.
struct AppendArgs {
  const uint4* k;          // [nf * T rows][rc chunks]
  const uint4* v;
  uint4* patch_pool;       // [pages][2][P][rc]
  uint4* special_pool;     // [pages][2][SPS][rc]
  int32_t T, P, S, SPS;
  int32_t rc;              // 16-byte chunks per token row (H * D * elt / 16)
  int32_t st0;             // special tokens written before this step
  int32_t sp_first;        // index of the page holding token st0 in the special page list
  int32_t patch_pages[kMaxStepFrames];
  int32_t spages[kMaxStepSpecialPages];
  const StepDesc* desc;    // graph-replayed step: st0, sp_first and the pages from here
};

hipError_t launch_append(const AppendArgs& a, int32_t nf, hipStream_t stream);

// Row table of a frame step: for each key position j of the visible set, the
// byte offset of K[j][head 0][0] inside its block's pool, with bit 31 set for
// the special pool.  Positions past kv_len (up to whole 64-key tiles) repeat
// position 0, whose scores the attention kernel masks (row 0 of patch page 0
// when kv_len is 0: every key of the step read from the caller's rows).
struct RowtabArgs {
  const int32_t* patch_ids;   // visible patch pages, in table order
  const int32_t* special_ids; // special pages, in order
  uint32_t* rowtab;
  int32_t P, SPS;
  int32_t patch_tokens;       // n_patch_pages * P
  int32_t kv_len;
  int32_t n_pos;              // n_tiles * 64
  int32_t row_bytes;          // H * D * element size
  float inv_P, inv_SPS;
  const StepDesc* desc;       // graph-replayed step: kv_len, patch_tokens from here (the
                              // grid covers the table's capacity)
  // Plan of lbm_append_run: positions [kv_len, kv_len + own_rows) are the
  // step's own rows (frame-major, own_T = P + own_S tokens a frame), which
  // each block's append writes before its attention reads them; their codes
  // are the rows' destinations in the pools, the last frames' patch pages of
  // the table and the last special tokens of the special stream (padding
  // repeats the first own row when no other key is visible).  0 otherwise.
  int32_t own_rows, own_T, own_S;
  float inv_T;
};

hipError_t launch_rowtab(const RowtabArgs& a, hipStream_t stream);

// Paged attention over a visible table.
struct AttnArgs {
  const void* q;              // [Tq][H][D]
  void* out;                  // [Tq][H][D]
  const void* patch_pool;     // [pages][2][P][H][D]
  const void* special_pool;   // [pages][2][SPS][H][D]
  const uint32_t* rowtab;     // [n_tiles * 64] row codes (see RowtabArgs)
  float* part_o;              // [splits][rows_pad][H][D] partial outputs, unnormalised, fp32
  float* part_ml;             // [splits][rows_pad][H][2] (running max in base-2 units, partial sum)
  int32_t Tq, H;
  int32_t vstride_patch;      // bytes from a K row to its V row: P * H * D * elt
  int32_t vstride_special;    // SPS * H * D * elt
  int32_t kv_len;             // visible keys (the frame's own rows included on a skip-append step)
  // Skip-append step: key positions [tr_start, kv_len) are the frame's own
  // rows, read from tk / tv ([kv_len - tr_start][H][D]) instead of the pools;
  // tr_start = kv_len otherwise.
  const void* tk;
  const void* tv;
  int32_t tr_start;
  int32_t row_bytes;          // H * D * element size
  // Graph-replayed step: kv_len, n_tiles and tiles_per_split come from here
  // (num_splits stays the capture's; splits left without keys write empty
  // partials).
  const StepDesc* desc;
  int32_t n_tiles;            // ceil(kv_len / 64)
  int32_t num_splits, tiles_per_split;
  int32_t n_qt;               // ceil(Tq / rows per workgroup of the kernel)
  int32_t rows_pad;           // ceil(Tq / kRowsPerGroup) * kRowsPerGroup
  int32_t total_items;        // n_qt * H * num_splits
  int32_t items_per_xcd;      // ceil(total_items / 8)
  float scale_log2;           // log2(e) / sqrt(D)
};

// One attention launch over n independent streams (caches), n <= kMaxBatch:
// the work items of stream s are [item_start[s], item_start[s+1]) of the
// launch's item range, each stream's laid out as a single-stream launch's.
constexpr int kMaxBatch = 8;

struct BatchArgs {
  int32_t n;
  int32_t total_items;        // item_start[n]
  int32_t items_per_xcd;      // ceil(total_items / 8)
  int32_t item_start[kMaxBatch + 1];
  AttnArgs s[kMaxBatch];
};

// Query rows per workgroup: the 16-bit kernel (8 wavefronts x 64) and the
// fp32 kernel (4 x 32).
constexpr int32_t kRowsPerWG16 = 2 * kRowsPerGroup;
constexpr int32_t kRowsPerWGf32 = 128;
static_assert(kRowsPerGroup % kRowsPerWGf32 == 0, "partial rows cover both kernels' groups");

// Rows of one split's partial-result block for Tq query rows (the kernels
// index partials by query row; the block is padded to whole row groups).
int32_t partial_rows(int32_t Tq);

// Fill the split/grid fields of `a` for a launch (Tq, kv_len, splits known)
// by a kernel with `rows_per_wg` query rows per workgroup, in `groups` query
// groups (0: the fewest that hold the rows).
void finish_attn_args(AttnArgs* a, int32_t head_dim, int32_t num_splits, int32_t rows_per_wg,
                      int32_t groups = 0);

// 16-bit inputs: bf16, or fp16 when `fp16`; `transient`: a skip-append step
// (tr_start < kv_len)
hipError_t launch_attn16(const BatchArgs& b, int32_t head_dim, bool fp16, bool transient,
                         hipStream_t stream);
hipError_t launch_attn_f32(const BatchArgs& b, int32_t head_dim, bool transient, hipStream_t stream);

// Combine the key-range splits' partials into the output (after an attention
// launch with num_splits > 1, on the same stream).
hipError_t launch_merge(const AttnArgs& a, int32_t head_dim, int32_t dtype, hipStream_t stream);

// Workgroups of the attention kernel resident per CU (for the planner).
int32_t attn_occupancy(int32_t dtype, int32_t head_dim);

}  // namespace lbm
