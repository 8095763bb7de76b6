// Device helpers shared by the bf16 and fp32 paged-attention kernels.
//
// Keys are addressed in logical-token space: position j of the visible set is
// patch token (j mod P) of visible patch page j / P while j < patch_tokens,
// then special token (j - patch_tokens) of the packed special stream, whose
// final page holds last_page_len valid tokens (table order scale -> live ->
// special: "How FlashInfer's Paged KV Cache Attention Outperforms SDPA
// Fallback in Streaming Inference", FAQ "How does the paged cache handle
// variable sequence lengths across frames?").  The per-step row table maps
// each position to its row; tiles of 64 keys are cut in this logical space,
// so a tile may straddle pages of either stream and the result does not
// depend on where pages sit in the pools.
#pragma once

#include <hip/hip_runtime.h>

#include "kernels.h"

namespace lbm {

constexpr int kThreads = 256;  // 4 wavefronts of 64 lanes

// Work item of workgroup `blk`: consecutive items go to one XCD (workgroup i
// runs on XCD i mod 8), so the query groups sharing one head's key range run
// side by side on one L2.  Returns the item within its stream and sets
// `stream`; stream -1 for a padding workgroup.
__device__ __forceinline__ int32_t work_item(const BatchArgs& b, int32_t blk, int32_t& stream) {
  const int32_t gi = (blk & 7) * b.items_per_xcd + (blk >> 3);
  if (gi >= b.total_items) {
    stream = -1;
    return -1;
  }
  int32_t s = 0;
  while (s + 1 < b.n && gi >= b.item_start[s + 1]) ++s;
  stream = s;
  return gi - b.item_start[s];
}

// K and V row addresses of the key whose row code is `code` (see RowtabArgs);
// `off` adds the head and column byte offset inside the row.
__device__ __forceinline__ void kv_rows(const AttnArgs& a, uint32_t code, int32_t off,
                                        const char*& kp, const char*& vp) {
  const bool special = (code >> 31) != 0;
  const char* base = special ? static_cast<const char*>(a.special_pool)
                             : static_cast<const char*>(a.patch_pool);
  kp = base + (code & 0x7fffffffu) + off;
  vp = kp + (special ? a.vstride_special : a.vstride_patch);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace lbm
