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

// Destination of chunk c of a fused append (see fused_append_wg).
__device__ __forceinline__ uint4* fused_append_dst(const FusedAppend& f, int64_t c) {
  const int32_t item = int32_t(c / f.rc);  // kv * rows + row
  const int32_t cc = int32_t(c - int64_t(item) * f.rc);
  const int32_t kv = item >= f.rows ? 1 : 0;
  const int32_t row = item - kv * f.rows;
  const int32_t fr = row / f.T;
  const int32_t t = row - fr * f.T;
  if (t < f.P) {
    const size_t page = size_t(f.desc->patch_pages[fr]);
    return f.patch_pool + ((page * 2 + kv) * f.P + t) * size_t(f.rc) + cc;
  }
  const int32_t g = f.desc->st0 + fr * f.S + (t - f.P);  // special token index in the stream
  const int32_t pi = g / f.SPS;
  const int32_t slot = g - pi * f.SPS;
  const size_t page = size_t(f.desc->spages[pi - f.desc->sp_first]);
  return f.special_pool + ((page * 2 + kv) * f.SPS + slot) * size_t(f.rc) + cc;
}

// Source of chunk c: K rows, then V rows.
__device__ __forceinline__ const uint4* fused_append_src(const FusedAppend& f, int64_t c) {
  const int64_t half = int64_t(f.rows) * f.rc;
  return c < half ? f.k + c : f.v + (c - half);
}

// A workgroup of a fused append (see FusedAppend): workgroup w of the wgs
// copies chunks [w * n / wgs, (w + 1) * n / wgs) of the step's n = 2 * rows *
// rc 16-byte chunks (K rows, then V rows, each row rc chunks), four loads in
// flight per lane before their stores.
__device__ __forceinline__ void fused_append_wg(const FusedAppend& f, int32_t w) {
  const int64_t n = int64_t(2) * f.rows * f.rc;
  const int64_t c0 = n * w / f.wgs, c1 = n * (w + 1) / f.wgs;
  const int64_t step = blockDim.x;
  int64_t c = c0 + threadIdx.x;
  for (; c + 3 * step < c1; c += 4 * step) {
    const uint4 x0 = *fused_append_src(f, c);
    const uint4 x1 = *fused_append_src(f, c + step);
    const uint4 x2 = *fused_append_src(f, c + 2 * step);
    const uint4 x3 = *fused_append_src(f, c + 3 * step);
    *fused_append_dst(f, c) = x0;
    *fused_append_dst(f, c + step) = x1;
    *fused_append_dst(f, c + 2 * step) = x2;
    *fused_append_dst(f, c + 3 * step) = x3;
  }
  for (; c < c1; c += step) *fused_append_dst(f, c) = *fused_append_src(f, c);
}

}  // namespace lbm
