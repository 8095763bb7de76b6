// Device helpers shared by the bf16 and fp32 paged-attention kernels.
//
// Keys are addressed in logical-token space: position j of the visible set is
// patch token (j mod P) of visible patch page j / P while j < patch_tokens,
// then special token (j - patch_tokens) of the packed special stream, whose
// final page holds last_page_len valid tokens (table order scale -> live ->
// special: "How FlashInfer's Paged KV Cache Attention Outperforms SDPA
// Fallback in Streaming Inference", FAQ "How does the paged cache handle
// variable sequence lengths across frames?").  Tiles of 64 keys are cut in
// this logical space, so a tile may straddle pages of either stream and the
// result does not depend on where pages sit in the pools.
#pragma once

#include <hip/hip_runtime.h>

#include "kernels.h"

namespace lbm {

constexpr int kThreads = 256;  // 4 wavefronts of 64, 32 query rows each

// Work item of workgroup `blk`: consecutive items go to one XCD (workgroup i
// runs on XCD i mod 8), so the query groups sharing one head's key range run
// side by side on one L2.  Returns -1 for a padding workgroup.
__device__ __forceinline__ int32_t work_item(const AttnArgs& a, int32_t blk) {
  const int32_t item = (blk & 7) * a.items_per_xcd + (blk >> 3);
  return item < a.total_items ? item : -1;
}

// j = q * d + r with 0 <= r < d, for 0 <= j < 2^24 (float estimate, one fix-up).
__device__ __forceinline__ void divmod_small(int32_t j, int32_t d, float inv_d, int32_t& q,
                                             int32_t& r) {
  q = int32_t(float(j) * inv_d);
  r = j - q * d;
  if (r < 0) {
    --q;
    r += d;
  } else if (r >= d) {
    ++q;
    r -= d;
  }
}

// Element pointer of K[j][head][0] (V is `vdelta` elements further), or null
// when j is past the visible set.
template <typename T>
__device__ __forceinline__ const T* key_row(const AttnArgs& a, int32_t head, int32_t j,
                                            int32_t hd, int32_t d, int32_t& vdelta) {
  int32_t pi, slot;
  if (j < a.patch_tokens) {
    divmod_small(j, a.P, a.inv_P, pi, slot);
    const size_t page = size_t(a.patch_ids[pi]);
    vdelta = a.P * hd;
    return reinterpret_cast<const T*>(a.patch_pool) + ((page * 2 * a.P + slot) * hd + head * d);
  }
  if (j < a.kv_len) {
    divmod_small(j - a.patch_tokens, a.SPS, a.inv_SPS, pi, slot);
    const size_t page = size_t(a.special_ids[pi]);
    vdelta = a.SPS * hd;
    return reinterpret_cast<const T*>(a.special_pool) + ((page * 2 * a.SPS + slot) * hd + head * d);
  }
  vdelta = 0;
  return nullptr;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Publish this workgroup's partial result and count arrivals for its
// (query group, head); returns true in the workgroup that arrives last, which
// then owns the merge.  The last one also re-arms the counter for the next
// launch.  Partials may live in another XCD's L2, hence agent-scope fences.
__device__ __forceinline__ bool arrive_last(const AttnArgs& a, int32_t unit) {
  __shared__ int32_t s_last;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  if (threadIdx.x == 0) {
    const int32_t prev =
        __hip_atomic_fetch_add(a.counters + unit, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = prev == a.num_splits - 1;
    if (last) __hip_atomic_store(a.counters + unit, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = last ? 1 : 0;
  }
  __syncthreads();
  const bool last = s_last != 0;
  if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  return last;
}

// Combine the splits' partials of one (query group, head) into the output:
// out = sum_s w_s O_s / sum_s w_s l_s, w_s = 2^((m_s - M) * scale_log2),
// M = max_s m_s.  Thread t merges half of the D columns of row t / 2.
template <typename OutT, int D>
__device__ __forceinline__ void merge_splits(const AttnArgs& a, int32_t qt, int32_t head) {
  constexpr int HALF = D / 2;
  const int32_t r = threadIdx.x >> 1;
  const int32_t c0 = (threadIdx.x & 1) * HALF;
  const int32_t q = qt * 128 + r;
  if (q >= a.Tq) return;
  const size_t split_stride = size_t(a.rows_pad) * a.H;
  const size_t rh = size_t(q) * a.H + head;
  float M = -INFINITY;
  for (int32_t s = 0; s < a.num_splits; ++s) M = fmaxf(M, a.part_ml[(s * split_stride + rh) * 2]);
  float acc[HALF];
#pragma unroll
  for (int i = 0; i < HALF; ++i) acc[i] = 0.f;
  float den = 0.f;
  for (int32_t s = 0; s < a.num_splits; ++s) {
    const float2 ml = *reinterpret_cast<const float2*>(a.part_ml + (s * split_stride + rh) * 2);
    const float w = fast_exp2((ml.x - M) * a.scale_log2);
    den += w * ml.y;
    const float4* po = reinterpret_cast<const float4*>(a.part_o + (s * split_stride + rh) * D + c0);
#pragma unroll
    for (int i = 0; i < HALF / 4; ++i) {
      const float4 o = po[i];
      acc[4 * i + 0] += w * o.x;
      acc[4 * i + 1] += w * o.y;
      acc[4 * i + 2] += w * o.z;
      acc[4 * i + 3] += w * o.w;
    }
  }
  const float inv = 1.f / den;
  OutT* op = reinterpret_cast<OutT*>(a.out) + rh * D + c0;
#pragma unroll
  for (int i = 0; i < HALF; ++i) op[i] = OutT(acc[i] * inv);
}

}  // namespace lbm
