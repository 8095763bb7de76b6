// Device part of the per-step plan: the row table.
//
// The plan is built once per frame step and reused by every block's run ("How
// FlashInfer's Paged KV Cache Attention Outperforms SDPA Fallback in Streaming
// Inference", section "Plan-Run Execution Workflow").  The host uploads the
// visible page ids (scale pages, latest window, special pages); this kernel
// expands them into one row code per key position so that the attention
// kernel's inner loop reads one table entry per key instead of dividing by the
// page size and looking the page up.  Position j is patch token j mod P of
// visible patch page j / P while j < patch_tokens, then special token
// (j - patch_tokens) of the packed special stream ("How the Paged KV Cache
// Attention Mechanism Enables Long Sequence Inference in LingBot-Map", section
// "Building the Visible Page Table").
#include "kernels.h"

namespace lbm {

namespace {

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

__device__ __forceinline__ uint32_t row_code(const RowtabArgs& a, int32_t j) {
  int32_t pi, slot;
  if (j < a.patch_tokens) {
    divmod_small(j, a.P, a.inv_P, pi, slot);
    const int64_t row = int64_t(a.patch_ids[pi]) * 2 * a.P + slot;
    return uint32_t(row * a.row_bytes);
  }
  divmod_small(j - a.patch_tokens, a.SPS, a.inv_SPS, pi, slot);
  const int64_t row = int64_t(a.special_ids[pi]) * 2 * a.SPS + slot;
  return uint32_t(row * a.row_bytes) | 0x80000000u;
}

// Destination code of own row r of a fused step: frame r / T, token r mod T,
// a patch token of the frame's page (the table's pages after the visible
// ones) or a special token of the stream after the visible ones.
__device__ __forceinline__ uint32_t own_code(const RowtabArgs& a, int32_t r) {
  int32_t fr, t;
  divmod_small(r, a.own_T, a.inv_T, fr, t);
  if (t < a.P) {
    const int64_t row = int64_t(a.patch_ids[a.patch_tokens / a.P + fr]) * 2 * a.P + t;
    return uint32_t(row * a.row_bytes);
  }
  int32_t pi, slot;
  divmod_small(a.kv_len - a.patch_tokens + fr * a.own_S + (t - a.P), a.SPS, a.inv_SPS, pi, slot);
  const int64_t row = int64_t(a.special_ids[pi]) * 2 * a.SPS + slot;
  return uint32_t(row * a.row_bytes) | 0x80000000u;
}

__global__ void rowtab_kernel(RowtabArgs a) {
  const int32_t j = blockIdx.x * blockDim.x + threadIdx.x;
  if (a.desc) {
    a.kv_len = a.desc->kv_len;
    a.patch_tokens = a.desc->patch_tokens;
    a.n_pos = a.desc->n_tiles * 64;
  }
  if (j >= a.n_pos) return;
  // padding positions repeat a written row: the first visible key, else the
  // first own row (lbm_append_run's plan, written by the block's append
  // before its attention), else row 0 of patch page 0 (a skip-append step,
  // whose kernel reads the padding from the caller's rows)
  uint32_t code;
  if (j < a.kv_len)
    code = row_code(a, j);
  else if (j - a.kv_len < a.own_rows)
    code = own_code(a, j - a.kv_len);
  else
    code = a.kv_len > 0 ? row_code(a, 0) : (a.own_rows > 0 ? own_code(a, 0) : 0u);
  a.rowtab[j] = code;
}

}  // namespace

hipError_t launch_rowtab(const RowtabArgs& a, hipStream_t stream) {
  const int threads = 256;
  const int blocks = (a.n_pos + threads - 1) / threads;
  hipLaunchKernelGGL(rowtab_kernel, dim3(blocks), dim3(threads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace lbm
