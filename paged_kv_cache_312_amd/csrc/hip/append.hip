// Append scatter: one frame step's K/V rows into their pages.
//
// On the pages, append splits each new frame into its patch tokens, written to
// a fresh or recycled patch page, and its special tokens, packed after the
// previous ones in the special pages; it runs once per block ("How the Paged
// KV Cache Attention Mechanism Enables Long Sequence Inference in LingBot-Map",
// section "Appending New Frames").  Only new rows move; recycled pages are
// overwritten in place ("... Memory Efficiency Analysis").
//
// One workgroup copies one token row (H*D elements) of K or V with 16-byte
// vector loads and stores; rows of a frame's patch part land in one contiguous
// run of its page, so consecutive workgroups stream contiguous memory.
#include "kernels.h"

namespace lbm {

__global__ void append_scatter_kernel(const AppendArgs a) {
  const int32_t row = blockIdx.x;  // token row of the step, 0 .. nf*T-1
  const int32_t kv = blockIdx.y;   // 0 = K, 1 = V
  const int32_t f = row / a.T;
  const int32_t t = row - f * a.T;
  const uint4* src = (kv ? a.v : a.k) + size_t(row) * a.rc;
  const int32_t* patch_pages = a.desc ? a.desc->patch_pages : a.patch_pages;
  const int32_t* spages = a.desc ? a.desc->spages : a.spages;
  uint4* dst;
  if (t < a.P) {
    const size_t page = size_t(patch_pages[f]);
    dst = a.patch_pool + ((page * 2 + kv) * a.P + t) * size_t(a.rc);
  } else {
    const int32_t st0 = a.desc ? a.desc->st0 : a.st0;
    const int32_t sp_first = a.desc ? a.desc->sp_first : a.sp_first;
    const int32_t g = st0 + f * a.S + (t - a.P);  // special token index in the stream
    const int32_t pi = g / a.SPS;
    const int32_t slot = g - pi * a.SPS;
    const size_t page = size_t(spages[pi - sp_first]);
    dst = a.special_pool + ((page * 2 + kv) * a.SPS + slot) * size_t(a.rc);
  }
  for (int32_t c = threadIdx.x; c < a.rc; c += blockDim.x) dst[c] = src[c];
}

hipError_t launch_append(const AppendArgs& a, int32_t nf, hipStream_t stream) {
  const int32_t rows = nf * a.T;
  int32_t threads = ((a.rc + 63) / 64) * 64;
  if (threads > 256) threads = 256;
  hipLaunchKernelGGL(append_scatter_kernel, dim3(rows, 2), dim3(threads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace lbm
