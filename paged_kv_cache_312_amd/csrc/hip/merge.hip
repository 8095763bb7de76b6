// Merge of key-range splits.
//
// When one (query group, head) is cut into several key ranges, each range
// leaves an unnormalised partial output O_s with its running max m_s and sum
// l_s; the result is out = sum_s w_s O_s / sum_s w_s l_s with
// w_s = 2^(m_s - M), M = max_s m_s -- the usual combination of online-softmax
// partials (each O_s and l_s is relative to its own m_s; maxima are kept in
// base-2 exponent units, i.e. raw scores times log2(e)/sqrt(D)).
// Memory-bound: one thread per 4 output columns of one (row, head).
#include "attn_common.h"

namespace lbm {
namespace {

template <typename OutT, int D>
__global__ __launch_bounds__(256) void merge_kernel(const AttnArgs a) {
  constexpr int CPR = D / 4;  // float4 chunks per (row, head)
  const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t total = int64_t(a.Tq) * a.H * CPR;
  if (idx >= total) return;
  const int32_t chunk = int32_t(idx % CPR);
  const int64_t rh = idx / CPR;  // (row, head) = row * H + head
  const size_t split_stride = size_t(a.rows_pad) * a.H;
  float M = -INFINITY;
  for (int32_t s = 0; s < a.num_splits; ++s)
    M = fmaxf(M, a.part_ml[(s * split_stride + rh) * 2]);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float den = 0.f;
  for (int32_t s = 0; s < a.num_splits; ++s) {
    const float2 ml = *reinterpret_cast<const float2*>(a.part_ml + (s * split_stride + rh) * 2);
    const float w = fast_exp2(ml.x - M);
    den += w * ml.y;
    const float4 o = *reinterpret_cast<const float4*>(a.part_o + (s * split_stride + rh) * D + chunk * 4);
    acc.x += w * o.x;
    acc.y += w * o.y;
    acc.z += w * o.z;
    acc.w += w * o.w;
  }
  const float inv = 1.f / den;
  OutT* op = reinterpret_cast<OutT*>(a.out) + rh * D + chunk * 4;
  op[0] = OutT(acc.x * inv);
  op[1] = OutT(acc.y * inv);
  op[2] = OutT(acc.z * inv);
  op[3] = OutT(acc.w * inv);
}

}  // namespace

hipError_t launch_merge(const AttnArgs& a, int32_t head_dim, int32_t dtype, hipStream_t stream) {
  const int64_t total = int64_t(a.Tq) * a.H * (head_dim / 4);
  const dim3 grid(uint32_t((total + 255) / 256)), block(256);
  if (dtype == LBM_BF16 && head_dim == 64)
    hipLaunchKernelGGL((merge_kernel<__bf16, 64>), grid, block, 0, stream, a);
  else if (dtype == LBM_F16 && head_dim == 64)
    hipLaunchKernelGGL((merge_kernel<_Float16, 64>), grid, block, 0, stream, a);
  else if (dtype == LBM_F32 && head_dim == 64)
    hipLaunchKernelGGL((merge_kernel<float, 64>), grid, block, 0, stream, a);
  else if (dtype == LBM_F32 && head_dim == 32)
    hipLaunchKernelGGL((merge_kernel<float, 32>), grid, block, 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace lbm
