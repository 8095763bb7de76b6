// Merge of key-range splits.
//
// When one (query group, head) is cut into several key ranges, each range
// leaves a partial output O_s with its running max m_s and sum l_s; the
// result is out = sum_s w_s O_s / sum_s w_s l_s with w_s = 2^(m_s - M),
// M = max_s m_s -- the usual combination of online-softmax partials (each
// O_s and l_s is relative to its own m_s; maxima are kept in base-2 exponent
// units, i.e. raw scores times log2(e)/sqrt(D)).  The fp32 kernel stores O_s
// unnormalised in fp32; the 16-bit kernels store O_s / l_s rounded to their
// input type (half the bytes; its range is that of V), which enters here
// weighted by w_s l_s.
// Memory-bound: one thread per 4 output columns of one (row, head), which
// issues the loads of up to eight splits' partials together and then combines
// them (a loop that loaded one split per iteration would wait out one memory
// latency per split).
#include "attn_common.h"

namespace lbm {
namespace {

// PartT: float (unnormalised O_s) or the 16-bit input type (O_s / l_s)
template <typename OutT, typename PartT, int D>
__global__ __launch_bounds__(256) void merge_kernel(const AttnArgs a) {
  constexpr bool kNorm = sizeof(PartT) == 2;
  constexpr int CPR = D / 4;    // float4 chunks per (row, head)
  constexpr int kBatch = 8;     // splits loaded together
  const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t total = int64_t(a.Tq) * a.H * CPR;
  if (idx >= total) return;
  const int32_t chunk = int32_t(idx % CPR);
  const int64_t rh = idx / CPR;  // (row, head) = row * H + head
  const size_t split_stride = size_t(a.rows_pad) * a.H;
  // M: the largest m_s so far; den and acc are relative to it.  A split
  // without keys has m = -inf, l = 0, O = 0 and weighs 0.
  float M = -INFINITY, den = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int32_t s0 = 0; s0 < a.num_splits; s0 += kBatch) {
    float2 ml[kBatch];
    float4 o[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const size_t srh = size_t(s0 + j) * split_stride + size_t(rh);
      if (s0 + j < a.num_splits) {
        ml[j] = *reinterpret_cast<const float2*>(a.part_ml + srh * 2);
        if constexpr (kNorm) {
          typedef PartT p4 __attribute__((ext_vector_type(4)));
          const p4 x = *reinterpret_cast<const p4*>(reinterpret_cast<const PartT*>(a.part_o) +
                                                    srh * D + chunk * 4);
          o[j] = make_float4(float(x[0]), float(x[1]), float(x[2]), float(x[3]));
        } else {
          o[j] = *reinterpret_cast<const float4*>(a.part_o + srh * D + chunk * 4);
        }
      } else {
        ml[j] = make_float2(-INFINITY, 0.f);
        o[j] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    float Mb = M;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) Mb = fmaxf(Mb, ml[j].x);
    if (Mb == -INFINITY) continue;  // no keys in any split so far
    const float r = fast_exp2(M - Mb);  // 0 while M is still -inf
    den *= r;
    acc.x *= r;
    acc.y *= r;
    acc.z *= r;
    acc.w *= r;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const float wl = fast_exp2(ml[j].x - Mb) * ml[j].y;
      const float w = kNorm ? wl : fast_exp2(ml[j].x - Mb);
      den += wl;
      acc.x += w * o[j].x;
      acc.y += w * o[j].y;
      acc.z += w * o[j].z;
      acc.w += w * o[j].w;
    }
    M = Mb;
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
    hipLaunchKernelGGL((merge_kernel<__bf16, __bf16, 64>), grid, block, 0, stream, a);
  else if (dtype == LBM_F16 && head_dim == 64)
    hipLaunchKernelGGL((merge_kernel<_Float16, _Float16, 64>), grid, block, 0, stream, a);
  else if (dtype == LBM_F32 && head_dim == 64)
    hipLaunchKernelGGL((merge_kernel<float, float, 64>), grid, block, 0, stream, a);
  else if (dtype == LBM_F32 && head_dim == 32)
    hipLaunchKernelGGL((merge_kernel<float, float, 32>), grid, block, 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace lbm
