// Merge of key-range splits.
//
// When one (query group, head) is cut into several key ranges, each range
// leaves a partial output O_s with its running max m_s and sum l_s; the
// result is out = sum_s w_s O_s / sum_s w_s l_s with w_s = 2^(m_s - M),
// M = max_s m_s -- the usual combination of online-softmax partials (each
// O_s and l_s is relative to its own m_s; maxima are kept in base-2 exponent
// units, i.e. raw scores times log2(e)/sqrt(D)).  Every kernel stores O_s
// unnormalised in fp32 (a partial rounded to a 16-bit type, then the output
// again, would round a value near V's own twice).
// Memory-bound: one thread per 16 bytes (4 columns) of each partial row of one
// (row, head), which issues the loads of up to eight splits' partials together
// and then combines them (a loop that loaded one split per iteration would wait
// out one memory latency per split), and writes its columns with one store.
#include "attn_common.h"

namespace lbm {
namespace {

template <typename OutT, int D>
__global__ __launch_bounds__(256) void merge_kernel(const AttnArgs a) {
  typedef float PartT;
  constexpr int CW = 16 / sizeof(PartT);  // columns per thread
  constexpr int CPR = D / CW;             // threads per (row, head)
  constexpr int kBatch = 8;               // splits loaded together
  typedef PartT pvec __attribute__((ext_vector_type(CW)));
  typedef OutT ovec __attribute__((ext_vector_type(CW)));
  const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t total = int64_t(a.Tq) * a.H * CPR;
  if (idx >= total) return;
  const int32_t chunk = int32_t(idx % CPR);
  const int64_t rh = idx / CPR;  // (row, head) = row * H + head
  const size_t split_stride = size_t(a.rows_pad) * a.H;
  const PartT* part = reinterpret_cast<const PartT*>(a.part_o);
  // M: the largest m_s so far; den and acc are relative to it.  A split
  // without keys has m = -inf, l = 0, O = 0 and weighs 0.
  float M = -INFINITY, den = 0.f;
  float acc[CW];
#pragma unroll
  for (int c = 0; c < CW; ++c) acc[c] = 0.f;
  for (int32_t s0 = 0; s0 < a.num_splits; s0 += kBatch) {
    float2 ml[kBatch];
    pvec o[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const size_t srh = size_t(s0 + j) * split_stride + size_t(rh);
      if (s0 + j < a.num_splits) {
        ml[j] = *reinterpret_cast<const float2*>(a.part_ml + srh * 2);
        o[j] = *reinterpret_cast<const pvec*>(part + srh * D + chunk * CW);
      } else {
        ml[j] = make_float2(-INFINITY, 0.f);
        o[j] = pvec(PartT(0));
      }
    }
    float Mb = M;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) Mb = fmaxf(Mb, ml[j].x);
    if (Mb == -INFINITY) continue;  // no keys in any split so far
    const float r = fast_exp2(M - Mb);  // 0 while M is still -inf
    den *= r;
#pragma unroll
    for (int c = 0; c < CW; ++c) acc[c] *= r;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const float w = fast_exp2(ml[j].x - Mb);
      den += w * ml[j].y;
#pragma unroll
      for (int c = 0; c < CW; ++c) acc[c] += w * float(o[j][c]);
    }
    M = Mb;
  }
  const float inv = 1.f / den;
  ovec res;
#pragma unroll
  for (int c = 0; c < CW; ++c) res[c] = OutT(acc[c] * inv);
  *reinterpret_cast<ovec*>(reinterpret_cast<OutT*>(a.out) + rh * D + chunk * CW) = res;
}

}  // namespace

hipError_t launch_merge(const AttnArgs& a, int32_t head_dim, int32_t dtype, hipStream_t stream) {
  const int64_t total = int64_t(a.Tq) * a.H * (head_dim / 4);  // 4 columns per thread
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
